"""Seeded synthetic inputs for the token-gated prefill path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no step of the method itself: only random draws, the fp32 -> bf16
rounding of inputs (round to nearest even), the workload table, and the
recipes that build test inputs (a planted high-score block, a per-query
scale array).

Workload table (names are what the workload is, with its sizes):

==========  =====  ======  ====  ===  ==============  =====  =======  ===
name        dtype  T       d     h    prunable        K      Hq/Hkv   D
==========  =====  ======  ====  ===  ==============  =====  =======  ===
tiny        f32    512     256   64   32..479         64     4/2      64
tiny-K32    f32    512     256   64   32..479         32     4/2      64
t16k        bf16   16384   2048  256  256..16127      2000   16/8     128
t32k-K100   bf16   32768   2048  256  256..32511      100    16/8     128
t32k-K500   bf16   32768   2048  256  256..32511      500    16/8     128
t32k-K2000  bf16   32768   2048  256  256..32511      2000   16/8     128
t32k-scale  bf16   32768   2048  256  256..32511      2000   16/8     128
t128k       bf16   131072  2048  256  256..130815     2000   16/8     128
t32k-dense  bf16   32768   2048  256  256..32511      32256  16/8     128
t16k-d256   bf16   16384   2048  256  256..16127      2000   8/2      256
==========  =====  ======  ====  ===  ==============  =====  =======  ===

The shapes are those of Qwen3-1.7B (hidden 2048, 16 query / 8 KV heads,
head dim 128), the model the TokenGate pages evaluate (t16k-d256 keeps
the 16k prompt and takes the pages' other supported head dim, 256, with
8 query / 2 KV heads, a shape chosen here); the lengths mirror
their 16k training length and 32k-128k evaluation tiers; the non-prunable
prefix and suffix mirror the instruction / question text around the
prunable document; the budgets mirror the README's K sweep.

Draw order per workload, from ``numpy.random.default_rng(seed)``:
residual N(0,1) [T, d]; W1 N(0, 1/d) [h, d]; w2 N(0, 1/h) [h]; then, over the
N kept tokens, Q N(0,1) [N, Hq, D], K N(0,1) [N, Hkv, D], V N(0,1)
[N, Hkv, D]; gain U(0.5, 2) [Hq].  b1 = 0, b2 = 0, gamma = 1, eps = 1e-6.
The dense workload then draws its key scores N(0,1) [N].  The planted block
position comes from ``default_rng([seed, 1])``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np


# ---------------------------------------------------------------------------
# bf16 bit handling (numpy has no bf16 type; bf16 arrays are uint16 bits)
# ---------------------------------------------------------------------------
def to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even; NaN -> quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # no uint32 overflow: the largest non-NaN pattern is 0xFF800000 (-inf)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
         >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def as_f64(a, dtype: str) -> np.ndarray:
    """Exact fp64 values of an input array stored as f32 or bf16 bits."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Workload table
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str            # "f32" or "bf16"
    T: int
    d: int
    h: int
    p_lo: int             # prunable tokens are p_lo .. p_hi-1
    p_hi: int
    K: int
    Hq: int
    Hkv: int
    D: int
    eps: float = 1e-6
    planted_block: bool = False
    q_scale_recipe: str = "none"   # "none" | "pos_rank"
    drawn_key_scores: bool = False  # key scores N(0,1) instead of gate scores
    tags: tuple = field(default_factory=tuple)

    @property
    def n_prunable(self) -> int:
        return self.p_hi - self.p_lo

    @property
    def n_nonprunable(self) -> int:
        return self.T - self.n_prunable

    @property
    def n_kept(self) -> int:
        """min(K, |P|) + |not P| (every non-prunable token is kept)."""
        return min(self.K, self.n_prunable) + self.n_nonprunable


_BASE = {
    "tiny": Workload("tiny", 1, "f32", 512, 256, 64, 32, 480, 64, 4, 2, 64),
    "t16k": Workload("t16k", 2, "bf16", 16384, 2048, 256, 256, 16128, 2000,
                     16, 8, 128),
    "t32k-K2000": Workload("t32k-K2000", 3, "bf16", 32768, 2048, 256, 256,
                           32512, 2000, 16, 8, 128, planted_block=True),
    "t128k": Workload("t128k", 4, "bf16", 131072, 2048, 256, 256, 130816,
                      2000, 16, 8, 128),
    "t32k-dense": Workload("t32k-dense", 5, "bf16", 32768, 2048, 256, 256,
                           32512, 32256, 16, 8, 128,
                           q_scale_recipe="pos_rank", drawn_key_scores=True),
}

WORKLOADS = dict(_BASE)
WORKLOADS["tiny-K32"] = replace(_BASE["tiny"], name="tiny-K32", K=32)
WORKLOADS["t32k-K100"] = replace(_BASE["t32k-K2000"], name="t32k-K100", K=100)
WORKLOADS["t32k-K500"] = replace(_BASE["t32k-K2000"], name="t32k-K500", K=500)
WORKLOADS["t32k-scale"] = replace(_BASE["t32k-K2000"], name="t32k-scale",
                                  q_scale_recipe="pos_rank")
WORKLOADS["t16k-d256"] = replace(_BASE["t16k"], name="t16k-d256", seed=6, Hq=8, Hkv=2, D=256)


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ---------------------------------------------------------------------------
# Generators
# ---------------------------------------------------------------------------
def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16_bits(x) if dtype == "bf16" else x


@dataclass
class GateInputs:
    resid: np.ndarray      # [T, d] f32 or bf16 bits
    prunable: np.ndarray   # [T] uint8
    w1: np.ndarray         # [h, d] f32 or bf16 bits
    b1: np.ndarray         # [h] f32
    w2: np.ndarray         # [h] f32
    b2: float
    gamma: np.ndarray      # [d] f32
    eps: float


@dataclass
class AttnInputs:
    q: np.ndarray          # [N, Hq, D]
    k: np.ndarray          # [N, Hkv, D]
    v: np.ndarray          # [N, Hkv, D]
    gain: np.ndarray       # [Hq] f32
    drawn_scores: np.ndarray | None  # [N] f32 (dense workload only)


def prunable_mask(w: Workload) -> np.ndarray:
    m = np.zeros(w.T, dtype=np.uint8)
    m[w.p_lo:w.p_hi] = 1
    return m


def generate(w: Workload):
    """(GateInputs, AttnInputs) for a workload, in the documented draw order."""
    rng = np.random.default_rng(w.seed)
    resid = _normal(rng, (w.T, w.d), 1.0, w.dtype)
    w1 = _normal(rng, (w.h, w.d), 1.0 / math.sqrt(w.d), w.dtype)
    w2 = rng.standard_normal(size=w.h, dtype=np.float32) * np.float32(1.0 / math.sqrt(w.h))
    gate = GateInputs(resid=resid, prunable=prunable_mask(w), w1=w1,
                      b1=np.zeros(w.h, np.float32), w2=w2.astype(np.float32),
                      b2=0.0, gamma=np.ones(w.d, np.float32), eps=w.eps)
    N = w.n_kept
    q = _normal(rng, (N, w.Hq, w.D), 1.0, w.dtype)
    k = _normal(rng, (N, w.Hkv, w.D), 1.0, w.dtype)
    v = _normal(rng, (N, w.Hkv, w.D), 1.0, w.dtype)
    gain = rng.uniform(0.5, 2.0, size=w.Hq).astype(np.float32)
    drawn = None
    if w.drawn_key_scores:
        drawn = rng.standard_normal(size=N, dtype=np.float32)
    return gate, AttnInputs(q=q, k=k, v=v, gain=gain, drawn_scores=drawn)


def score_bound(gate: GateInputs, dtype: str) -> float:
    """An upper bound on |score| of any token for these gate weights:
    |b2| + sum_j |w2_j| (|b1_j| + sqrt(d) * ||W1_j * gamma||_2), because a
    normalised row has 2-norm at most sqrt(d) and |SiLU(z)| <= |z|."""
    w1 = as_f64(gate.w1, dtype) * gate.gamma.astype(np.float64)[None, :]
    d = w1.shape[1]
    rown = np.sqrt((w1 * w1).sum(axis=1))
    return float(abs(gate.b2) + np.sum(np.abs(gate.w2.astype(np.float64)) *
                                       (np.abs(gate.b1.astype(np.float64)) +
                                        math.sqrt(d) * rown)))


def planted_block(w: Workload, gate: GateInputs):
    """(p0, values): a block of 64 tokens at a seeded position p0 inside the
    prunable span whose scores B+1+j (j = 0..63) exceed every real score."""
    rng = np.random.default_rng([w.seed, 1])
    p0 = int(rng.integers(w.p_lo, w.p_hi - 64 + 1))
    B = math.ceil(score_bound(gate, w.dtype))
    vals = (B + 1 + np.arange(64)).astype(np.float32)
    return p0, vals


def apply_planted_block(scores: np.ndarray, w: Workload, gate: GateInputs):
    p0, vals = planted_block(w, gate)
    out = np.array(scores, dtype=np.float32, copy=True)
    out[p0:p0 + 64] = vals
    return out


def q_scale_pos_rank(kept_idx) -> np.ndarray:
    """Per-query scale clip(ln(1 + (pos+1)/(rank+1)), 1, 2): pos is the kept
    token's original position, rank its index among the kept tokens."""
    pos = np.asarray(kept_idx, dtype=np.float64)
    rank = np.arange(pos.shape[0], dtype=np.float64)
    return np.clip(np.log1p((pos + 1.0) / (rank + 1.0)), 1.0, 2.0).astype(np.float32)
