"""Oracle checks of one pass of the whole path (gate -> top-K -> gather ->
bias attention), shared by the eager chain tests and the graph-replay tests.

Tolerances and rules (TokenGate pages: ai.info summary "Key Contributions"
items 1-3):
* gate scores: fp32 |diff| <= 1e-5 max(1, |ref|); bf16 max |diff| <= 2e-2;
* kept set: equal to the oracle's selection on the GPU's own fp32 scores,
  bit for bit; where every token's oracle score is computed, it may differ
  from the selection on the oracle's fp64 scores only at tokens whose score
  lies within twice the score tolerance of the threshold;
* gather: bit-exact rows, positions and scores;
* attention: as the gate, on O and on the log-sum-exp, over every row when
  N <= 2600 and otherwise over the first and last row of every 128-query
  block plus a random sample.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads
from gpu_util import BF16_ABS, F32_REL, assert_close_abs, assert_close_f32, report


def attn_rows(N, seed):
    """None (every row) for short kept sets; else the first and last row of
    every 128-query block, the tail and a random sample."""
    if N <= 2600:
        return None
    rng = np.random.default_rng(seed)
    starts = np.arange(0, N, 128)
    return np.unique(np.concatenate([starts, np.minimum(starts + 127, N - 1),
                                     np.arange(N - 32, N), rng.choice(N, 48, replace=False)]))


def check_chain(w, resid, prunable, gate, attn, r, tag, planted=None, q=None):
    """Checks the outputs `r` of one pass against the oracle.

    resid, q    host arrays the pass read (bf16 bits or f32); q defaults to
                the workload's drawn Q
    gate, attn  the workload's GateInputs / AttnInputs (weights, K, V, gain)
    r           dict: scores [T] f32, n_kept int, kept [N] int32,
                resid_kept [N, d] host array (bf16 bits or f32), pos [N],
                score_kept [N] f32, key_score [N] f32 (what the attention
                used), q_scale [N] or None, out [N, Hq, D] fp64, lse [Hq, N]
    """
    N = w.n_kept
    q = attn.q if q is None else q

    # gate: every row for the smaller workloads, sampled rows beyond
    full_gate = w.T <= 16384
    if full_gate:
        rows = np.arange(w.T)
    else:
        rng = np.random.default_rng(w.seed + 1)
        rows = np.unique(np.concatenate([np.arange(512), np.arange(w.T - 512, w.T),
                                         rng.choice(w.T, 2000, replace=False)]))
    ref_s = oracle.gate_score(workloads.as_f64(resid[rows], w.dtype), prunable[rows],
                              workloads.as_f64(gate.w1, w.dtype), gate.w2, b2=gate.b2,
                              gamma=gate.gamma, b1=gate.b1, eps=gate.eps)
    got_s = r["scores"].astype(np.float64)
    if planted is not None:
        p0, vals = planted
        ref_s = ref_s.copy()
        sel = (rows >= p0) & (rows < p0 + 64)
        ref_s[sel] = vals[rows[sel] - p0]
    if w.dtype == "f32":
        assert_close_f32(got_s[rows], ref_s, tag + "_gate")
    else:
        assert_close_abs(got_s[rows], ref_s, BF16_ABS, tag + "_gate")

    # select: exact on the GPU's own scores
    ref_kept = oracle.topk_select(r["scores"], prunable, w.K)
    assert r["n_kept"] == N == len(ref_kept), (tag, r["n_kept"], N, len(ref_kept))
    assert np.array_equal(r["kept"], ref_kept), tag + ": kept set"
    if full_gate:   # against the oracle's own scores: differences only near the threshold
        ref_kept2 = oracle.topk_select(ref_s.astype(np.float32), prunable, w.K)
        diff = np.setxor1d(ref_kept, ref_kept2)
        if diff.size:
            tol = F32_REL if w.dtype == "f32" else BF16_ABS
            pr = np.nonzero(prunable)[0]
            thr = np.sort(ref_s[pr])[::-1][min(w.K, len(pr)) - 1]
            assert np.all(np.abs(ref_s[diff] - thr) <= 2 * tol), \
                tag + ": selection differs far from the threshold"
        report(tag + "_select", N=N, differs_from_fp64_selection=int(diff.size))
    if planted is not None:
        p0, _ = planted
        assert set(range(p0, p0 + 64)) <= set(r["kept"].tolist()), tag + ": planted block"

    # gather: bit-exact
    g_rows, g_pos, g_sk = oracle.compact_gather(resid, r["scores"], ref_kept)
    assert r["resid_kept"].tobytes() == g_rows.tobytes(), tag + ": gathered rows"
    assert np.array_equal(r["pos"], g_pos), tag + ": positions"
    assert r["score_kept"].tobytes() == g_sk.tobytes(), tag + ": gathered scores"

    # attention on the key scores the pass used, all rows or a sample
    arows = attn_rows(N, w.seed + 2)
    ro, rl = oracle.bias_attn(workloads.as_f64(q, w.dtype), workloads.as_f64(attn.k, w.dtype),
                              workloads.as_f64(attn.v, w.dtype), r["key_score"], attn.gain,
                              q_scale=r["q_scale"], rows=arows)
    go, gl = r["out"], r["lse"]
    if arows is not None:
        go, gl = go[arows], gl[:, arows]
    if w.dtype == "f32":
        assert_close_f32(go, ro, tag + "_attn")
        assert_close_f32(gl, rl, tag + "_lse")
    else:
        assert_close_abs(go, ro, BF16_ABS, tag + "_attn")
        assert_close_abs(gl, rl, BF16_ABS, tag + "_lse")
