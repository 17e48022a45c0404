"""tg_bias_attn_bwd on the GPU vs the fp64 oracle backward (TokenGate pages:
ai.info summary "Key Contributions" items 2 and 3 -- the gradients that train
the gate through the attention bias).

The forward runs on the GPU (tg_bias_attn_fwd, giving out and lse), the
backward takes them; the oracle recomputes everything in fp64 from the same
exact bf16 inputs.

Tolerance, per output tensor: max |gpu - ref| <= rel * max |ref| + floor,
rel = 2e-2 for dq, dk, dv and dscore, 5e-2 for dgain, and the absolute floor
2^-16 max |dV_ref| (dV = P^T dO carries the scale of dO without
cancellation).  The floor covers outputs that are exactly 0 by cancellation,
such as every gradient of a lone visible key: there dP_rc and Delta_r are
the same D-term fp32 sum formed in two orders, and dZ is their rounding
difference, a few 2^-24 D-term rounding steps at the scale of dO V.  The GPU path rounds P
and dZ to bf16 as MFMA operands (a relative 2^-9 step each, errors that
average out over the sums), stores dq/dk/dv as bf16 (another 2^-9), and forms
Delta_r = <dO_r, O_r> from the forward's bf16 output O.  That last rounding
moves Delta_r by up to 2^-9 sum_d |dO O|, and every dZ[r, c] by P[r, c] times
that; dgain_h = sum_{r,c} c_r s_c dZ is a sum with cancellation (each row's
dZ sums to 0), so this error is not averaged away: up to about
2^-9 sqrt(D) (2.2% at D = 128) of its magnitude on short prompts, hence the
wider bound.  Observed errors are reported per test (dgain <= 1.7%)."""
import numpy as np
import pytest
import torch

import learned_token_pruning_gate_amd as tg
import oracle
import workloads
from gpu_util import as_f64, report, to_dev

pytestmark = pytest.mark.gpu

BWD_REL = {"dq": 2e-2, "dk": 2e-2, "dv": 2e-2, "dscore": 2e-2, "dgain": 5e-2}


def make(rng, N, Hq, Hkv, D, bias=True, qscale=True):
    draw = lambda shape: workloads.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    q, k, v, do = draw((N, Hq, D)), draw((N, Hkv, D)), draw((N, Hkv, D)), draw((N, Hq, D))
    s = rng.standard_normal(N).astype(np.float32) if bias else None
    g = rng.uniform(0.5, 2.0, size=Hq).astype(np.float32)
    c = rng.uniform(1.0, 2.0, size=N).astype(np.float32) if qscale else None
    return q, k, v, do, s, g, c


def gpu_bwd(q, k, v, do, s, g, c, causal=True, repeat=1):
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    sd = None if s is None else to_dev(s)
    gd = to_dev(g)
    cd = None if c is None else to_dev(c)
    out, lse = tg.tg_bias_attn_fwd(qd, kd, vd, sd, gd, cd, causal=causal)
    res = [tg.tg_bias_attn_bwd(qd, kd, vd, sd, gd, out, dod, lse, q_scale=cd, causal=causal)
           for _ in range(repeat)]
    torch.cuda.synchronize()
    return res if repeat > 1 else res[0]


def ref_bwd(q, k, v, do, s, g, c, causal=True):
    f = lambda x: workloads.as_f64(x, "bf16")
    ss = np.zeros(q.shape[0]) if s is None else s
    return oracle.bias_attn_bwd(f(q), f(k), f(v), ss, g, f(do), q_scale=c, causal=causal)


def check(got, ref, tag, bias=True):
    names = ("dq", "dk", "dv", "dscore", "dgain")
    worst = {}
    floor = 2.0 ** -16 * (float(np.max(np.abs(ref[2]))) if ref[2].size else 0.0)
    for name, a, b in zip(names, got, ref):
        if a is None:
            assert not bias and name in ("dscore", "dgain")
            continue
        a = as_f64(a)
        scale = float(np.max(np.abs(b))) if b.size else 0.0
        err = float(np.max(np.abs(a - b))) if b.size else 0.0
        worst[name] = err / max(scale, 1e-30)
        assert err <= BWD_REL[name] * scale + floor, (tag, name, err, scale, floor)
    report(tag, **{"rel_err_" + k: v for k, v in worst.items()})


SHAPES = [  # N, Hq, Hkv, D, causal, bias, qscale
    (1, 2, 1, 128, True, True, True),
    (17, 4, 2, 64, True, True, True),
    (100, 8, 8, 128, True, True, False),
    (255, 16, 8, 128, True, True, True),
    (300, 16, 2, 128, True, False, True),     # 8 heads per KV head, no bias
    (129, 6, 2, 64, True, True, True),        # 3 heads per KV head
    (612, 16, 8, 128, False, True, True),     # non-causal
    (1000, 4, 4, 64, True, True, True),       # ragged query and key blocks
    (260, 8, 4, 128, False, False, False),
    # head dim 256: two launches per gradient kernel, one per 128-dim half
    (1, 2, 1, 256, True, True, True),
    (77, 4, 2, 256, True, True, True),        # one ragged key block
    (300, 8, 4, 256, True, True, True),
    (1000, 4, 2, 256, True, True, True),      # dK/dV split over query chunks
    (260, 8, 8, 256, False, True, False),     # non-causal, 1 head per KV head
    (513, 16, 2, 256, True, False, True),     # 8 heads per KV head, no bias
    (129, 6, 2, 256, True, True, True),       # 3 heads per KV head
]


@pytest.mark.parametrize("N,Hq,Hkv,D,causal,bias,qscale", SHAPES)
def test_attn_bwd_shapes(N, Hq, Hkv, D, causal, bias, qscale):
    rng = np.random.default_rng(N * 7 + Hq + D + causal)
    q, k, v, do, s, g, c = make(rng, N, Hq, Hkv, D, bias, qscale)
    got = gpu_bwd(q, k, v, do, s, g, c, causal)
    ref = ref_bwd(q, k, v, do, s, g, c, causal)
    check(got, ref, "attn_bwd_N%d_H%d_%d_D%d_c%d_b%d" % (N, Hq, Hkv, D, causal, bias), bias)


@pytest.mark.parametrize("D", [128, 256])
def test_attn_bwd_masked_key_and_rows(D):
    """A -inf score deletes its key (zero dk, dv, dscore for it); rows that
    see only deleted keys get zero dq."""
    rng = np.random.default_rng(41)
    N = 300
    q, k, v, do, s, g, c = make(rng, N, 8, 4, D)
    s[0] = -np.inf     # row 0 sees only key 0
    s[77] = -np.inf
    dq, dk, dv, ds, dg = gpu_bwd(q, k, v, do, s, g, c)
    for t in (dk[0], dk[77], dv[0], dv[77], dq[0]):
        assert torch.all(t.float() == 0)
    assert float(ds[0]) == 0.0 and float(ds[77]) == 0.0
    assert torch.all(torch.isfinite(dg))
    ref = ref_bwd(q, k, v, do, s, g, c)
    check((dq, dk, dv, ds, dg), ref, "attn_bwd_masked_D%d" % D)


@pytest.mark.parametrize("D", [128, 256])
def test_attn_bwd_small_q_scale_deletes_keys(D):
    """At per-query scales far below 1 (0.1 and 0.01) a -inf score still
    deletes its key: rows that see only deleted keys get zero gradients,
    deleted keys get zero dk, dv and dscore, and the rest matches the oracle
    run on the keys that remain."""
    rng = np.random.default_rng(94 + D)
    N = 400
    q, k, v, do, s, g, _ = make(rng, N, 8, 4, D)
    c = np.where(np.arange(N) % 2 == 0, 0.1, 0.01).astype(np.float32)
    s[:50] = -np.inf                      # rows 0..49 see only deleted keys
    s[rng.choice(np.arange(50, N), 20, replace=False)] = -np.inf
    dq, dk, dv, ds, dg = gpu_bwd(q, k, v, do, s, g, c)
    dead = np.isneginf(s)
    for t in (dk, dv):
        assert torch.all(t[torch.from_numpy(dead)].float() == 0)
    assert torch.all(dq[:50].float() == 0)
    assert torch.all(ds.cpu()[torch.from_numpy(dead)] == 0)
    ref = ref_bwd(q, k, v, do, s, g, c)
    check((dq, dk, dv, ds, dg), ref, "attn_bwd_small_qscale_D%d" % D)


@pytest.mark.parametrize("D", [128, 256])
def test_attn_bwd_invariants_and_determinism(D):
    """sum_c dscore_c = 0 (a row's softmax ignores a shared shift of its
    scores) and two calls agree bit for bit."""
    rng = np.random.default_rng(42)
    q, k, v, do, s, g, c = make(rng, 700, 16, 8, D)
    (dq1, dk1, dv1, ds1, dg1), (dq2, dk2, dv2, ds2, dg2) = gpu_bwd(q, k, v, do, s, g, c,
                                                                  repeat=2)
    for a, b in ((dq1, dq2), (dk1, dk2), (dv1, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(ds1, ds2) and torch.equal(dg1, dg2)
    tot = float(ds1.double().sum())
    assert abs(tot) <= 1e-3 * float(ds1.double().abs().sum()), tot


@pytest.mark.parametrize("name", ["t16k", "t16k-d256"])
def test_attn_bwd_t16k_full(name):
    """The 16k prompt's kept set (N = 2512; 16/8 heads at D = 128, 8/2 heads
    at D = 256): every gradient element against the oracle."""
    w = workloads.get(name)
    _, a = workloads.generate(w)
    rng = np.random.default_rng(93)
    s = rng.standard_normal(w.n_kept).astype(np.float32)
    do = workloads.to_bf16_bits(rng.standard_normal(a.q.shape).astype(np.float32))
    got = gpu_bwd(a.q, a.k, a.v, do, s, a.gain, None)
    ref = ref_bwd(a.q, a.k, a.v, do, s, a.gain, None)
    check(got, ref, "attn_bwd_full_" + name)
