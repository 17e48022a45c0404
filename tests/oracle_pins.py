"""Pins that tie the oracle to facts outside itself (CPU only).

Every ``pin_*`` function takes an ``oracle.Oracle`` and raises
AssertionError when the oracle disagrees with:

* values the TokenGate pages print (``tests/golden/``),
* PyTorch fp64 library routines (rms_norm, linear, silu,
  scaled_dot_product_attention) and numpy's stable lexsort,
* closed forms and exhaustive brute force on tiny inputs,
* invariants the method implies (zero bias is plain causal attention, a -inf
  score deletes a key, a key-constant bias is a softmax no-op, K = |P| keeps
  everything, kept = min(K, |P|) + |not P|).

``test_oracle_pins.py`` runs them against the real oracle and
``test_oracle_mutants.py`` runs them against copies of the oracle with a
planted mistake, each of which must fail at least one pin.

Passages (TokenGate pages): the gate is the ai.info summary "Key
Contributions" item 1 and the README mirror "How it works"; the selection
rule is "Key Contributions" item 1 and "Methodology in Plain English";
token-gated attention is "Key Contributions" items 2-3 and "Methodology in
Plain English".
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(got, ref, rtol, atol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    ok = np.isclose(got, ref, rtol=rtol, atol=atol, equal_nan=True)
    assert ok.all(), "%s: max |diff| %g" % (
        what, float(np.nanmax(np.abs(got - ref)[~ok])))


# ===========================================================================
# Gate
# ===========================================================================
def torch_gate(x, prunable, w1, b1, w2, b2, gamma, eps):
    """fp64 PyTorch library routines: rms_norm, linear, silu."""
    xt = torch.from_numpy(np.asarray(x, np.float64))
    wt = None if gamma is None else torch.from_numpy(np.asarray(gamma, np.float64))
    u = F.rms_norm(xt, (xt.shape[1],), weight=wt, eps=eps)
    bt = None if b1 is None else torch.from_numpy(np.asarray(b1, np.float64))
    z = F.linear(u, torch.from_numpy(np.asarray(w1, np.float64)), bt)
    a = F.silu(z)
    s = F.linear(a, torch.from_numpy(np.asarray(w2, np.float64))[None, :],
                 torch.tensor([float(b2)], dtype=torch.float64))[:, 0]
    s = s.numpy().copy()
    s[np.asarray(prunable) == 0] = 0.0
    return s


def pin_gate_torch_random(orc):
    for T, d, h, seed in [(7, 16, 4, 0), (33, 64, 16, 1), (64, 40, 24, 2)]:
        rng = np.random.default_rng(seed)
        x = rng.standard_normal((T, d)) * rng.uniform(0.1, 5.0, size=(T, 1))
        prunable = (rng.random(T) < 0.7).astype(np.uint8)
        w1 = rng.standard_normal((h, d)) / math.sqrt(d)
        b1 = rng.standard_normal(h) * 0.3
        w2 = rng.standard_normal(h) / math.sqrt(h)
        gamma = rng.uniform(0.5, 1.5, size=d)
        got = orc.gate_score(x, prunable, w1, w2, b2=0.25, gamma=gamma, b1=b1,
                             eps=1e-6)
        ref = torch_gate(x, prunable, w1, b1, w2, 0.25, gamma, 1e-6)
        _close(got, ref, 1e-12, 1e-12, "gate vs torch")
        assert np.all(got[prunable == 0] == 0.0)


def pin_gate_torch_tiny_workload(orc):
    w = workloads.get("tiny")
    g, _ = workloads.generate(w)
    x = workloads.as_f64(g.resid, w.dtype)
    w1 = workloads.as_f64(g.w1, w.dtype)
    got = orc.gate_score(x, g.prunable, w1, g.w2, b2=g.b2, gamma=g.gamma,
                         b1=g.b1, eps=g.eps)
    ref = torch_gate(x, g.prunable, w1, g.b1, g.w2, g.b2, g.gamma, g.eps)
    _close(got, ref, 1e-12, 1e-13, "gate tiny workload")
    assert np.count_nonzero(got) == w.n_prunable


def pin_gate_constant_row(orc):
    """x = kappa*1 normalises to u_i = gamma_i*kappa/sqrt(kappa^2 + eps)."""
    d, kappa, eps = 8, 1e-3, 1e-6      # eps matters at this kappa
    gamma = np.arange(1, d + 1, dtype=np.float64) / 4.0
    w1 = np.zeros((2, d))
    w1[0, 2] = 1.0
    w1[1, 5] = -2.0
    b1 = np.array([0.5, 0.0])
    w2 = np.array([1.5, -0.75])
    ucoef = kappa / math.sqrt(kappa * kappa + eps)
    silu = lambda z: z / (1.0 + math.exp(-z))
    expect = -0.125 + 1.5 * silu(gamma[2] * ucoef + 0.5) - 0.75 * silu(-2.0 * gamma[5] * ucoef)
    got = orc.gate_score(np.full((1, d), kappa), np.ones(1, np.uint8), w1, w2,
                         b2=-0.125, gamma=gamma, b1=b1, eps=eps)
    assert abs(got[0] - expect) <= 1e-14 * max(1.0, abs(expect)), (got[0], expect)


def pin_gate_by_hand(orc):
    """x = (3, 4): mean square 12.5; W1 = [1, -1] gives z = -1/sqrt(12.5)."""
    z = (3.0 - 4.0) / math.sqrt(12.5)
    expect = z / (1.0 + math.exp(-z))
    got = orc.gate_score(np.array([[3.0, 4.0]]), np.ones(1, np.uint8),
                         np.array([[1.0, -1.0]]), np.array([1.0]), eps=0.0)
    assert abs(got[0] - expect) <= 1e-15, (got[0], expect)
    # SiLU(1) = 1/(1 + e^-1) = 0.7310585786300049
    got1 = orc.gate_score(np.array([[1.0, 1.0]]), np.ones(1, np.uint8),
                          np.array([[0.5, 0.5]]), np.array([1.0]), eps=0.0)
    assert abs(got1[0] - 0.7310585786300049) <= 1e-15, got1[0]


def pin_gate_zero_weights(orc):
    rng = np.random.default_rng(5)
    T, d, h = 9, 12, 5
    b1 = rng.standard_normal(h)
    w2 = rng.standard_normal(h)
    got = orc.gate_score(rng.standard_normal((T, d)), np.ones(T, np.uint8),
                         np.zeros((h, d)), w2, b2=0.75, b1=b1)
    expect = 0.75 + sum(w2[j] * b1[j] / (1.0 + math.exp(-b1[j])) for j in range(h))
    _close(got, np.full(T, expect), 1e-14, 0, "zero weights")


def pin_gate_scale_invariance(orc):
    """RMSNorm divides out a positive row scale (exactly when eps = 0)."""
    rng = np.random.default_rng(9)
    T, d, h = 11, 32, 8
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((h, d))
    w2 = rng.standard_normal(h)
    p = np.ones(T, np.uint8)
    s1 = orc.gate_score(x, p, w1, w2, eps=0.0)
    s2 = orc.gate_score(x * 37.5, p, w1, w2, eps=0.0)
    _close(s1, s2, 1e-12, 1e-14, "scale invariance")


def pin_gate_nonprunable(orc):
    rng = np.random.default_rng(3)
    T, d, h = 10, 16, 4
    x = rng.standard_normal((T, d))
    p = np.array([1, 0, 1, 0, 0, 1, 1, 1, 0, 1], np.uint8)
    w1 = rng.standard_normal((h, d))
    w2 = rng.standard_normal(h)
    s = orc.gate_score(x, p, w1, w2, b2=3.0)
    assert np.all(s[p == 0] == 0.0)
    assert np.all(s[p == 1] != 0.0)
    x2 = x.copy()
    x2[p == 0] = 1e30
    assert np.array_equal(s, orc.gate_score(x2, p, w1, w2, b2=3.0))


# ===========================================================================
# Selection and compaction
# ===========================================================================
def _dominates(s, t, u):
    """Token t must be kept before token u: higher score, or equal score
    and lower index; NaN is below every number; -0 == +0."""
    st, su = s[t], s[u]
    if math.isnan(st) or math.isnan(su):
        if math.isnan(st) and math.isnan(su):
            return t < u
        return math.isnan(su)
    return st > su or (st == su and t < u)


def brute_force_select(scores, prunable, K):
    """Enumerate every K-subset of the prunable tokens and return the one in
    which each kept token dominates each dropped token (it is unique)."""
    s = [float(x) for x in np.asarray(scores, np.float32)]
    P = [t for t in range(len(s)) if prunable[t]]
    k = min(K, len(P))
    found = []
    for sub in itertools.combinations(P, k):
        kept = set(sub)
        dropped = [u for u in P if u not in kept]
        if all(_dominates(s, t, u) for t in kept for u in dropped):
            found.append(kept)
    assert len(found) == 1, "selection must be unique, found %d" % len(found)
    keep = found[0] | {t for t in range(len(s)) if not prunable[t]}
    return np.array(sorted(keep), dtype=np.int32)


def lexsort_select(scores, prunable, K):
    """numpy's stable lexsort on (is NaN, -score, index)."""
    s = np.asarray(scores, np.float32).astype(np.float64)
    P = np.nonzero(np.asarray(prunable))[0]
    sp = s[P]
    isn = np.isnan(sp)
    neg = np.where(isn, 0.0, -sp)
    order = np.lexsort((P, neg, isn))
    chosen = P[order[:min(K, len(P))]]
    keep = np.union1d(chosen, np.nonzero(np.asarray(prunable) == 0)[0])
    return keep.astype(np.int32)


def pin_select_brute_force(orc):
    rng = np.random.default_rng(11)
    specials = np.array([np.nan, -0.0, 0.0, np.inf, -np.inf], np.float32)
    for trial in range(60):
        T = int(rng.integers(1, 11))
        prunable = (rng.random(T) < 0.75).astype(np.uint8)
        # few distinct values so ties are common, plus IEEE special values
        s = rng.integers(-2, 3, size=T).astype(np.float32)
        sel = rng.random(T) < 0.3
        s[sel] = rng.choice(specials, size=int(sel.sum()))
        nP = int(prunable.sum())
        for K in sorted({0, 1, nP // 2, max(nP - 1, 0), nP, nP + 3}):
            got = orc.topk_select(s, prunable, K)
            ref = brute_force_select(s, prunable, K)
            assert np.array_equal(got, ref), (trial, s, prunable, K, got, ref)


def pin_select_lexsort(orc):
    rng = np.random.default_rng(12)
    for T, K in [(100, 7), (1000, 100), (4097, 1000), (5000, 0), (3000, 2999)]:
        prunable = (rng.random(T) < 0.9).astype(np.uint8)
        s = rng.standard_normal(T).astype(np.float32)
        # quantise part of the scores to create ties
        s[: T // 3] = np.round(s[: T // 3] * 4) / 4
        got = orc.topk_select(s, prunable, K)
        ref = lexsort_select(s, prunable, K)
        assert np.array_equal(got, ref), (T, K)


def pin_select_kept_count_identity(orc):
    """kept = min(K, |P|) + |not P|, instantiated by the README example."""
    with open(os.path.join(GOLDEN, "readme_kept_count.json")) as f:
        g = json.load(f)
    T, K, n_kept = g["T"], g["K"], g["n_kept"]
    nNP = n_kept - K
    rng = np.random.default_rng(13)
    prunable = np.ones(T, np.uint8)
    prunable[rng.choice(T, size=nNP, replace=False)] = 0
    s = rng.standard_normal(T).astype(np.float32)
    assert len(orc.topk_select(s, prunable, K)) == n_kept
    for b in g["budgets"]:
        k = T if b is None else b          # None keeps every state token
        want = T if b is None else b + nNP
        assert len(orc.topk_select(s, prunable, k)) == want


def pin_select_invariants(orc):
    rng = np.random.default_rng(14)
    T = 2000
    prunable = np.zeros(T, np.uint8)
    prunable[100:1900] = 1
    s = rng.standard_normal(T).astype(np.float32)
    nP, nNP = 1800, 200
    for K in [0, 1, 64, 1799, 1800, 5000]:
        kept = orc.topk_select(s, prunable, K)
        assert len(kept) == min(K, nP) + nNP
        assert np.all(np.diff(kept) > 0)               # strictly increasing
        assert set(np.nonzero(prunable == 0)[0]) <= set(kept.tolist())
    assert np.array_equal(orc.topk_select(s, prunable, nP), np.arange(T))
    assert np.array_equal(orc.topk_select(s, prunable, 0),
                          np.nonzero(prunable == 0)[0])
    try:
        orc.topk_select(s, prunable, -1)
    except ValueError:
        pass
    else:
        raise AssertionError("K < 0 must be rejected")


def pin_select_tie_block(orc):
    """64 equal scores with the cut inside the block: lowest indices win."""
    T = 300
    prunable = np.ones(T, np.uint8)
    s = np.full(T, -5.0, np.float32)
    s[40:50] = 9.0                    # 10 clear winners
    s[100:164] = 3.0                  # tie block
    kept = orc.topk_select(s, prunable, 10 + 20)
    expect = np.concatenate([np.arange(40, 50), np.arange(100, 120)])
    assert np.array_equal(kept, expect), kept


def pin_select_planted_block(orc):
    """A block whose scores exceed every real score is kept for every K >= 64."""
    w = workloads.get("tiny")
    g, _ = workloads.generate(w)
    B = workloads.score_bound(g, w.dtype)
    x = workloads.as_f64(g.resid, w.dtype)
    s = orc.gate_score(x, g.prunable, workloads.as_f64(g.w1, w.dtype), g.w2,
                       b2=g.b2, gamma=g.gamma, b1=g.b1, eps=g.eps)
    assert np.max(np.abs(s)) <= B
    s = workloads.apply_planted_block(s.astype(np.float32), w, g)
    p0, _ = workloads.planted_block(w, g)
    for K in [64, 65, 100, w.n_prunable]:
        kept = set(orc.topk_select(s, g.prunable, K).tolist())
        assert set(range(p0, p0 + 64)) <= kept, K
    kept = orc.topk_select(s, g.prunable, 32)
    assert set(range(p0 + 32, p0 + 64)) <= set(kept.tolist())


# ===========================================================================
# Gather
# ===========================================================================
def pin_gather_fancy_indexing(orc):
    rng = np.random.default_rng(15)
    for dtype in (np.uint16, np.float32):
        T, d = 257, 24
        resid = rng.integers(0, 65535, size=(T, d)).astype(dtype) if dtype == np.uint16 \
            else rng.standard_normal((T, d)).astype(np.float32)
        scores = rng.standard_normal(T).astype(np.float32)
        idx = np.sort(rng.choice(T, size=77, replace=False)).astype(np.int32)
        rk, pos, sk = orc.compact_gather(resid, scores, idx)
        assert rk.tobytes() == resid[idx].tobytes()
        assert np.array_equal(pos, idx)
        assert sk.tobytes() == scores[idx].tobytes()
    rk, pos, sk = orc.compact_gather(resid, scores, np.zeros(0, np.int32))
    assert rk.shape == (0, d) and pos.shape == (0,) and sk.shape == (0,)


def pin_kv_gather_take(orc):
    """numpy.take along the token axis (a library routine), bit for bit."""
    rng = np.random.default_rng(16)
    for L, T, N in [(1, 9, 4), (3, 131, 40), (2, 64, 64)]:
        cache = rng.integers(0, 65535, size=(L, T, 2, 8)).astype(np.uint16)
        idx = np.sort(rng.choice(T, size=N, replace=False)).astype(np.int32)
        got = orc.kv_gather(cache, idx)
        assert got.shape == (L, N, 2, 8)
        assert got.tobytes() == np.take(cache, idx, axis=1).tobytes()
    assert orc.kv_gather(cache, np.zeros(0, np.int32)).shape == (2, 0, 2, 8)


# ===========================================================================
# Token-gated attention
# ===========================================================================
def torch_bias_attn(q, k, v, key_score, gain, q_scale, scale, causal):
    """fp64 scaled_dot_product_attention with a float mask:
    z = c_r (scale q.k + gain_h s_c) is SDPA on Q' = c_r Q with additive
    mask c_r gain_h s_c (and -inf above the diagonal); K/V repeated per
    query head group."""
    q = torch.from_numpy(np.asarray(q, np.float64))
    k = torch.from_numpy(np.asarray(k, np.float64))
    v = torch.from_numpy(np.asarray(v, np.float64))
    N, Hq, D = q.shape
    G = Hq // k.shape[1]
    c = torch.ones(N, dtype=torch.float64) if q_scale is None else \
        torch.from_numpy(np.asarray(q_scale, np.float64))
    s = torch.from_numpy(np.asarray(key_score, np.float64))
    g = torch.from_numpy(np.asarray(gain, np.float64))
    qh = (q * c[:, None, None]).permute(1, 0, 2)               # [Hq, N, D]
    kh = k.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
    vh = v.repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
    mask = c[None, :, None] * g[:, None, None] * s[None, None, :]  # [Hq, N, N]
    if causal:
        upper = torch.triu(torch.ones(N, N, dtype=torch.bool), diagonal=1)
        mask = mask.masked_fill(upper[None], float("-inf"))
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


def _attn_case(rng, N, Hq, Hkv, D, with_scale=True):
    q = rng.standard_normal((N, Hq, D))
    k = rng.standard_normal((N, Hkv, D))
    v = rng.standard_normal((N, Hkv, D))
    s = rng.standard_normal(N)
    g = rng.uniform(0.5, 2.0, size=Hq)
    c = rng.uniform(1.0, 2.0, size=N) if with_scale else None
    return q, k, v, s, g, c


def pin_attn_torch_sdpa(orc):
    rng = np.random.default_rng(21)
    for N, Hq, Hkv, D, causal, scaled in [(1, 2, 1, 8, True, True),
                                          (17, 4, 2, 16, True, True),
                                          (64, 4, 4, 32, True, False),
                                          (96, 6, 2, 64, True, True),
                                          (33, 4, 2, 16, False, True)]:
        q, k, v, s, g, c = _attn_case(rng, N, Hq, Hkv, D, scaled)
        scale = 1.0 / math.sqrt(D)
        got, _ = orc.bias_attn(q, k, v, s, g, q_scale=c, causal=causal)
        ref = torch_bias_attn(q, k, v, s, g, c, scale, causal)
        _close(got, ref, 1e-11, 1e-12, "attn vs sdpa N=%d" % N)


def pin_attn_brute_force(orc):
    """Explicit softmax with math.exp loops on tiny inputs, LSE included."""
    rng = np.random.default_rng(22)
    N, Hq, Hkv, D = 5, 4, 2, 3
    q, k, v, s, g, c = _attn_case(rng, N, Hq, Hkv, D)
    scale = 0.7
    got, lse = orc.bias_attn(q, k, v, s, g, q_scale=c, scale=scale)
    G = Hq // Hkv
    for r in range(N):
        for h in range(Hq):
            kv = h // G
            zs = [c[r] * (scale * sum(q[r, h, e] * k[j, kv, e] for e in range(D))
                          + g[h] * s[j]) for j in range(r + 1)]
            ws = [math.exp(z) for z in zs]
            tot = sum(ws)
            for e in range(D):
                o = sum(ws[j] * v[j, kv, e] for j in range(r + 1)) / tot
                assert abs(got[r, h, e] - o) <= 1e-12 * max(1.0, abs(o))
            assert abs(lse[h, r] - math.log(tot)) <= 1e-12 * max(1.0, abs(math.log(tot)))


def pin_attn_zero_bias_is_causal_attention(orc):
    rng = np.random.default_rng(23)
    N, Hq, Hkv, D = 40, 4, 2, 16
    q, k, v, _, g, _ = _attn_case(rng, N, Hq, Hkv, D)
    got, _ = orc.bias_attn(q, k, v, np.zeros(N), g)
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).repeat_interleave(G, 1).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(v).repeat_interleave(G, 1).permute(1, 0, 2).contiguous()
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(1, 0, 2).numpy()
    _close(got, ref, 1e-11, 1e-12, "zero bias")


def pin_attn_neg_inf_deletes_key(orc):
    rng = np.random.default_rng(24)
    N, Hq, Hkv, D = 30, 4, 2, 8
    q, k, v, s, g, c = _attn_case(rng, N, Hq, Hkv, D)
    for cdel in [0, 7, 29]:
        s2 = s.copy()
        s2[cdel] = -np.inf
        got, lse = orc.bias_attn(q, k, v, s2, g, q_scale=c)
        keep = np.array([i for i in range(N) if i != cdel])
        red, red_lse = orc.bias_attn(q[keep], k[keep], v[keep], s[keep], g,
                                     q_scale=c[keep])
        _close(got[keep], red, 1e-12, 1e-13, "-inf deletes key %d" % cdel)
        _close(lse[:, keep], red_lse, 1e-12, 1e-13, "-inf lse")
    # row 0 with its only key deleted is fully masked: O = 0, LSE = -inf
    s3 = s.copy()
    s3[0] = -np.inf
    got, lse = orc.bias_attn(q, k, v, s3, g)
    assert np.all(got[0] == 0.0) and np.all(np.isneginf(lse[:, 0]))


def pin_attn_key_constant_bias(orc):
    rng = np.random.default_rng(25)
    N, Hq, Hkv, D = 24, 4, 2, 8
    q, k, v, s, g, c = _attn_case(rng, N, Hq, Hkv, D)
    beta = 3.25
    o1, l1 = orc.bias_attn(q, k, v, s, g, q_scale=c)
    o2, l2 = orc.bias_attn(q, k, v, s + beta, g, q_scale=c)
    _close(o1, o2, 1e-12, 1e-13, "key-constant bias")
    _close(l2, l1 + c[None, :] * g[:, None] * beta, 1e-12, 1e-12, "lse shift")


def pin_attn_closed_forms(orc):
    rng = np.random.default_rng(26)
    N, Hq, Hkv, D = 20, 4, 2, 8
    q, k, v, s, g, c = _attn_case(rng, N, Hq, Hkv, D)
    G = Hq // Hkv
    # row 0 sees only itself
    got, _ = orc.bias_attn(q, k, v, s, g, q_scale=c)
    for h in range(Hq):
        assert np.array_equal(got[0, h], v[0, h // G])
    # Q = 0 and zero bias: causal running mean of V
    got, _ = orc.bias_attn(np.zeros_like(q), k, v, np.zeros(N), g)
    for h in range(Hq):
        mean = np.cumsum(v[:, h // G], axis=0) / np.arange(1, N + 1)[:, None]
        _close(got[:, h], mean, 1e-13, 1e-14, "running mean")
    # Q = 0: weights are softmax_c(c_r g_h s_c) over c <= r
    got, _ = orc.bias_attn(np.zeros_like(q), k, v, s, g, q_scale=c)
    for r in [1, 9, 19]:
        for h in range(Hq):
            w = np.exp(c[r] * g[h] * s[: r + 1])
            ref = (w[:, None] * v[: r + 1, h // G]).sum(0) / w.sum()
            _close(got[r, h], ref, 1e-12, 1e-13, "Q=0")


def pin_attn_rows_subset(orc):
    """Computing a subset of query rows gives the same rows as computing all."""
    rng = np.random.default_rng(27)
    N, Hq, Hkv, D = 50, 4, 2, 16
    q, k, v, s, g, c = _attn_case(rng, N, Hq, Hkv, D)
    full, lf = orc.bias_attn(q, k, v, s, g, q_scale=c)
    rows = np.array([49, 0, 13, 13, 31])
    sub, ls = orc.bias_attn(q, k, v, s, g, q_scale=c, rows=rows)
    assert np.array_equal(sub, full[rows]) and np.array_equal(ls, lf[:, rows])


# ---------------------------------------------------------------------------
# attention backward
# ---------------------------------------------------------------------------
def torch_bias_attn_grads(q, k, v, key_score, gain, q_scale, scale, causal, dout):
    """fp64 torch autograd through an explicit masked softmax: gradients of
    sum(O * dout) for q, k, v, key_score, gain."""
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    q, k, v, s, g = t(q), t(k), t(v), t(key_score), t(gain)
    N, Hq, D = q.shape
    G = Hq // k.shape[1]
    c = torch.ones(N, dtype=torch.float64) if q_scale is None else \
        torch.from_numpy(np.asarray(q_scale, np.float64))
    kh = k.repeat_interleave(G, dim=1)                          # [N, Hq, D]
    vh = v.repeat_interleave(G, dim=1)
    dots = torch.einsum("rhe,che->hrc", q, kh)                  # [Hq, N, N]
    z = c[None, :, None] * (scale * dots + g[:, None, None] * s[None, None, :])
    if causal:
        upper = torch.triu(torch.ones(N, N, dtype=torch.bool), diagonal=1)
        z = z.masked_fill(upper[None], float("-inf"))
    p = torch.softmax(z, dim=-1)
    o = torch.einsum("hrc,che->rhe", p, vh)
    (o * torch.from_numpy(np.asarray(dout, np.float64))).sum().backward()
    return [x.grad.numpy() for x in (q, k, v, s, g)]


def pin_attn_bwd_torch_autograd(orc):
    rng = np.random.default_rng(31)
    for N, Hq, Hkv, D, causal, scaled in [(1, 2, 1, 4, True, True),
                                          (23, 4, 2, 8, True, True),
                                          (19, 4, 4, 16, True, False),
                                          (21, 6, 2, 8, False, True)]:
        q, k, v, s, g, c = _attn_case(rng, N, Hq, Hkv, D, scaled)
        do = rng.standard_normal((N, Hq, D))
        scale = 1.0 / math.sqrt(D)
        got = orc.bias_attn_bwd(q, k, v, s, g, do, q_scale=c, causal=causal)
        ref = torch_bias_attn_grads(q, k, v, s, g, c, scale, causal, do)
        for name, a, b in zip(("dq", "dk", "dv", "dscore", "dgain"), got, ref):
            _close(a, b, 1e-10, 1e-12, "attn bwd %s N=%d causal=%d" % (name, N, causal))


def pin_attn_bwd_finite_differences(orc):
    """Central differences of sum(O * dO) through the oracle's forward."""
    rng = np.random.default_rng(32)
    N, Hq, Hkv, D = 6, 4, 2, 3
    q, k, v, s, g, c = _attn_case(rng, N, Hq, Hkv, D)
    do = rng.standard_normal((N, Hq, D))
    scale = 0.6
    dq, dk, dv, ds, dg = orc.bias_attn_bwd(q, k, v, s, g, do, q_scale=c, scale=scale)

    def loss(q_, k_, v_, s_, g_):
        o, _ = orc.bias_attn(q_, k_, v_, s_, g_, q_scale=c, scale=scale)
        return float(np.sum(o * do))

    eps = 1e-6
    base = [q, k, v, s, g]
    grads = [dq, dk, dv, ds, dg]
    picks = [(0, (3, 1, 0)), (0, (5, 2, 2)), (1, (1, 0, 2)), (1, (4, 1, 1)), (2, (2, 1, 0)),
             (2, (0, 0, 1)), (3, (2,)), (3, (5,)), (4, (0,)), (4, (3,))]
    for which, idx in picks:
        plus = [x.copy() for x in base]
        minus = [x.copy() for x in base]
        plus[which][idx] += eps
        minus[which][idx] -= eps
        fd = (loss(*plus) - loss(*minus)) / (2 * eps)
        an = grads[which][idx]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, idx, fd, an)


def pin_attn_bwd_invariants(orc):
    rng = np.random.default_rng(33)
    N, Hq, Hkv, D = 30, 4, 2, 8
    q, k, v, s, g, c = _attn_case(rng, N, Hq, Hkv, D)
    do = rng.standard_normal((N, Hq, D))
    dq, dk, dv, ds, dg = orc.bias_attn_bwd(q, k, v, s, g, do, q_scale=c)
    # adding a constant to every score of a row leaves the softmax unchanged
    assert abs(ds.sum()) <= 1e-10 * np.abs(ds).sum()
    # a key-constant score: dgain_h = kappa * sum of each row's dZ = 0
    _, _, _, _, dg0 = orc.bias_attn_bwd(q, k, v, np.full(N, 1.7), g, do, q_scale=c)
    assert np.all(np.abs(dg0) <= 1e-10 * (1.0 + np.abs(dg).max()))
    # no upstream gradient, no gradient
    for a in orc.bias_attn_bwd(q, k, v, s, g, np.zeros_like(do), q_scale=c):
        assert np.all(a == 0.0)
    # a -inf score deletes its key: zero gradients for it; with row 7's own
    # upstream gradient zeroed too, the rest equals the problem without token 7
    s2 = s.copy()
    s2[7] = -np.inf
    do2 = do.copy()
    do2[7] = 0.0
    dq2, dk2, dv2, ds2, dg2 = orc.bias_attn_bwd(q, k, v, s2, g, do2, q_scale=c)
    assert np.all(dk2[7] == 0) and np.all(dv2[7] == 0) and ds2[7] == 0 and np.all(np.isfinite(dg2))
    keep = np.array([i for i in range(N) if i != 7])
    r = orc.bias_attn_bwd(q[keep], k[keep], v[keep], s[keep], g, do[keep], q_scale=c[keep])
    _close(dq2[keep], r[0], 1e-12, 1e-12, "bwd delete dq")
    _close(dk2[keep], r[1], 1e-12, 1e-12, "bwd delete dk")
    _close(ds2[keep], r[3], 1e-12, 1e-12, "bwd delete dscore")
    _close(dg2, r[4], 1e-12, 1e-12, "bwd delete dgain")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
