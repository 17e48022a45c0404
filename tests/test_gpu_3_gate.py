"""[a1] tg_gate_score on the GPU vs the fp64 oracle (TokenGate pages:
ai.info summary "Key Contributions" item 1; README mirror "How it works").

Tolerance: fp32 path |diff| <= 1e-5 max(1, |ref|); bf16 path max |diff| <= 2e-2
(the bf16 path multiplies exact bf16 inputs on MFMA with fp32 accumulation;
a non-unit RMSNorm weight is applied to x before a bf16 rounding)."""
import math

import numpy as np
import pytest
import torch

import learned_token_pruning_gate_amd as tg
import oracle
import workloads
from gpu_util import BF16_ABS, assert_close_abs, assert_close_f32, report, to_dev

pytestmark = pytest.mark.gpu


def run_gpu(resid, prunable, w1, w2, b2, gamma, b1, eps, dtype, stride_pad=0, packed=False):
    if stride_pad:
        full = np.zeros((resid.shape[0], resid.shape[1] + stride_pad), resid.dtype)
        full[:, : resid.shape[1]] = resid
        r = to_dev(full, dtype)[:, : resid.shape[1]]
    else:
        r = to_dev(resid, dtype)
    if packed:
        assert gamma is None and dtype == "bf16"
        wp = tg.tg_gate_pack_w1(to_dev(w1, dtype))
        out = tg.tg_gate_score_packed(r, to_dev(prunable), wp, to_dev(w2), b2=b2,
                                      b1=None if b1 is None else to_dev(b1), eps=eps)
    else:
        out = tg.tg_gate_score(r, to_dev(prunable), to_dev(w1, dtype), to_dev(w2), b2=b2,
                               rms_weight=None if gamma is None else to_dev(gamma),
                               b1=None if b1 is None else to_dev(b1), eps=eps)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def run_oracle(resid, prunable, w1, w2, b2, gamma, b1, eps, dtype):
    return oracle.gate_score(workloads.as_f64(resid, dtype), prunable,
                             workloads.as_f64(w1, dtype), w2, b2=b2, gamma=gamma, b1=b1,
                             eps=eps)


def test_gate_f32_tiny_workload():
    w = workloads.get("tiny")
    g, _ = workloads.generate(w)
    args = (g.resid, g.prunable, g.w1, g.w2, g.b2, g.gamma, g.b1, g.eps, w.dtype)
    got = run_gpu(*args)
    ref = run_oracle(*args)
    assert_close_f32(got, ref, "gate_f32_tiny")
    assert np.all(got[g.prunable == 0] == 0)


@pytest.mark.parametrize("T,d,h,with_gamma,with_b1,frac", [
    (1000, 2048, 256, False, False, 0.9),   # ragged tail (1000 = 15*64 + 40)
    (777, 264, 64, True, True, 0.5),        # d not a multiple of 64
    (300, 128, 128, True, False, 1.0),
    (513, 512, 192, False, True, 0.3),
    (64, 2048, 256, False, False, 0.0),     # no prunable token at all
    (1, 64, 64, True, True, 1.0),
    (4096, 1024, 256, True, True, 0.95),
])
def test_gate_bf16_cases(T, d, h, with_gamma, with_b1, frac):
    rng = np.random.default_rng(T + d + h)
    resid = workloads.to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32) *
                                   rng.uniform(0.2, 3.0, size=(T, 1)).astype(np.float32))
    w1 = workloads.to_bf16_bits(rng.standard_normal((h, d)).astype(np.float32) / math.sqrt(d))
    w2 = (rng.standard_normal(h) / math.sqrt(h)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, size=d).astype(np.float32) if with_gamma else None
    b1 = (rng.standard_normal(h) * 0.2).astype(np.float32) if with_b1 else None
    prunable = (rng.random(T) < frac).astype(np.uint8)
    prunable[T // 2: T // 2 + 70] = 0           # a whole non-prunable tile
    args = (resid, prunable, w1, w2, 0.125, gamma, b1, 1e-6, "bf16")
    got = run_gpu(*args, stride_pad=8 if T % 2 else 0)
    ref = run_oracle(*args)
    assert np.all(got[prunable == 0] == 0)
    assert_close_abs(got, ref, BF16_ABS, "gate_bf16_T%d_d%d_h%d" % (T, d, h))


def _random_case(T, d, h, with_gamma, with_b1, frac):
    rng = np.random.default_rng(T + d + h)
    resid = workloads.to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32) *
                                   rng.uniform(0.2, 3.0, size=(T, 1)).astype(np.float32))
    w1 = workloads.to_bf16_bits(rng.standard_normal((h, d)).astype(np.float32) / math.sqrt(d))
    w2 = (rng.standard_normal(h) / math.sqrt(h)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, size=d).astype(np.float32) if with_gamma else None
    b1 = (rng.standard_normal(h) * 0.2).astype(np.float32) if with_b1 else None
    prunable = (rng.random(T) < frac).astype(np.uint8)
    prunable[T // 2: T // 2 + 70] = 0
    return (resid, prunable, w1, w2, 0.125, gamma, b1, 1e-6, "bf16")


@pytest.mark.parametrize("T,d,h,with_b1,frac", [
    (1000, 2048, 256, False, 0.9),   # ragged tail, fully unrolled 32-stage kernel
    (300, 128, 128, False, 1.0),     # two stages: shorter than the load ring
    (513, 192, 64, True, 0.7),       # three stages
    (513, 512, 192, True, 0.3),
    (700, 1088, 256, True, 0.8),     # 17 stages: the ring wraps with a partial turn
    (64, 2048, 256, False, 0.0),     # no prunable token at all
    (4096, 1024, 256, True, 0.95),
])
@pytest.mark.parametrize("packed", [False, True])
def test_gate_bf16_stream_cases(T, d, h, with_b1, frac, packed):
    """Shapes the streaming kernel takes (unit RMSNorm weight, d % 64 == 0),
    with W1 row-major and packed."""
    args = _random_case(T, d, h, False, with_b1, frac)
    got = run_gpu(*args, stride_pad=8 if T % 2 else 0, packed=packed)
    ref = run_oracle(*args)
    assert np.all(got[args[1] == 0] == 0)
    assert_close_abs(got, ref, BF16_ABS,
                     "gate_bf16_stream_T%d_d%d_h%d_%s" % (T, d, h, "packed" if packed else "rowmajor"))


@pytest.mark.parametrize("T,d,with_b1,frac", [
    (66000, 1088, False, 0.6),  # 128-row tiles, 17 stages (the ring wraps partway)
])
@pytest.mark.parametrize("packed", [False, True])
def test_gate_bf16_stream_128_rows(T, d, with_b1, frac, packed):
    """At h = 256 and a hidden size other than 2048, prompts long enough for
    two rounds of 128-row workgroups on every CU take 128-row tiles: every
    row against the oracle."""
    args = _random_case(T, d, 256, False, with_b1, frac)
    got = run_gpu(*args, stride_pad=8 if T % 2 else 0, packed=packed)
    ref = run_oracle(*args)
    assert np.all(got[args[1] == 0] == 0)
    assert_close_abs(got, ref, BF16_ABS,
                     "gate_bf16_stream128_T%d_d%d_%s" % (T, d, "packed" if packed else "rowmajor"))


@pytest.mark.parametrize("T,d,with_b1,frac", [
    (33001, 2048, True, 0.8),   # two 64-row workgroups per CU, 32-stage kernel, ragged tail
    (40000, 1088, False, 0.6),  # the same, 17 stages (the ring wraps partway)
    (65613, 2048, True, 0.8),   # 32-stage kernel above the 128-row threshold, ragged tail
])
@pytest.mark.parametrize("packed", [False, True])
def test_gate_bf16_stream_two_per_cu(T, d, with_b1, frac, packed):
    """At h = 256, prompts with two rounds of 64-row workgroups per CU but
    not two of 256-row ones at hidden size 2048 (or not two of 128-row ones
    at other sizes; 32705 <= T < 130817 or 65409 on 256 CUs) run two
    workgroups on each CU at a time: against the oracle on the first and
    last rows, every workgroup's first and last rows, and random rows."""
    args = _random_case(T, d, 256, False, with_b1, frac)
    resid, prunable, w1, w2, b2, gamma, b1, eps, dt = args
    got = run_gpu(*args, stride_pad=8 if T % 2 else 0, packed=packed)
    rng = np.random.default_rng(T + d)
    edges = np.arange(0, T, 64)
    rows = np.unique(np.concatenate([
        np.arange(0, 200), np.arange(T - 200, T), edges, np.minimum(edges + 63, T - 1),
        rng.choice(T, size=2000, replace=False)]))
    sub = np.zeros(T, np.uint8)
    sub[rows] = prunable[rows]
    ref = run_oracle(resid[rows], sub[rows], w1, w2, b2, gamma, b1, eps, dt)
    assert np.all(got[prunable == 0] == 0)
    assert np.count_nonzero(got) <= int(prunable.sum())
    assert_close_abs(got[rows], ref, BF16_ABS,
                     "gate_bf16_stream2wg_T%d_d%d_%s" % (T, d, "packed" if packed else "rowmajor"))


@pytest.mark.parametrize("T,d,with_b1,frac", [
    (131172, 2048, True, 0.8),   # 256-row tiles, 32-stage kernel, ragged last tile
    (140001, 1088, False, 0.6),  # 256-row tiles, 17 stages (the ring wraps partway)
])
@pytest.mark.parametrize("packed", [False, True])
def test_gate_bf16_stream_256_rows(T, d, with_b1, frac, packed):
    """At h = 256, prompts long enough for two rounds of 256-row workgroups
    on every CU take 256-row tiles: against the oracle on the first and last
    rows, the rows at every tenth workgroup boundary and random rows."""
    args = _random_case(T, d, 256, False, with_b1, frac)
    resid, prunable, w1, w2, b2, gamma, b1, eps, dt = args
    got = run_gpu(*args, stride_pad=8 if T % 2 else 0, packed=packed)
    rng = np.random.default_rng(T + d)
    edges = np.arange(0, T, 2560)
    rows = np.unique(np.concatenate([
        np.arange(0, 300), np.arange(T - 300, T), edges, np.minimum(edges + 255, T - 1),
        rng.choice(T, size=2000, replace=False)]))
    sub = np.zeros(T, np.uint8)
    sub[rows] = prunable[rows]
    ref = run_oracle(resid[rows], sub[rows], w1, w2, b2, gamma, b1, eps, dt)
    assert np.all(got[prunable == 0] == 0)
    assert np.count_nonzero(got) <= int(prunable.sum())
    assert_close_abs(got[rows], ref, BF16_ABS,
                     "gate_bf16_stream256_T%d_d%d_%s" % (T, d, "packed" if packed else "rowmajor"))


@pytest.mark.parametrize("h,d", [(256, 2048), (64, 128), (192, 320)])
def test_gate_pack_w1_layout(h, d):
    """The packed W1 is the documented permutation of W1's elements: block
    ((ks * h/16 + ht) * 2 + kk) holds, at lane l, W1[16 ht + l % 16]
    [64 ks + 32 kk + 8 (l / 16) .. + 7]."""
    rng = np.random.default_rng(h * d)
    w1 = workloads.to_bf16_bits(rng.standard_normal((h, d)).astype(np.float32))
    wp = tg.tg_gate_pack_w1(to_dev(w1, "bf16"))
    torch.cuda.synchronize()
    got = wp.view(torch.int16).cpu().numpy().view(np.uint16)
    blocks = got.reshape(d // 64, h // 16, 2, 4, 16, 8)   # ks, ht, kk, l // 16, l % 16, e
    want = w1.reshape(h // 16, 16, d // 64, 2, 4, 8).transpose(2, 0, 3, 4, 1, 5)
    assert np.array_equal(blocks, want)


def test_gate_packed_equals_rowmajor_bitwise():
    """Packed and row-major W1 feed the same kernel in the same order."""
    w = workloads.get("t16k")
    g, _ = workloads.generate(w)
    a = run_gpu(g.resid, g.prunable, g.w1, g.w2, g.b2, None, None, g.eps, w.dtype)
    b = run_gpu(g.resid, g.prunable, g.w1, g.w2, g.b2, None, None, g.eps, w.dtype, packed=True)
    assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("weight", ["explicit", "null", "packed"])
def test_gate_bf16_t16k_full(weight):
    """Every row of the 16k workload; an explicit all-ones RMSNorm weight and
    a NULL one (the same values) take different kernels."""
    w = workloads.get("t16k")
    g, _ = workloads.generate(w)
    gamma = g.gamma if weight == "explicit" else None
    args = (g.resid, g.prunable, g.w1, g.w2, g.b2, gamma, g.b1, g.eps, w.dtype)
    got = run_gpu(*args, packed=weight == "packed")
    ref = run_oracle(*args)
    assert_close_abs(got, ref, BF16_ABS, "gate_bf16_t16k_full_" + weight)


@pytest.mark.parametrize("name,packed", [("t32k-K2000", False), ("t128k", False),
                                         ("t128k", True)])
def test_gate_bf16_sampled_rows(name, packed):
    """Full-size launch; the oracle checks a sample of rows (first, last,
    every tile boundary region and random rows)."""
    w = workloads.get(name)
    g, _ = workloads.generate(w)
    got = run_gpu(g.resid, g.prunable, g.w1, g.w2, g.b2, None, g.b1, g.eps, w.dtype,
                  packed=packed)
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([
        np.arange(0, 300), np.arange(w.T - 300, w.T),
        rng.choice(w.T, size=3000, replace=False)]))
    sub_mask = np.zeros(w.T, np.uint8)
    sub_mask[rows] = g.prunable[rows]
    ref = oracle.gate_score(workloads.as_f64(g.resid[rows], w.dtype), sub_mask[rows],
                            workloads.as_f64(g.w1, w.dtype), g.w2, b2=g.b2, gamma=g.gamma,
                            b1=g.b1, eps=g.eps)
    assert_close_abs(got[rows], ref, BF16_ABS,
                     "gate_bf16_%s_sampled%s" % (name, "_packed" if packed else ""))
    assert np.all(got[g.prunable == 0] == 0)
    assert np.count_nonzero(got) == w.n_prunable


def test_gate_deterministic():
    w = workloads.get("t16k")
    g, _ = workloads.generate(w)
    a = run_gpu(g.resid, g.prunable, g.w1, g.w2, g.b2, None, None, g.eps, w.dtype)
    b = run_gpu(g.resid, g.prunable, g.w1, g.w2, g.b2, None, None, g.eps, w.dtype)
    assert a.tobytes() == b.tobytes()
