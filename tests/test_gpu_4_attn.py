"""[a5] tg_bias_attn_fwd on the GPU vs the fp64 oracle (TokenGate pages:
ai.info summary "Key Contributions" items 2-3, "Methodology in Plain
English").  Tolerances: fp32 |diff| <= 1e-5 max(1, |ref|); bf16 max |diff|
<= 2e-2 on O and on LSE."""
import numpy as np
import pytest
import torch

import learned_token_pruning_gate_amd as tg
import oracle
import workloads
from gpu_util import (BF16_ABS, LSE_ABS_BF16, as_f64, assert_close_abs, assert_close_f32,
                      report, to_dev)

pytestmark = pytest.mark.gpu


def make(rng, N, Hq, Hkv, D, dtype, bias=True, qscale=True):
    def draw(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return workloads.to_bf16_bits(x) if dtype == "bf16" else x
    q, k, v = draw((N, Hq, D)), draw((N, Hkv, D)), draw((N, Hkv, D))
    s = rng.standard_normal(N).astype(np.float32) if bias else None
    g = rng.uniform(0.5, 2.0, size=Hq).astype(np.float32)
    c = rng.uniform(1.0, 2.0, size=N).astype(np.float32) if qscale else None
    return q, k, v, s, g, c


def gpu(q, k, v, s, g, c, dtype, causal=True, scale=0.0):
    o, lse = tg.tg_bias_attn_fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype),
                                 None if s is None else to_dev(s), to_dev(g),
                                 None if c is None else to_dev(c), softmax_scale=scale,
                                 causal=causal)
    torch.cuda.synchronize()
    return o, lse


def gpu_split(q, k, v, s, g, c, causal=True):
    """The split-key entry point with a workspace of the queried size (the
    shape must be one that splits)."""
    N, Hq, D = q.shape
    nb = tg.tg_bias_attn_workspace_size(N, Hq, k.shape[1], D, causal)
    assert nb > 0, "shape runs unsplit"
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)   # the call needs no initialised workspace (0xFF.. floats are NaN)
    o, lse = tg.tg_bias_attn_fwd_ws(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                    None if s is None else to_dev(s), to_dev(g), ws,
                                    None if c is None else to_dev(c), causal=causal)
    torch.cuda.synchronize()
    return o, lse


def ref(q, k, v, s, g, c, dtype, causal=True, rows=None):
    N = q.shape[0]
    ss = np.zeros(N) if s is None else s
    return oracle.bias_attn(workloads.as_f64(q, dtype), workloads.as_f64(k, dtype),
                            workloads.as_f64(v, dtype), ss, g, q_scale=c, causal=causal,
                            rows=rows)


@pytest.mark.parametrize("name", ["tiny", "tiny-K32"])
@pytest.mark.parametrize("qscale", [None, "ones", "spread"])
def test_attn_f32_tiny(name, qscale):
    w = workloads.get(name)
    _, a = workloads.generate(w)
    rng = np.random.default_rng(3)
    N = w.n_kept
    s = rng.standard_normal(N).astype(np.float32)
    c = None if qscale is None else (np.ones(N, np.float32) if qscale == "ones"
                                     else rng.uniform(1, 2, N).astype(np.float32))
    o, lse = gpu(a.q, a.k, a.v, s, a.gain, c, "f32")
    ro, rl = ref(a.q, a.k, a.v, s, a.gain, c, "f32")
    assert_close_f32(as_f64(o), ro, "attn_f32_%s_%s" % (name, qscale))
    assert_close_f32(lse.cpu().numpy(), rl, "attn_f32_lse_%s_%s" % (name, qscale))


SHAPES = [  # N, Hq, Hkv, D
    (1, 2, 1, 128), (17, 4, 2, 64), (64, 16, 8, 128), (100, 8, 8, 128),
    (255, 8, 2, 128), (300, 16, 2, 128), (129, 6, 2, 64), (612, 16, 8, 128),
    (1000, 4, 4, 64),
    # head dim 256 (the pages' second supported head dim)
    (1, 2, 1, 256), (100, 4, 2, 256), (513, 8, 2, 256), (129, 2, 2, 256), (300, 8, 1, 256),
    # grids of more than 1024 workgroups: the 8-wave launch (two query
    # blocks per workgroup sharing each key tile)
    (2100, 64, 64, 64), (4500, 32, 8, 64),
]


@pytest.mark.parametrize("N,Hq,Hkv,D", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_attn_bf16_shapes(N, Hq, Hkv, D, causal):
    rng = np.random.default_rng(N * 31 + Hq + D + causal)
    q, k, v, s, g, c = make(rng, N, Hq, Hkv, D, "bf16")
    o, lse = gpu(q, k, v, s, g, c, "bf16", causal=causal)
    ro, rl = ref(q, k, v, s, g, c, "bf16", causal=causal)
    tag = "attn_bf16_N%d_H%d_%d_D%d_c%d" % (N, Hq, Hkv, D, causal)
    assert_close_abs(as_f64(o), ro, BF16_ABS, tag)
    assert_close_abs(lse.cpu().numpy(), rl, LSE_ABS_BF16, tag + "_lse")


# Grids of more than 1024 four-wave workgroups take the large-grid launch
# (8-wave workgroups whose two wave groups alternate between matrix products
# and softmax): 1, 2 and 4 query heads per KV head, head dims 64 and 128,
# ragged last query blocks.  Rows checked: the first and last of every 64-row
# block plus a random sample.
LARGE_SHAPES = [  # N, Hq, Hkv, D
    (4500, 32, 16, 128), (9000, 16, 4, 128), (3001, 64, 64, 128), (4500, 32, 8, 64),
    (8191, 16, 8, 128),
]


@pytest.mark.parametrize("N,Hq,Hkv,D", LARGE_SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_attn_bf16_large_grid(N, Hq, Hkv, D, causal):
    rng = np.random.default_rng(N * 13 + Hq + D + causal)
    q, k, v, s, g, c = make(rng, N, Hq, Hkv, D, "bf16")
    s[rng.choice(N, 20, replace=False)] = -np.inf      # some deleted keys
    o, lse = gpu(q, k, v, s, g, c, "bf16", causal=causal)
    rows = dense_rows(N, block=64, seed=N)
    ro, rl = ref(q, k, v, s, g, c, "bf16", causal=causal, rows=rows)
    tag = "attn_large_N%d_H%d_%d_D%d_c%d" % (N, Hq, Hkv, D, causal)
    assert_close_abs(as_f64(o)[rows], ro, BF16_ABS, tag)
    assert_close_abs(lse.cpu().numpy()[:, rows], rl, LSE_ABS_BF16, tag + "_lse")


@pytest.mark.parametrize("bias,qscale", [(False, False), (True, False), (False, True)])
def test_attn_bf16_optional_inputs(bias, qscale):
    rng = np.random.default_rng(77)
    q, k, v, s, g, c = make(rng, 333, 16, 8, 128, "bf16", bias=bias, qscale=qscale)
    o, lse = gpu(q, k, v, s, g, c, "bf16")
    ro, rl = ref(q, k, v, s, g, c, "bf16")
    assert_close_abs(as_f64(o), ro, BF16_ABS, "attn_bf16_opt_b%d_q%d" % (bias, qscale))


@pytest.mark.parametrize("causal", [True, False])
def test_attn_f32_head_dim_256(causal):
    rng = np.random.default_rng(256 + causal)
    q, k, v, s, g, c = make(rng, 40, 2, 1, 256, "f32")
    o, lse = gpu(q, k, v, s, g, c, "f32", causal=causal)
    ro, rl = ref(q, k, v, s, g, c, "f32", causal=causal)
    assert_close_f32(as_f64(o), ro, "attn_f32_D256_c%d" % causal)
    assert_close_f32(lse.cpu().numpy(), rl, "attn_f32_D256_lse_c%d" % causal)


def test_attn_custom_scale():
    rng = np.random.default_rng(78)
    q, k, v, s, g, c = make(rng, 200, 4, 2, 128, "bf16")
    o, _ = gpu(q, k, v, s, g, c, "bf16", scale=0.05)
    ro, _ = oracle.bias_attn(workloads.as_f64(q, "bf16"), workloads.as_f64(k, "bf16"),
                             workloads.as_f64(v, "bf16"), s, g, q_scale=c, scale=0.05)
    assert_close_abs(as_f64(o), ro, BF16_ABS, "attn_bf16_scale005")


# ---- invariants on the GPU --------------------------------------------------
def test_attn_zero_bias_equals_no_bias_bitwise():
    rng = np.random.default_rng(80)
    q, k, v, _, g, c = make(rng, 500, 16, 8, 128, "bf16")
    o1, l1 = gpu(q, k, v, np.zeros(500, np.float32), g, c, "bf16")
    o2, l2 = gpu(q, k, v, None, g, c, "bf16")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_attn_row0_is_v0_exactly():
    """Row 0 sees only key 0, whose weight is exactly 1: O[0] = V[0] bitwise."""
    rng = np.random.default_rng(81)
    q, k, v, s, g, c = make(rng, 70, 8, 4, 128, "bf16")
    o, _ = gpu(q, k, v, s, g, c, "bf16")
    o0 = o[0].view(torch.int16).cpu().numpy().view(np.uint16)
    for h in range(8):
        assert np.array_equal(o0[h], v[0, h // 2])


def test_attn_neg_inf_score_deletes_key():
    rng = np.random.default_rng(82)
    N = 260
    q, k, v, s, g, c = make(rng, N, 8, 4, 128, "bf16")
    for cdel in (5, 64, 200):
        s2 = s.copy()
        s2[cdel] = -np.inf
        o, _ = gpu(q, k, v, s2, g, c, "bf16")
        keep = np.array([i for i in range(N) if i != cdel])
        o_red, _ = gpu(q[keep], k[keep], v[keep], s[keep], g, c[keep], "bf16")
        assert_close_abs(as_f64(o)[keep], as_f64(o_red), BF16_ABS, "attn_delete_%d" % cdel)


def test_attn_key_constant_bias_is_noop():
    rng = np.random.default_rng(83)
    q, k, v, s, g, c = make(rng, 300, 16, 8, 128, "bf16")
    o1, l1 = gpu(q, k, v, s, g, c, "bf16")
    o2, l2 = gpu(q, k, v, s + np.float32(2.5), g, c, "bf16")
    assert_close_abs(as_f64(o1), as_f64(o2), BF16_ABS, "attn_const_bias")
    shift = c[None, :].astype(np.float64) * g[:, None].astype(np.float64) * 2.5
    assert_close_abs(l2.cpu().numpy() - l1.cpu().numpy(), shift, LSE_ABS_BF16,
                     "attn_const_bias_lse")


def test_attn_fully_masked_row():
    rng = np.random.default_rng(84)
    q, k, v, s, g, c = make(rng, 40, 4, 2, 64, "bf16")
    s[0] = -np.inf                  # row 0 sees only key 0
    o, lse = gpu(q, k, v, s, g, c, "bf16")
    assert torch.all(o[0].float() == 0)
    assert torch.all(torch.isneginf(lse[:, 0]))
    ro, rl = ref(q, k, v, s, g, c, "bf16")
    assert_close_abs(as_f64(o)[1:], ro[1:], BF16_ABS, "attn_masked_row_rest")


def test_attn_deterministic():
    rng = np.random.default_rng(85)
    q, k, v, s, g, c = make(rng, 2512, 16, 8, 128, "bf16")
    o1, l1 = gpu(q, k, v, s, g, c, "bf16")
    o2, l2 = gpu(q, k, v, s, g, c, "bf16")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


# ---- full sizes --------------------------------------------------------------
@pytest.mark.parametrize("entry", ["unsplit", "split"])
def test_attn_bf16_t16k_full(entry):
    """N = 2512 kept tokens, 16/8 heads, D = 128, causal: every output row.
    "split" is the launch the chain and the benchmark time
    (tg_bias_attn_fwd_ws with the queried workspace); gpu_split fails if the
    cost model stops splitting this shape."""
    w = workloads.get("t16k")
    _, a = workloads.generate(w)
    rng = np.random.default_rng(90)
    s = rng.standard_normal(w.n_kept).astype(np.float32)
    if entry == "split":
        o, lse = gpu_split(a.q, a.k, a.v, s, a.gain, None)
    else:
        o, lse = gpu(a.q, a.k, a.v, s, a.gain, None, "bf16")
    ro, rl = ref(a.q, a.k, a.v, s, a.gain, None, "bf16")
    assert_close_abs(as_f64(o), ro, BF16_ABS, "attn_bf16_t16k_full_" + entry)
    assert_close_abs(lse.cpu().numpy(), rl, LSE_ABS_BF16, "attn_bf16_t16k_full_lse_" + entry)


def dense_rows(N, block=128, seed=91):
    """Rows checked on the dense 32k prompt: the first and last row of every
    block of `block` queries (a workgroup's query block of the large-grid
    launch), the tail, and a random sample."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, N, block)
    return np.unique(np.concatenate([starts, np.minimum(starts + block - 1, N - 1),
                                     [1, 63, 64, 65], np.arange(N - 40, N),
                                     rng.choice(N, size=60, replace=False)]))


def test_attn_bf16_dense_sampled_rows():
    """N = 32768 (every token kept): the first and last row of each 128-query
    block plus a random sample, with the workload's drawn key scores and its
    per-query scale array, through tg_bias_attn_fwd_ws as the benchmark
    calls it (no workspace: the shape fills the chip unsplit)."""
    w = workloads.get("t32k-dense")
    _, a = workloads.generate(w)
    N = w.n_kept
    assert tg.tg_bias_attn_workspace_size(N, w.Hq, w.Hkv, w.D) == 0
    c = workloads.q_scale_pos_rank(np.arange(N))
    o, lse = tg.tg_bias_attn_fwd_ws(to_dev(a.q, "bf16"), to_dev(a.k, "bf16"),
                                    to_dev(a.v, "bf16"), to_dev(a.drawn_scores),
                                    to_dev(a.gain), None, to_dev(c))
    torch.cuda.synchronize()
    rows = dense_rows(N)
    ro, rl = ref(a.q, a.k, a.v, a.drawn_scores, a.gain, c, "bf16", rows=rows)
    assert_close_abs(as_f64(o)[rows], ro, BF16_ABS, "attn_bf16_dense_sampled")
    assert_close_abs(lse.cpu().numpy()[:, rows], rl, LSE_ABS_BF16, "attn_bf16_dense_lse")


# ---- split-key path (tg_bias_attn_fwd_ws) ---------------------------------------
SPLIT_SHAPES = [  # N, Hq, Hkv, D, causal: each takes the split (3 to 7 chunks per long row)
    (1000, 16, 2, 128, True), (2000, 8, 8, 128, False),    # 4 and 1 heads per KV head
    (1000, 4, 4, 64, True), (1000, 4, 4, 64, False),       # 1 head per KV head
    (1700, 6, 2, 64, True), (1700, 6, 2, 64, False),       # 3 heads per KV head
    (2512, 8, 4, 128, True), (2512, 16, 8, 128, False),    # the 16k prompt's kept set size
    (2512, 16, 8, 128, True),                              # ... at its heads: the timed launch
    (1500, 16, 8, 128, True),
    (1800, 12, 4, 64, True),
    (2999, 8, 8, 128, True),                               # ragged last query block
    (4000, 8, 8, 128, True),
    (2000, 16, 8, 64, True),
    # head dim 256: one workgroup per CU
    (2512, 8, 2, 256, True), (2512, 8, 2, 256, False),
    (1000, 4, 2, 256, True),
    (700, 6, 2, 256, True),
]


@pytest.mark.parametrize("N,Hq,Hkv,D,causal", SPLIT_SHAPES)
def test_attn_bf16_split_shapes(N, Hq, Hkv, D, causal):
    rng = np.random.default_rng(N * 37 + Hq + D + causal)
    q, k, v, s, g, c = make(rng, N, Hq, Hkv, D, "bf16")
    o, lse = gpu_split(q, k, v, s, g, c, causal=causal)
    ro, rl = ref(q, k, v, s, g, c, "bf16", causal=causal)
    tag = "attn_split_N%d_H%d_%d_D%d_c%d" % (N, Hq, Hkv, D, causal)
    assert_close_abs(as_f64(o), ro, BF16_ABS, tag)
    assert_close_abs(lse.cpu().numpy(), rl, LSE_ABS_BF16, tag + "_lse")


def test_attn_split_masked_chunks():
    """Keys 0..1599 deleted by a -inf score: for the long rows, whole chunks
    hold no visible key (running max -inf, sum 0) and the merge must skip
    them; rows 0..1599 see no key at all (O = 0, lse = -inf)."""
    rng = np.random.default_rng(86)
    N = 2512
    q, k, v, s, g, c = make(rng, N, 8, 4, 128, "bf16")
    s[:1600] = -np.inf
    o, lse = gpu_split(q, k, v, s, g, c)
    assert torch.all(o[:1600].float() == 0)
    assert torch.all(torch.isneginf(lse[:, :1600]))
    ro, rl = ref(q[1600:], k[1600:], v[1600:], s[1600:], g, c[1600:], "bf16")
    assert_close_abs(as_f64(o)[1600:], ro, BF16_ABS, "attn_split_masked_rest")
    assert_close_abs(lse.cpu().numpy()[:, 1600:], rl, LSE_ABS_BF16, "attn_split_masked_lse")


def test_attn_split_all_masked():
    rng = np.random.default_rng(87)
    q, k, v, s, g, c = make(rng, 2512, 8, 4, 128, "bf16")
    s[:] = -np.inf
    o, lse = gpu_split(q, k, v, s, g, c)
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(lse))


def test_attn_split_matches_unsplit_and_is_deterministic():
    rng = np.random.default_rng(88)
    q, k, v, s, g, c = make(rng, 2512, 8, 4, 128, "bf16")
    o1, l1 = gpu_split(q, k, v, s, g, c)
    o2, l2 = gpu_split(q, k, v, s, g, c)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    o3, l3 = gpu(q, k, v, s, g, c, "bf16")
    assert_close_abs(as_f64(o1), as_f64(o3), BF16_ABS, "attn_split_vs_unsplit")
    # the first 64 queries see one key tile: the same arithmetic either way
    assert torch.equal(o1[:64].view(torch.int16), o3[:64].view(torch.int16))


def test_attn_split_workspace_unused_shape_runs_unsplit():
    """A shape the split does not apply to accepts a NULL workspace and
    matches tg_bias_attn_fwd bit for bit."""
    rng = np.random.default_rng(89)
    q, k, v, s, g, c = make(rng, 100, 16, 8, 128, "bf16")
    assert tg.tg_bias_attn_workspace_size(100, 16, 8, 128) == 0
    o1, l1 = tg.tg_bias_attn_fwd_ws(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                    to_dev(s), to_dev(g), None, to_dev(c))
    o2, l2 = gpu(q, k, v, s, g, c, "bf16")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_attn_bf16_t16k_full_split():
    """The 16k prompt's kept set at head dim 256 (8/2 heads) through the
    split path: every output row."""
    w = workloads.get("t16k-d256")
    _, a = workloads.generate(w)
    rng = np.random.default_rng(92)
    s = rng.standard_normal(w.n_kept).astype(np.float32)
    o, lse = gpu_split(a.q, a.k, a.v, s, a.gain, None)
    ro, rl = ref(a.q, a.k, a.v, s, a.gain, None, "bf16")
    assert_close_abs(as_f64(o), ro, BF16_ABS, "attn_bf16_t16k_full_split")
    assert_close_abs(lse.cpu().numpy(), rl, LSE_ABS_BF16, "attn_bf16_t16k_full_split_lse")


@pytest.mark.parametrize("entry", ["unsplit", "split"])
def test_attn_small_q_scale_deletes_keys(entry):
    """A -inf score deletes its key at any per-query scale, including ones
    far below 1 (here 0.1 and 0.01): rows whose visible keys are all deleted
    give O = 0 and lse = -inf, and the other rows match the oracle on the
    keys that remain."""
    rng = np.random.default_rng(93)
    N, Hq, Hkv, D = 2512, 8, 4, 128
    q, k, v, s, g, _ = make(rng, N, Hq, Hkv, D, "bf16")
    c = np.where(np.arange(N) % 2 == 0, 0.1, 0.01).astype(np.float32)
    s[:300] = -np.inf
    if entry == "split":
        o, lse = gpu_split(q, k, v, s, g, c)
    else:
        o, lse = gpu(q, k, v, s, g, c, "bf16")
    assert torch.all(o[:300].float() == 0)
    assert torch.all(torch.isneginf(lse[:, :300]))
    ro, rl = ref(q[300:], k[300:], v[300:], s[300:], g, c[300:], "bf16")
    assert_close_abs(as_f64(o)[300:], ro, BF16_ABS, "attn_small_qscale_" + entry)
    assert_close_abs(lse.cpu().numpy()[:, 300:], rl, LSE_ABS_BF16,
                     "attn_small_qscale_lse_" + entry)


@pytest.mark.parametrize("Hq,Hkv,D,causal", [
    (8, 4, 128, True), (8, 4, 128, False), (8, 2, 256, True), (8, 4, 64, False)])
@pytest.mark.parametrize("entry", ["unsplit", "split"])
def test_attn_rising_logits_move_the_reference(entry, Hq, Hkv, D, causal):
    """Logits that keep rising along the keys move the softmax reference many
    times within a row: scores grow by 0.05 per key (about 180 log2 units
    over the prompt at gain 1), so the weights against a reference taken
    early pass 2^32 every few tiles, and one key's score jumps by 150 so
    that its weight overflows fp32 against any earlier reference.  Every
    row against the oracle, causal and not, at head dims 64, 128 and 256
    (every shape here also splits)."""
    rng = np.random.default_rng(97 + D + (1 if causal else 0))
    N = 2512
    q, k, v, _, g, c = make(rng, N, Hq, Hkv, D, "bf16")
    s = (0.05 * np.arange(N) + 0.3 * rng.standard_normal(N)).astype(np.float32)
    s[1500] += 150.0
    g = rng.uniform(0.8, 1.2, size=Hq).astype(np.float32)
    if entry == "split":
        o, lse = gpu_split(q, k, v, s, g, c, causal=causal)
    else:
        o, lse = gpu(q, k, v, s, g, c, "bf16", causal=causal)
    ro, rl = ref(q, k, v, s, g, c, "bf16", causal=causal)
    name = "attn_rising_%s_D%d_c%d" % (entry, D, causal)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    assert_close_abs(as_f64(o), ro, BF16_ABS, name)
    assert_close_abs(lse.cpu().numpy(), rl, LSE_ABS_BF16, name + "_lse")
