"""[a4] tg_compact_gather on the GPU vs the oracle: bit-exact rows, positions
and scores (TokenGate pages: ai.info summary "Key Contributions" item 1)."""
import numpy as np
import pytest
import torch

import learned_token_pruning_gate_amd as tg
import oracle
import workloads
from gpu_util import dev, report, to_dev

pytestmark = pytest.mark.gpu


def _case(rng, dtype, T, d, N, extra_cols=0):
    width = d + extra_cols
    if dtype == "bf16":
        full = rng.integers(0, 1 << 16, size=(T, width), dtype=np.uint16)
    else:
        full = rng.standard_normal((T, width)).astype(np.float32)
        full.ravel()[:: 97] = np.nan
    scores = rng.standard_normal(T).astype(np.float32)
    scores[:: 13] = np.nan
    idx = np.sort(rng.choice(T, size=N, replace=False)).astype(np.int32)
    return full, scores, idx


@pytest.mark.parametrize("dtype,T,d,N,extra", [
    ("bf16", 257, 24, 77, 0),
    ("bf16", 1000, 2048, 300, 0),
    ("bf16", 999, 2048, 999, 8),        # identity, row stride > d
    ("bf16", 50, 7, 20, 1),             # 14-byte rows: 2-byte copy path
    ("bf16", 64, 6, 30, 0),             # 12-byte rows: 4-byte copy path
    ("f32", 513, 256, 128, 0),
    ("f32", 100, 3, 50, 1),
    ("bf16", 5, 8, 1, 0),
])
def test_gather_matches_oracle(dtype, T, d, N, extra):
    rng = np.random.default_rng(T * 7 + d)
    full, scores, idx = _case(rng, dtype, T, d, N, extra)
    host_rows = np.ascontiguousarray(full[:, :d])
    ref_rows, ref_pos, ref_sk = oracle.compact_gather(host_rows, scores, idx)
    dfull = to_dev(full, dtype)
    resid = dfull[:, :d]
    rk, pos, sk = tg.tg_compact_gather(resid, to_dev(scores), to_dev(idx), N)
    torch.cuda.synchronize()
    got_rows = rk.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" \
        else rk.cpu().numpy()
    assert got_rows.tobytes() == ref_rows.tobytes()
    assert np.array_equal(pos.cpu().numpy(), ref_pos)
    assert sk.cpu().numpy().tobytes() == ref_sk.tobytes()
    report("gather_%s_T%d_d%d_N%d" % (dtype, T, d, N), bit_exact=True)


def test_gather_empty_and_optional_outputs():
    rng = np.random.default_rng(1)
    full, scores, idx = _case(rng, "bf16", 64, 16, 10)
    resid = to_dev(full, "bf16")
    rk, pos, sk = tg.tg_compact_gather(resid, to_dev(scores), to_dev(idx), 0)
    assert rk.shape == (0, 16) and pos.shape == (0,)
    # positions and scores only (no row copy)
    lib = tg.load()
    pos = torch.full((10,), -7, dtype=torch.int32, device=dev())
    st = lib.tg_compact_gather(tg.TG_DTYPE_BF16, 64, 10, 16, resid.data_ptr(), 16,
                               to_dev(scores).data_ptr(), to_dev(idx).data_ptr(), None, 16,
                               pos.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), idx)


def test_gather_out_of_range_index_gives_zero_row():
    rng = np.random.default_rng(2)
    T, d = 40, 16
    full, scores, _ = _case(rng, "bf16", T, d, 5)
    idx = np.array([0, -1, 39, 40, 2**30], dtype=np.int32)
    rk, pos, sk = tg.tg_compact_gather(to_dev(full, "bf16"), to_dev(scores), to_dev(idx), 5)
    torch.cuda.synchronize()
    rows = rk.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(rows[0], full[0]) and np.array_equal(rows[2], full[39])
    assert np.all(rows[[1, 3, 4]] == 0)
    assert pos.cpu().numpy().tolist() == [0, -1, 39, -1, -1]
    s = sk.cpu().numpy()
    assert s[1] == 0 and s[3] == 0 and s[4] == 0


@pytest.mark.parametrize("name", ["t16k", "t128k", "t32k-dense"])
def test_gather_full_size(name):
    """At the workload's real shape: the kept set of random scores, gathered."""
    w = workloads.get(name)
    rng = np.random.default_rng(w.seed + 100)
    resid = rng.integers(0, 1 << 16, size=(w.T, w.d), dtype=np.uint16)
    prunable = workloads.prunable_mask(w)
    scores = rng.standard_normal(w.T).astype(np.float32)
    idx = oracle.topk_select(scores, prunable, w.K)
    assert len(idx) == w.n_kept
    rk, pos, sk = tg.tg_compact_gather(to_dev(resid, "bf16"), to_dev(scores), to_dev(idx),
                                       len(idx))
    torch.cuda.synchronize()
    got = rk.view(torch.int16).cpu().numpy().view(np.uint16)
    assert got.tobytes() == resid[idx].tobytes()
    assert np.array_equal(pos.cpu().numpy(), idx)
    assert sk.cpu().numpy().tobytes() == scores[idx].tobytes()
    report("gather_full_" + name, N=len(idx), bit_exact=True)
