"""[a2, a3] tg_topk_select on the GPU vs the oracle, bit-exact on identical
fp32 scores (TokenGate pages: ai.info summary "Key Contributions" item 1 and
"Methodology in Plain English"; README mirror "Quick start" for K = None)."""
import numpy as np
import pytest
import torch

import learned_token_pruning_gate_amd as tg
import oracle
import workloads
from gpu_util import dev, report, to_dev

pytestmark = pytest.mark.gpu


def gpu_select(scores, prunable, K, workspace=None, capacity=None):
    T = len(scores)
    kept = torch.full((capacity if capacity is not None else max(T, 1),), -5,
                      dtype=torch.int32, device=dev())
    kept, n = tg.tg_topk_select(to_dev(scores), to_dev(prunable), K, kept_idx=kept,
                                workspace=workspace)
    torch.cuda.synchronize()
    n = int(n.item())
    return kept.cpu().numpy(), n


def check(scores, prunable, K, name, workspace=None):
    ref = oracle.topk_select(scores, prunable, K)
    got, n = gpu_select(scores, prunable, K, workspace)
    assert n == len(ref), (name, n, len(ref))
    assert np.array_equal(got[:n], ref), name
    report("select_" + name, T=len(scores), K=K, N=n, bit_exact=True)


def _scores(rng, T, kind):
    s = rng.standard_normal(T).astype(np.float32)
    if kind == "ties":
        s = np.round(s * 2).astype(np.float32) / 2
    elif kind == "special":
        sp = np.array([np.nan, -0.0, 0.0, np.inf, -np.inf, 1e-45, -1e-45], np.float32)
        pick = rng.random(T) < 0.2
        s[pick] = rng.choice(sp, size=int(pick.sum()))
    elif kind == "equal":
        s[:] = 1.5
    elif kind == "few":
        s = rng.integers(-3, 4, size=T).astype(np.float32)
    return s


@pytest.mark.parametrize("T", [1, 7, 1000, 1023, 1024, 1025, 4097, 16384, 24576, 24577, 32767,
                               32768, 32769, 100003, 524288, 524289])
@pytest.mark.parametrize("kind", ["normal", "ties", "special", "equal", "few"])
def test_select_random(T, kind):
    rng = np.random.default_rng(T + len(kind))
    s = _scores(rng, T, kind)
    prunable = (rng.random(T) < 0.85).astype(np.uint8)
    nP = int(prunable.sum())
    for K in sorted({0, 1, max(nP // 3, 1), max(nP - 1, 0), nP, nP + 5}):
        check(s, prunable, K, "%s_T%d_K%d" % (kind, T, K))


def test_select_contiguous_span_and_budgets():
    """The README's budget sweep (None, 2000, 500, 100) on a 32,191-token
    prompt with 44 non-prunable tokens: kept = min(K, |P|) + 44."""
    T, nNP = 32191, 44
    rng = np.random.default_rng(5)
    prunable = np.ones(T, np.uint8)
    prunable[:30] = 0
    prunable[-14:] = 0
    s = rng.standard_normal(T).astype(np.float32)
    for K, want in [(T, T), (2000, 2044), (500, 544), (100, 144)]:
        ref = oracle.topk_select(s, prunable, K)
        got, n = gpu_select(s, prunable, K)
        assert n == want == len(ref) and np.array_equal(got[:n], ref)


def test_select_tie_cut_inside_block():
    T = 5000
    prunable = np.ones(T, np.uint8)
    s = np.full(T, -1.0, np.float32)
    s[3000:3064] = 2.0
    s[10:20] = 3.0
    for K in (10, 11, 40, 73, 74, 75):
        check(s, prunable, K, "tieblock_K%d" % K)


def test_select_workspace_reuse_and_self_cleaning():
    rng = np.random.default_rng(8)
    T1, T2 = 70000, 3000
    ws = torch.zeros(tg.tg_topk_workspace_size(T1), dtype=torch.uint8, device=dev())
    for T, K in [(T1, 1234), (T2, 77), (T1, 0), (T2, T2), (T1, 50000)]:
        s = _scores(rng, T, "ties")
        p = (rng.random(T) < 0.9).astype(np.uint8)
        check(s, p, K, "reuse_T%d_K%d" % (T, K), workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0, "workspace not left zeroed"


def test_select_capacity_smaller_than_kept():
    rng = np.random.default_rng(9)
    T = 3000
    s = rng.standard_normal(T).astype(np.float32)
    p = np.ones(T, np.uint8)
    ref = oracle.topk_select(s, p, 500)
    got, n = gpu_select(s, p, 500, capacity=100)
    assert n == 500 and np.array_equal(got[:100], ref[:100])


@pytest.mark.parametrize("name", ["tiny", "tiny-K32", "t16k", "t32k-K100", "t32k-K500",
                                  "t32k-K2000", "t128k", "t32k-dense"])
def test_select_workload_shapes(name):
    """Random scores at each workload's real shape (its mask and K)."""
    w = workloads.get(name)
    rng = np.random.default_rng(w.seed + 7)
    s = rng.standard_normal(w.T).astype(np.float32)
    p = workloads.prunable_mask(w)
    ref = oracle.topk_select(s, p, w.K)
    assert len(ref) == w.n_kept
    got, n = gpu_select(s, p, w.K)
    assert n == w.n_kept and np.array_equal(got[:n], ref)
    report("select_shape_" + name, N=n, bit_exact=True)


def test_select_determinism():
    rng = np.random.default_rng(10)
    T = 131072
    s = _scores(rng, T, "ties")
    p = np.ones(T, np.uint8)
    a, na = gpu_select(s, p, 2000)
    b, nb = gpu_select(s, p, 2000)
    assert na == nb and np.array_equal(a[:na], b[:nb])


_TIMEOUT_CHILD = r"""
import torch
import learned_token_pruning_gate_amd as tg
dev = torch.device("cuda", 0)
g = torch.Generator(device=dev).manual_seed(3)
for T, K, grid in ((40000, 1000, True), (1000, 100, False)):
    s = torch.randn(T, generator=g, device=dev)
    p = torch.ones(T, dtype=torch.uint8, device=dev)
    ws = torch.zeros(tg.tg_topk_workspace_size(T), dtype=torch.uint8, device=dev)
    kept = torch.full((T,), -5, dtype=torch.int32, device=dev)
    kept, n = tg.tg_topk_select(s, p, K, kept_idx=kept, workspace=ws)
    torch.cuda.synchronize()
    want = -1 if grid else K
    assert int(n.item()) == want, (T, int(n.item()), want)
    assert int(ws.count_nonzero().item()) == 0, "workspace not left zeroed"
print("timeout path ok")
"""


def test_select_grid_timeout_reported():
    """The grid path's barrier waits are bounded.  Forced to give up (with
    TG_TEST_SELECT_TIMEOUT=1 every barrier waits for one arrival more than
    there are workgroups, with a short poll bound), the call still ends,
    reports n_kept = -1 and leaves the workspace zeroed; a short prompt (one
    workgroup, no barrier) in the same process is unaffected.  Runs in a
    child process, since the library reads the variable once."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, TG_TEST_SELECT_TIMEOUT="1",
               PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", _TIMEOUT_CHILD], env=env, cwd=root,
                       capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "timeout path ok" in r.stdout
