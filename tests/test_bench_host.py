"""bench.py host checks (CPU only; nothing touches a GPU).

* more than one GPU is refused with a message and exit status 2, before
  torch is imported;
* the per-launch algorithmic bytes and flops that the roofline divides by
  its measured times, at the 16k-token prompt: the figures stated beside
  each kernel's bound (gate 66.1 MB, gather 20.6 MB, attention 30.9 MB and
  25.9 GFLOP over the 2512 kept tokens).
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "only one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_algorithmic_units_at_16k():
    import bench
    import workloads

    w = workloads.get("t16k")
    N = w.n_kept
    assert N == 2512          # 2000 kept of 15872 prunable, plus 512 never pruned
    a = bench.algorithmic(w, N)
    # gate: every prunable residual row once (bf16), W1 once, mask and scores
    assert abs(a["gate"]["bytes"] / 1e6 - 66.14) < 0.01
    # and its products: one d x h product per prunable row
    assert a["gate"]["flops"] == 2 * 15872 * 2048 * 256
    # gather: each kept row read and written once, plus index, position, score
    assert abs(a["gather"]["bytes"] / 1e6 - 20.62) < 0.01
    # attention: Q, K, V read and O written once, plus the key bias
    assert abs(a["attn"]["bytes"] / 1e6 - 30.89) < 0.01
    # causal: query i sees i + 1 keys, in both the logit and the value product
    assert abs(a["attn"]["flops"] / 1e9 - 25.857) < 0.001
    # select and gather do no arithmetic the roofline counts
    assert a["select"]["flops"] == 0 and a["gather"]["flops"] == 0
