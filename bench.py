"""Benchmark of the token-gated prefill path on one MI355X.

One step = the whole path over one prompt: gate scoring of T tokens, top-K
selection + compaction, gather of the kept rows, and token-gated attention
over the N kept tokens (one gate plus one upper attention layer).  Inputs
are seeded synthetic tensors of the workload's shapes, resident in HBM
before the timed region; outputs are preallocated.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload t32k-dense]

The default workload is the dense 32k prompt (T = 32768, every token kept,
16/8 heads, head dim 128): the compute-bound configuration on which the
attention's share of the MFMA peak is quoted.  The same run also times the
other bf16 prompts (16k, 32k with K = 100/500/2000, 128k) and reports each
one's step time and per-stage times under "other_workloads" (--no-others
skips them).

By default each timed step is one replay of the four calls captured as a HIP
graph (tg_chain_create); --mode eager launches them one by one.  Per-stage
times come from HIP events around each call of an eager run of the same
steps.  The attention gets a split-key workspace (tg_bias_attn_fwd_ws) when
its shape uses one; --attn-split off runs tg_bias_attn_fwd.

Prints one JSON line: tokens/s for the whole step, per-stage event timings,
the roofline of the dominant kernel, and the CPU oracle timed on a bounded
sample of the same workload (a reported baseline, not the target).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "token-gated prefill tokens/s (score+topK+gather+bias attn); attn TFLOP/s vs peak"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 vector

KERNEL_SOURCES = {
    "gate": "gate_score.hip", "select": "topk_select.hip",
    "gather": "compact_gather.hip", "attn": "bias_attn.hip",
}


def source_sha(stage: str) -> str:
    p = os.path.join(ROOT, "learned_token_pruning_gate_amd", "csrc", KERNEL_SOURCES[stage])
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def algorithmic(w, N, kv_layers=0):
    """Per-launch algorithmic bytes and flops of each stage (what the method
    must move or compute, not what a kernel happens to touch)."""
    b = 2 if w.dtype == "bf16" else 4
    nP, T, d, h = w.n_prunable, w.T, w.d, w.h
    D, Hq, Hkv = w.D, w.Hq, w.Hkv
    return {
        "kv": dict(bytes=2 * 2 * kv_layers * N * Hkv * D * b + 4 * N, flops=0),
        "gate": dict(bytes=nP * d * b + T + 4 * T + h * d * b, flops=2 * nP * d * h),
        "select": dict(bytes=4 * nP + T + 4 * N, flops=0),
        "gather": dict(bytes=2 * N * d * b + 16 * N, flops=0),
        "attn": dict(bytes=(2 * Hq + 2 * Hkv) * N * D * b + 8 * N,
                     flops=2 * D * Hq * N * (N + 1)),
    }


def load_traffic(workload, stage):
    """HBM bytes per launch measured by rocprofv3 --pmc (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy-kernel calibration) for this workload and
    stage, if recorded for the current kernel source; None otherwise."""
    p = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(workload, {}).get(stage)
    if not rec or rec.get("source_sha") != source_sha(stage):
        return None
    return rec.get("bytes_per_launch")


def host_cpu():
    """(CPU model, OMP_NUM_THREADS as set or None) of this host."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.environ.get("OMP_NUM_THREADS")


def cpu_baseline(w, g, a, N, kept, scores_gpu, key_score):
    """The oracle, as it stands, on a bounded sample of the same workload,
    scaled to tokens/s of the whole step."""
    import numpy as np

    import oracle
    import workloads

    T = w.T
    pr = np.nonzero(g.prunable)[0]
    # gate: every prunable row up to 16384 of them (spread evenly beyond)
    n_gate = min(16384, len(pr))
    gate_rows = pr[np.linspace(0, len(pr) - 1, n_gate).astype(np.int64)]
    t0 = time.perf_counter()
    oracle.gate_score(workloads.as_f64(g.resid[gate_rows], w.dtype), g.prunable[gate_rows],
                      workloads.as_f64(g.w1, w.dtype), g.w2, b2=g.b2, gamma=g.gamma, b1=g.b1,
                      eps=g.eps)
    t_gate_sample = time.perf_counter() - t0
    t_gate = t_gate_sample * len(pr) / n_gate
    t0 = time.perf_counter()
    oracle.topk_select(scores_gpu, g.prunable, w.K)
    t_sel = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.compact_gather(g.resid, scores_gpu, kept)
    t_gat = time.perf_counter() - t0
    # attention: query rows spread over [0, N); a 64-row probe sets how many
    # rows fill about one second, capped at N (every row)
    q64, k64, v64 = (workloads.as_f64(x, w.dtype) for x in (a.q, a.k, a.v))

    def attn_rows(n):
        rows = np.unique(np.linspace(0, N - 1, n).astype(np.int64))
        t0 = time.perf_counter()
        oracle.bias_attn(q64, k64, v64, key_score, a.gain, rows=rows)
        return rows, time.perf_counter() - t0

    rows, t_att_sample = attn_rows(min(64, N))
    per_work = t_att_sample / float(np.sum(rows + 1))
    want = int(1.0 / max(per_work, 1e-12) / max(1.0, (N + 1) / 2.0))
    if want > len(rows):
        rows, t_att_sample = attn_rows(min(N, want))
    n_rows = len(rows)
    # causal work of row r is proportional to r + 1
    t_att = t_att_sample * (N * (N + 1) / 2) / float(np.sum(rows + 1))
    total = t_gate + t_sel + t_gat + t_att
    sample_s = t_gate_sample + t_sel + t_gat + t_att_sample
    threads = oracle.num_threads()
    model, omp = host_cpu()
    return {
        "value": T / total, "unit": "tokens/s", "cores": threads,
        "kind": "oracle", "cpu_model": model, "omp_num_threads": omp,
        "nproc": os.cpu_count(),
        "sample": ("fp64 C oracle on this host: gate on %d of %d prunable rows, full top-K "
                   "and gather, attention on %d of %d query rows (all heads); each stage "
                   "scaled to the full step by its row count (attention by causal work); "
                   "%.1f s wall on %d threads (about %.0f s of CPU work)"
                   % (n_gate, len(pr), n_rows, N, sample_s, threads, sample_s * threads)),
        "stage_seconds_est": {"gate": t_gate, "select": t_sel, "gather": t_gat,
                              "attn": t_att},
    }




OTHER_WORKLOADS = ("t16k", "t32k-K100", "t32k-K500", "t32k-K2000", "t128k")


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="t32k-dense")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the step and stage times of the other bf16 workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", action="store_true",
                    help="also time steps with the last-level cache flushed before each")
    ap.add_argument("--rms-weight", action="store_true",
                    help="pass the workload's RMSNorm weight explicitly; by default it is "
                         "NULL, which the ABI defines as all ones (the workload's weight)")
    ap.add_argument("--w1", choices=["packed", "rowmajor"], default="packed",
                    help="gate W1 layout: packed once before timing (tg_gate_pack_w1, the "
                         "weight-load step) or row-major [h, d]; packed needs bf16 and a "
                         "unit RMSNorm weight")
    ap.add_argument("--kv-layers", type=int, default=0,
                    help="also gather this many lower layers' K/V cache [L, T, Hkv, D] to "
                         "the kept tokens (tg_kv_gather) on a second stream beside the "
                         "attention; 0 (default) times the path without it")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="how the timed steps are launched: one replay of the chain "
                         "captured as a HIP graph (tg_chain_create, the pages' serving "
                         "recipe) per step, or the four calls launched one by one; "
                         "the per-stage events always come from an eager run")
    ap.add_argument("--attn-split", choices=["on", "off"], default="on",
                    help="give the attention a split-key workspace "
                         "(tg_bias_attn_fwd_ws: long rows' keys cut into chunks on separate "
                         "workgroups, then merged) when the shape uses one; off runs "
                         "tg_bias_attn_fwd")
    ap.add_argument("--no-attn-bwd", action="store_true",
                    help="skip the separate timing of the attention backward "
                         "(tg_bias_attn_bwd on the step's forward outputs; reported beside "
                         "the step, not part of it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy, the reference kernel that "
                         "scales FETCH_SIZE / WRITE_SIZE counter readings to bytes")
    return ap.parse_args(argv)


def run_workload(w, args, full):
    """Times the path on one workload.  full=False: the graph-replayed step
    and the per-stage events only (the other workloads' lines); full=True:
    also the bias self-check, the backward, the cold-cache stages and the
    CPU oracle baseline."""
    import numpy as np
    import torch

    import learned_token_pruning_gate_amd as tg
    import workloads

    print("bench: workload %s" % w.name, file=sys.stderr, flush=True)
    g, a = workloads.generate(w)
    N = w.n_kept
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(x, dt=None):
        x = np.ascontiguousarray(x)
        if dt == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    dt = w.dtype
    resid, prunable = up(g.resid, dt), up(g.prunable)
    w1, w2, b1, gamma = up(g.w1, dt), up(g.w2), up(g.b1), up(g.gamma)
    q, k, v, gain = up(a.q, dt), up(a.k, dt), up(a.v, dt), up(a.gain)
    scores = torch.empty(w.T, dtype=torch.float32, device=dev)
    kept = torch.empty(w.T, dtype=torch.int32, device=dev)
    n_kept = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.zeros(tg.tg_topk_workspace_size(w.T), dtype=torch.uint8, device=dev)
    resid_kept = torch.empty((N, w.d), dtype=resid.dtype, device=dev)
    pos_kept = torch.empty(N, dtype=torch.int32, device=dev)
    score_kept = torch.empty(N, dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.Hq, N), dtype=torch.float32, device=dev)
    drawn = up(a.drawn_scores) if w.drawn_key_scores else None
    q_scale = None

    # Prepared C calls: argument marshalling done once, outside the timed loop.
    lib = tg.load()
    use_packed = (args.w1 == "packed" and dt == "bf16" and not args.rms_weight and
                  tg.tg_gate_w1_packed_bytes(torch.bfloat16, w.h, w.d) > 0)
    if use_packed:   # weight-load step, once, before any timing
        w1 = tg.tg_gate_pack_w1(w1)
    if w.q_scale_recipe == "pos_rank":
        # the per-query scale is an input of the attention call: derive it
        # from this prompt's kept set (one untimed pass of gate + select)
        sc = (tg.tg_gate_score_packed(resid, prunable, w1, w2, b2=g.b2, b1=b1, eps=g.eps)
              if use_packed else
              tg.tg_gate_score(resid, prunable, w1, w2, b2=g.b2, b1=b1, eps=g.eps,
                               rms_weight=gamma if args.rms_weight else None))
        kidx, _ = tg.tg_topk_select(sc, prunable, w.K)
        torch.cuda.synchronize()
        q_scale = up(workloads.q_scale_pos_rank(kidx.cpu().numpy()[:N]))
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    dtc = tg.TG_DTYPE_BF16 if dt == "bf16" else tg.TG_DTYPE_F32
    key_ptr = P(drawn) if drawn is not None else P(score_kept)
    F = ctypes.c_float
    gate_args = (dtc, w.T, w.d, w.h, P(resid), resid.stride(0), P(prunable),
                 P(gamma) if args.rms_weight else None,
                 F(g.eps), P(w1), P(b1), P(w2), F(g.b2), P(scores), sp)
    sel_args = (w.T, P(scores), P(prunable), w.K, P(kept), kept.numel(), P(n_kept), P(ws),
                ws.numel(), sp)
    gat_args = (dtc, w.T, N, w.d, P(resid), resid.stride(0), P(scores), P(kept),
                P(resid_kept), resid_kept.stride(0), P(pos_kept), P(score_kept), sp)
    att_ws_bytes = (tg.tg_bias_attn_workspace_size(N, w.Hq, w.Hkv, w.D, True, q.dtype)
                    if args.attn_split == "on" else 0)
    att_ws = (torch.empty(att_ws_bytes, dtype=torch.uint8, device=dev) if att_ws_bytes
              else None)
    att_args = (dtc, N, w.Hq, w.Hkv, w.D, P(q), P(k), P(v), key_ptr, P(gain), P(q_scale),
                F(0.0), 1, P(out), P(lse), P(att_ws), att_ws_bytes, sp)

    def check(st, name):
        if st != 0:
            raise RuntimeError("%s failed: %s %s" % (name, tg.tg_status_str(st),
                                                     tg.tg_last_error()))

    stages = ["gate", "select", "gather", "attn"]
    kvl = args.kv_layers if full else 0
    if kvl > 0:
        kv_k = torch.randn((kvl, w.T, w.Hkv, w.D), device=dev).to(q.dtype)
        kv_v = torch.randn((kvl, w.T, w.Hkv, w.D), device=dev).to(q.dtype)
        kv_ko = torch.empty((kvl, N, w.Hkv, w.D), dtype=q.dtype, device=dev)
        kv_vo = torch.empty_like(kv_ko)
        kv_args = (dtc, kvl, w.T, N, w.Hkv, w.D, P(kv_k), P(kv_v), P(kept), P(kv_ko), P(kv_vo))
        side = torch.cuda.Stream(device=dev)      # default priority
        side_p = ctypes.c_void_p(side.cuda_stream)
        fork_ev, join_ev = torch.cuda.Event(), torch.cuda.Event()

    gate_fn = lib.tg_gate_score_packed if use_packed else lib.tg_gate_score

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        check(gate_fn(*gate_args), "tg_gate_score")
        if ev is not None:
            ev[1].record(stream)
        check(lib.tg_topk_select(*sel_args), "tg_topk_select")
        if ev is not None:
            ev[2].record(stream)
        check(lib.tg_compact_gather(*gat_args), "tg_compact_gather")
        if ev is not None:
            ev[3].record(stream)
        if kvl > 0:   # lower layers' KV gather on the side stream, beside the attention
            fork_ev.record(stream)
            side.wait_event(fork_ev)
            if ev is not None:
                ev[5].record(side)
            check(lib.tg_kv_gather(*kv_args, side_p), "tg_kv_gather")
            if ev is not None:
                ev[6].record(side)
            join_ev.record(side)
        check(lib.tg_bias_attn_fwd_ws(*att_args), "tg_bias_attn_fwd_ws")
        if ev is not None:
            ev[4].record(stream)
        if kvl > 0:
            stream.wait_event(join_ev)

    if full and args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    per_stage_ms = {s: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in events]))
                    for j, s in enumerate(stages)}
    if kvl > 0:
        per_stage_ms["kv"] = float(np.mean([e[5].elapsed_time(e[6]) for e in events]))
    eager_ms = elapsed * 1e3 / args.steps

    graph_ms = None
    if args.mode == "graph":
        chain = tg.tg_chain_create(
            resid=resid, prunable=prunable, w1=w1, w2=w2, b1=b1, eps=g.eps, b2=g.b2,
            w1_packed=use_packed, rms_weight=gamma if args.rms_weight else None,
            scores=scores, K=w.K, kept_idx=kept, n_kept=n_kept, workspace=ws, N=N,
            resid_kept=resid_kept, pos_kept=pos_kept, score_kept=score_kept, q=q, k=k, v=v,
            attn_key_score=drawn if drawn is not None else score_kept, gain=gain,
            q_scale=q_scale, out=out, lse=lse, attn_workspace=att_ws,
            **(dict(kv_k_cache=kv_k, kv_v_cache=kv_v, kv_k_kept=kv_ko, kv_v_kept=kv_vo)
               if kvl > 0 else {}))
        for _ in range(max(args.warmup, 1)):
            chain.launch(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            chain.launch(stream)
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        chain.close()
    ms_per_step = graph_ms if graph_ms is not None else eager_ms
    value = w.T / (ms_per_step * 1e-3)

    alg = algorithmic(w, N, kvl)
    stage_info = {}
    for s in stages + (["kv"] if kvl > 0 else []):
        t = per_stage_ms[s] * 1e-3
        info = {"ms": per_stage_ms[s], "bytes": alg[s]["bytes"],
                "GB_s": alg[s]["bytes"] / t / 1e9,
                "hbm_frac": alg[s]["bytes"] / t / 1e9 / PEAK_HBM_GBS}
        if alg[s]["flops"]:
            peak = PEAK_BF16_TFLOPS if dt == "bf16" else PEAK_F32_TFLOPS
            info["TFLOP_s"] = alg[s]["flops"] / t / 1e12
            info["mfma_frac"] = info["TFLOP_s"] / peak
        stage_info[s] = info
    dominant = max(stages, key=lambda s: per_stage_ms[s])
    di = stage_info[dominant]
    if dominant == "attn" or (dominant == "gate" and di.get("mfma_frac", 0) > di["hbm_frac"]):
        roof = {"bound": "mfma", "achieved": di["TFLOP_s"],
                "peak": PEAK_BF16_TFLOPS if dt == "bf16" else PEAK_F32_TFLOPS,
                "unit": "TFLOP/s", "frac": di["mfma_frac"]}
    else:
        roof = {"bound": "hbm", "achieved": di["GB_s"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": di["hbm_frac"]}
    roof["kernel"] = dominant
    roof["traffic"] = load_traffic(w.name, dominant)

    config = {"workload": w.name, "T": w.T, "d": w.d, "h": w.h,
              "n_prunable": w.n_prunable, "K": w.K, "N_kept": N, "Hq": w.Hq,
              "Hkv": w.Hkv, "D": w.D, "causal": True, "global_batch": 1,
              "gate_w1": "packed" if use_packed else "row-major",
              "kv_layers": kvl, "attn_split": att_ws is not None,
              "parallelism": "single-gpu"}
    if not full:
        return {"config": config, "ms_per_step": ms_per_step, "tokens_per_s": value,
                "eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms,
                "stage_ms": per_stage_ms,
                "attn_frac_of_peak": stage_info["attn"].get("mfma_frac"),
                "gate_hbm_frac": stage_info["gate"]["hbm_frac"],
                "gather_hbm_frac": stage_info["gather"]["hbm_frac"]}

    # cost of the bias path: the attention call alone, with the step's key-score
    # bias and per-query scale, against the same call with both left out (a
    # plain causal GQA flash attention); the pages put the biased call at
    # 1.0-1.1x the plain one
    def time_attn(a_args, reps):
        for _ in range(2):
            check(lib.tg_bias_attn_fwd_ws(*a_args), "tg_bias_attn_fwd_ws")
        b0, b1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record(stream)
        for _ in range(reps):
            check(lib.tg_bias_attn_fwd_ws(*a_args), "tg_bias_attn_fwd_ws")
        b1_.record(stream)
        torch.cuda.synchronize()
        return b0.elapsed_time(b1_) * 1e3 / reps

    plain_args = (dtc, N, w.Hq, w.Hkv, w.D, P(q), P(k), P(v), None, None, None,
                  F(0.0), 1, P(out), P(lse), P(att_ws), att_ws_bytes, sp)
    reps = max(min(args.steps, 20), 5)
    with_us, plain_us = time_attn(att_args, reps), time_attn(plain_args, reps)
    bias_cost = {"with_bias_us": with_us, "plain_us": plain_us, "ratio": with_us / plain_us,
                 "calls": reps, "pages_ratio": "1.0-1.1"}

    # attention backward (the gate's training path), timed on its own: not
    # part of the prefill step
    bwd_info = None
    if dt == "bf16" and w.D in (64, 128) and not args.no_attn_bwd:
        gen = torch.Generator(device=dev).manual_seed(17)
        dout = torch.randn(q.shape, generator=gen, device=dev).to(q.dtype)
        dq_, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dscore_ = torch.empty(N, dtype=torch.float32, device=dev)
        dgain_ = torch.empty(w.Hq, dtype=torch.float32, device=dev)
        bws = torch.empty(max(tg.tg_bias_attn_bwd_workspace_size(N, w.Hq, w.Hkv, w.D), 16),
                          dtype=torch.uint8, device=dev)
        check(lib.tg_bias_attn_fwd_ws(*att_args), "tg_bias_attn_fwd_ws")   # out, lse
        bwd_args = (dtc, N, w.Hq, w.Hkv, w.D, P(q), P(k), P(v), key_ptr, P(gain), P(q_scale),
                    F(0.0), 1, P(out), P(dout), P(lse), P(dq_), P(dk_), P(dv_), P(dscore_),
                    P(dgain_), P(bws), bws.numel(), sp)
        check(lib.tg_bias_attn_bwd(*bwd_args), "tg_bias_attn_bwd")
        bwd_calls = max(min(args.steps, 10), 3)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(bwd_calls):
            check(lib.tg_bias_attn_bwd(*bwd_args), "tg_bias_attn_bwd")
        e1.record(stream)
        torch.cuda.synchronize()
        bwd_ms = e0.elapsed_time(e1) / bwd_calls
        bwd_flops = 5 * w.D * w.Hq * N * (N + 1)   # S, dP, dV, dK, dQ products (causal)
        bwd_info = {"ms": bwd_ms, "flops": bwd_flops,
                    "TFLOP_s": bwd_flops / (bwd_ms * 1e-3) / 1e12,
                    "mfma_frac": bwd_flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                    "calls": bwd_calls}
        del dout, dq_, dk_, dv_, bws

    cold = None
    if args.cold:
        flush = torch.empty(1 << 29, dtype=torch.uint8, device=dev)  # 512 MiB > MALL
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(10)]
        for e in ev:
            flush.fill_(1)
            step(e)
        torch.cuda.synchronize()
        cold = {s: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev]))
                for j, s in enumerate(stages)}
        del flush

    result = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": config,
        "mode": args.mode,
        "eager_ms_per_step": eager_ms,
        "graph_ms_per_step": graph_ms,
        "attn_tflops": stage_info["attn"].get("TFLOP_s"),
        "attn_frac_of_peak": stage_info["attn"].get("mfma_frac"),
        "roofline": roof,
        "stages": stage_info,
        "attn_bwd": bwd_info,
        "attn_bias_cost": bias_cost,
    }
    if cold:
        result["cold_stage_ms"] = cold

    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle) on a sample of %s" % w.name, file=sys.stderr,
              flush=True)
        kept_host = kept.cpu().numpy()[:N]
        key_host = (drawn if drawn is not None else score_kept).cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(w, g, a, N, kept_host, scores.cpu().numpy(),
                                              key_host)
    return result


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py: only one GPU is measured (the path runs on one MI355X; "
              "sharding across GPUs is designed but not built); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads

    result = run_workload(workloads.get(args.workload), args, full=True)
    if not args.no_others:
        others = {}
        for name in OTHER_WORKLOADS:
            if name == args.workload:
                continue
            others[name] = run_workload(workloads.get(name), args, full=False)
            torch.cuda.empty_cache()
        result["other_workloads"] = others
    print(json.dumps(result))


if __name__ == "__main__":
    main()
