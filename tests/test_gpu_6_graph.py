"""The four calls captured as one HIP graph (tg_chain_create / launch): every
replay must reproduce the eager chain bit for bit, also after the inputs are
refilled in place and with eager work and synchronisation between replays,
and the replays' outputs, before and after the refill, must match the oracle
(tests/chain_oracle.py).  (TokenGate pages: ai.info summary "Key
Contributions" item 4, the graph-captured serving recipe.)"""
import numpy as np
import pytest
import torch

import learned_token_pruning_gate_amd as tg
import oracle
import workloads
from chain_oracle import check_chain
from dataclasses import replace
from gpu_util import as_f64, bf16_bits, report, to_dev

pytestmark = pytest.mark.gpu


def make_case(w, packed, kv_layers=0, split=False, g=None, a=None):
    if g is None:
        g, a = workloads.generate(w)
    dt = w.dtype
    c = dict(resid=to_dev(g.resid, dt), prunable=to_dev(g.prunable), w2=to_dev(g.w2),
             b1=to_dev(g.b1), q=to_dev(a.q, dt), k=to_dev(a.k, dt), v=to_dev(a.v, dt),
             gain=to_dev(a.gain))
    w1 = to_dev(g.w1, dt)
    c["w1"] = tg.tg_gate_pack_w1(w1) if packed else w1
    N, dev = w.n_kept, c["resid"].device
    c.update(scores=torch.empty(w.T, dtype=torch.float32, device=dev),
             kept_idx=torch.empty(w.T, dtype=torch.int32, device=dev),
             n_kept=torch.empty(1, dtype=torch.int32, device=dev),
             workspace=torch.zeros(tg.tg_topk_workspace_size(w.T), dtype=torch.uint8, device=dev),
             resid_kept=torch.empty((N, w.d), dtype=c["resid"].dtype, device=dev),
             pos_kept=torch.empty(N, dtype=torch.int32, device=dev),
             score_kept=torch.empty(N, dtype=torch.float32, device=dev),
             out=torch.empty_like(c["q"]),
             lse=torch.empty((w.Hq, N), dtype=torch.float32, device=dev))
    if split:
        nb = tg.tg_bias_attn_workspace_size(N, w.Hq, w.Hkv, w.D)
        assert nb > 0
        c["attn_workspace"] = torch.empty(nb, dtype=torch.uint8, device=dev)
    if kv_layers:
        gen = torch.Generator(device=dev).manual_seed(21)
        for n in ("kv_k_cache", "kv_v_cache"):
            c[n] = torch.randn((kv_layers, w.T, w.Hkv, w.D), generator=gen, device=dev).to(
                c["q"].dtype)
        c["kv_k_kept"] = torch.empty((kv_layers, N, w.Hkv, w.D), dtype=c["q"].dtype, device=dev)
        c["kv_v_kept"] = torch.empty_like(c["kv_k_kept"])
    return c


OUTS = ("scores", "kept_idx", "n_kept", "resid_kept", "pos_kept", "score_kept", "out", "lse",
        "kv_k_kept", "kv_v_kept")


def outs(c):
    return [n for n in OUTS if n in c]


def eager(c, w, packed):
    if packed:
        tg.tg_gate_score_packed(c["resid"], c["prunable"], c["w1"], c["w2"], b1=c["b1"],
                                eps=w.eps, scores=c["scores"])
    else:
        tg.tg_gate_score(c["resid"], c["prunable"], c["w1"], c["w2"], b1=c["b1"], eps=w.eps,
                         scores=c["scores"])
    tg.tg_topk_select(c["scores"], c["prunable"], w.K, kept_idx=c["kept_idx"],
                      n_kept=c["n_kept"], workspace=c["workspace"])
    tg.tg_compact_gather(c["resid"], c["scores"], c["kept_idx"], w.n_kept,
                         resid_kept=c["resid_kept"], pos_kept=c["pos_kept"],
                         score_kept=c["score_kept"])
    if "kv_k_cache" in c:
        tg.tg_kv_gather(c["kept_idx"], w.n_kept, c["kv_k_cache"], c["kv_v_cache"],
                        c["kv_k_kept"], c["kv_v_kept"])
    if "attn_workspace" in c:
        tg.tg_bias_attn_fwd_ws(c["q"], c["k"], c["v"], c["score_kept"], c["gain"],
                               c["attn_workspace"], out=c["out"], lse=c["lse"])
    else:
        tg.tg_bias_attn_fwd(c["q"], c["k"], c["v"], c["score_kept"], c["gain"], out=c["out"],
                            lse=c["lse"])
    torch.cuda.synchronize()
    return {n: c[n].clone() for n in outs(c)}


def clobber(c):
    for n in outs(c):
        if c[n].dtype in (torch.float32, torch.bfloat16):
            c[n].fill_(float("nan"))
        else:
            c[n].fill_(-7)


def same(c, ref, what):
    for n in outs(c):
        a, b = c[n], ref[n]
        if n == "kept_idx":   # entries past the kept count are unspecified
            k = int(ref["n_kept"].item())
            a, b = a[:k], b[:k]
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), (what, n)


def host(t, dt):
    return bf16_bits(t) if dt == "bf16" else t.cpu().numpy()


def replay_outputs(c, w):
    """The chain's outputs in the form check_chain takes."""
    N = w.n_kept
    return dict(scores=c["scores"].cpu().numpy(), n_kept=int(c["n_kept"].item()),
                kept=c["kept_idx"].cpu().numpy()[:N], resid_kept=host(c["resid_kept"], w.dtype),
                pos=c["pos_kept"].cpu().numpy(), score_kept=c["score_kept"].cpu().numpy(),
                key_score=c["score_kept"].cpu().numpy(), q_scale=None, out=as_f64(c["out"]),
                lse=c["lse"].cpu().numpy())


CASES = [
    ("tiny", False, 0, False),
    ("t16k", True, 0, True),     # the benchmark's chain: packed W1, split attention
    ("t16k", True, 0, False),
    ("t16k", False, 0, False),
    ("t16k", True, 2, False),    # with the lower layers' KV gather on a forked stream
    ("t16k-d256", True, 2, True),   # head dim 256: the split-key attention and its workspace
    ("multi", True, 0, False),   # T > 32768: the multi-workgroup top-K and its workspace
]


@pytest.mark.parametrize("name,packed,kv_layers,split", CASES)
def test_graph_replays_match_eager(name, packed, kv_layers, split):
    if name == "multi":
        w = replace(workloads.get("t16k"), name="graph-40k", seed=11, T=40000, d=512, h=128,
                    p_lo=100, p_hi=39900, K=700)
    else:
        w = workloads.get(name)
    g, a = workloads.generate(w)
    c = make_case(w, packed, kv_layers, split, g, a)
    ref = eager(c, w, packed)
    kv = {n: c[n] for n in ("kv_k_cache", "kv_v_cache", "kv_k_kept", "kv_v_kept") if n in c}
    chain = tg.tg_chain_create(
        resid=c["resid"], prunable=c["prunable"], w1=c["w1"], w2=c["w2"], b1=c["b1"],
        eps=w.eps, w1_packed=packed, scores=c["scores"], K=w.K, kept_idx=c["kept_idx"],
        n_kept=c["n_kept"], workspace=c["workspace"], N=w.n_kept, resid_kept=c["resid_kept"],
        pos_kept=c["pos_kept"], score_kept=c["score_kept"], q=c["q"], k=c["k"], v=c["v"],
        attn_key_score=c["score_kept"], gain=c["gain"], out=c["out"], lse=c["lse"],
        attn_workspace=c.get("attn_workspace"), **kv)
    for rep in range(3):
        clobber(c)                     # eager work between replays
        torch.cuda.synchronize()
        chain.launch()
        torch.cuda.synchronize()
        same(c, ref, "%s replay %d" % (name, rep))
        if rep == 0:
            check_chain(w, g.resid, g.prunable, g, a, replay_outputs(c, w),
                        "graph_%s_p%d_kv%d_s%d" % (name, packed, kv_layers, split))
            kept_host = c["kept_idx"].cpu().numpy()[:w.n_kept]
            for src, dst in (("kv_k_cache", "kv_k_kept"), ("kv_v_cache", "kv_v_kept")):
                if src in c:   # the lower layers' KV gather, bit-exact
                    want = oracle.kv_gather(host(c[src], w.dtype), kept_host)
                    assert host(c[dst], w.dtype).tobytes() == want.tobytes(), (name, dst)
    # refill the inputs in place: the graph reads the new values
    gen = torch.Generator(device=c["resid"].device).manual_seed(5)
    c["resid"].copy_(torch.randn(c["resid"].shape, generator=gen, device=c["resid"].device)
                     .to(c["resid"].dtype))
    c["q"].mul_(0.5)
    ref2 = eager(c, w, packed)
    clobber(c)
    torch.cuda.synchronize()
    chain.launch()
    chain.launch()                     # two replays in a row on one stream
    torch.cuda.synchronize()
    same(c, ref2, name + " refilled")
    check_chain(w, host(c["resid"], w.dtype), g.prunable, g, a, replay_outputs(c, w),
                "graph_%s_p%d_kv%d_s%d_refilled" % (name, packed, kv_layers, split),
                q=host(c["q"], w.dtype))
    chain.close()
    report("graph_chain_" + name, packed=packed, kv_layers=kv_layers, split=split, replays=5,
           bit_exact=True)


# ---- one graph per padded length ---------------------------------------------
# The serving recipe captures the pruned pass once per padded length (ai.info
# summary "Key Contributions" item 4): here one graph captured at a bucket's
# capacity (T_cap tokens, N_cap kept rows) is replayed on prompts of other
# lengths.  The replay reads the prompt's length from a device int32 and the
# kept count from the select's n_kept; every kept row past the count is
# padding (zero rows, position -1, score 0, attention output 0, lse -inf).
# Buffer contents past the prompt and past the kept count are garbage on
# purpose, so that reading them would show.

BUCKETS = [
    # capacity workload, prompts (T, prunable lo, hi), KV layers, split attention
    (dict(T=16384, d=2048, h=256, K=2000, Hq=16, Hkv=8, D=128, N_cap=2600, seed=31),
     [(16384, 256, 16128), (12000, 200, 11800), (16384, 256, 16128), (5000, 100, 4900)],
     1, True),
    # T > 32768: the multi-workgroup select reads the length at run time too
    (dict(T=40000, d=512, h=128, K=700, Hq=8, Hkv=4, D=64, N_cap=1000, seed=32),
     [(36000, 100, 35900), (33001, 50, 32900)], 0, False),
    # a capacity long enough for the gate's 128-row tiles
    (dict(T=66000, d=512, h=256, K=900, Hq=8, Hkv=4, D=64, N_cap=1400, seed=33),
     [(65900, 100, 65500), (40001, 300, 39801)], 0, False),
]


@pytest.mark.parametrize("cap,prompts,kv_layers,split", BUCKETS)
def test_graph_per_padded_length(cap, prompts, kv_layers, split):
    dev = torch.device("cuda", 0)
    T_cap, N_cap, d, h = cap["T"], cap["N_cap"], cap["d"], cap["h"]
    Hq, Hkv, D, K = cap["Hq"], cap["Hkv"], cap["D"], cap["K"]
    rng = np.random.default_rng(cap["seed"])
    w1_h = workloads.to_bf16_bits(rng.standard_normal((h, d)).astype(np.float32) / np.sqrt(d))
    w2_h = (rng.standard_normal(h) / np.sqrt(h)).astype(np.float32)
    gain_h = rng.uniform(0.5, 2.0, Hq).astype(np.float32)
    w1 = tg.tg_gate_pack_w1(to_dev(w1_h, "bf16"))
    bf = torch.bfloat16
    c = dict(resid=torch.empty((T_cap, d), dtype=bf, device=dev),
             prunable=torch.empty(T_cap, dtype=torch.uint8, device=dev),
             w2=to_dev(w2_h), gain=to_dev(gain_h),
             q=torch.empty((N_cap, Hq, D), dtype=bf, device=dev),
             k=torch.empty((N_cap, Hkv, D), dtype=bf, device=dev),
             v=torch.empty((N_cap, Hkv, D), dtype=bf, device=dev),
             scores=torch.empty(T_cap, dtype=torch.float32, device=dev),
             kept_idx=torch.empty(T_cap, dtype=torch.int32, device=dev),
             n_kept=torch.empty(1, dtype=torch.int32, device=dev),
             workspace=torch.zeros(tg.tg_topk_workspace_size(T_cap), dtype=torch.uint8,
                                   device=dev),
             resid_kept=torch.empty((N_cap, d), dtype=bf, device=dev),
             pos_kept=torch.empty(N_cap, dtype=torch.int32, device=dev),
             score_kept=torch.empty(N_cap, dtype=torch.float32, device=dev),
             lse=torch.empty((Hq, N_cap), dtype=torch.float32, device=dev),
             prompt_len=torch.empty(1, dtype=torch.int32, device=dev))
    c["out"] = torch.empty_like(c["q"])
    kv = {}
    if kv_layers:
        for n in ("kv_k_cache", "kv_v_cache"):
            kv[n] = torch.empty((kv_layers, T_cap, Hkv, D), dtype=bf, device=dev)
        kv["kv_k_kept"] = torch.empty((kv_layers, N_cap, Hkv, D), dtype=bf, device=dev)
        kv["kv_v_kept"] = torch.empty_like(kv["kv_k_kept"])
    attn_ws = None
    if split:
        nb = tg.tg_bias_attn_workspace_size(N_cap, Hq, Hkv, D)
        assert nb > 0, "the capacity shape is expected to take the split"
        attn_ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    chain = tg.tg_chain_create(
        resid=c["resid"], prunable=c["prunable"], w1=w1, w2=c["w2"], eps=1e-6, w1_packed=True,
        scores=c["scores"], K=K, kept_idx=c["kept_idx"], n_kept=c["n_kept"],
        workspace=c["workspace"], N=N_cap, resid_kept=c["resid_kept"], pos_kept=c["pos_kept"],
        score_kept=c["score_kept"], q=c["q"], k=c["k"], v=c["v"],
        attn_key_score=c["score_kept"], gain=c["gain"], out=c["out"], lse=c["lse"],
        attn_workspace=attn_ws, prompt_len=c["prompt_len"], **kv)
    gate = workloads.GateInputs(resid=None, prunable=None, w1=w1_h,
                                b1=np.zeros(h, np.float32), w2=w2_h, b2=0.0,
                                gamma=np.ones(d, np.float32), eps=1e-6)
    for i, (T, lo, hi) in enumerate(prompts):
        print("padded-length prompt %d: T=%d of %d" % (i, T, T_cap), flush=True)
        pr = np.zeros(T, np.uint8)
        pr[lo:hi] = 1
        N = min(K, hi - lo) + (T - (hi - lo))
        assert N <= N_cap
        resid_h = workloads.to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
        q_h = workloads.to_bf16_bits(rng.standard_normal((N, Hq, D)).astype(np.float32))
        k_h = workloads.to_bf16_bits(rng.standard_normal((N, Hkv, D)).astype(np.float32))
        v_h = workloads.to_bf16_bits(rng.standard_normal((N, Hkv, D)).astype(np.float32))
        # garbage past the prompt and past the kept count
        c["resid"].fill_(float("nan"))
        c["prunable"].fill_(1)
        for n in ("q", "k", "v"):
            c[n].normal_(0.0, 30.0)
        c["resid"][:T] = to_dev(resid_h, "bf16")
        c["prunable"][:T] = to_dev(pr)
        c["q"][:N], c["k"][:N], c["v"][:N] = to_dev(q_h, "bf16"), to_dev(k_h, "bf16"), \
            to_dev(v_h, "bf16")
        caches = {}
        for n in ("kv_k_cache", "kv_v_cache"):
            if n in kv:
                kv[n].normal_()
                caches[n] = host(kv[n], "bf16")
        for n in ("out", "lse", "resid_kept", "score_kept"):
            c[n].fill_(float("nan"))
        c["pos_kept"].fill_(-7)
        c["prompt_len"].fill_(T)
        torch.cuda.synchronize()
        chain.launch()
        torch.cuda.synchronize()

        assert int(c["n_kept"].item()) == N
        w = replace(workloads.get("t16k"), name="bucket-T%d" % T, seed=cap["seed"] + i, T=T, d=d,
                    h=h, p_lo=lo, p_hi=hi, K=K, Hq=Hq, Hkv=Hkv, D=D)
        assert w.n_kept == N
        attn = workloads.AttnInputs(q=q_h, k=k_h, v=v_h, gain=gain_h, drawn_scores=None)
        r = dict(scores=c["scores"][:T].cpu().numpy(), n_kept=N,
                 kept=c["kept_idx"][:N].cpu().numpy(),
                 resid_kept=host(c["resid_kept"][:N], "bf16"),
                 pos=c["pos_kept"][:N].cpu().numpy(), score_kept=c["score_kept"][:N].cpu().numpy(),
                 key_score=c["score_kept"][:N].cpu().numpy(), q_scale=None,
                 out=as_f64(c["out"][:N]), lse=c["lse"][:, :N].cpu().numpy())
        check_chain(w, resid_h, pr, gate, attn, r, "graph_bucket_T%d_of_%d" % (T, T_cap))
        # the padding rows past the kept count
        assert torch.all(c["resid_kept"][N:].float() == 0)
        assert torch.all(c["pos_kept"][N:] == -1)
        assert torch.all(c["score_kept"][N:] == 0)
        assert torch.all(c["out"][N:].float() == 0)
        assert torch.all(torch.isneginf(c["lse"][:, N:]))
        for src, dst in (("kv_k_cache", "kv_k_kept"), ("kv_v_cache", "kv_v_kept")):
            if src in kv:
                want = oracle.kv_gather(caches[src][:, :T], r["kept"])
                assert host(kv[dst][:, :N], "bf16").tobytes() == want.tobytes(), dst
                assert torch.all(kv[dst][:, N:].float() == 0), dst
    chain.close()
    report("graph_per_padded_length", T_cap=T_cap, N_cap=N_cap,
           prompts=[p[0] for p in prompts], split=split, kv_layers=kv_layers)
