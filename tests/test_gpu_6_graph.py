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
