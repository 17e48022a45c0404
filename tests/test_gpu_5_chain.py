"""End-to-end: gate -> select -> gather -> bias attention on the GPU, each
stage checked against the oracle on every workload (tests/chain_oracle.py
states the rules and tolerances).

The attention runs through tg_bias_attn_fwd_ws with the workspace that
tg_bias_attn_workspace_size gives for the shape (none when it runs unsplit),
which is the launch that the captured chain and the benchmark time; the
"unsplit" cases take the same pass through tg_bias_attn_fwd."""
import numpy as np
import pytest
import torch

import learned_token_pruning_gate_amd as tg
import workloads
from chain_oracle import check_chain
from gpu_util import as_f64, bf16_bits, to_dev

pytestmark = pytest.mark.gpu

ALL = ["tiny", "tiny-K32", "t16k", "t32k-K100", "t32k-K500", "t32k-K2000", "t32k-scale",
       "t128k", "t32k-dense", "t16k-d256"]


def run_chain(w, g, a, planted=None, entry="ws"):
    dt = w.dtype
    resid = to_dev(g.resid, dt)
    prunable = to_dev(g.prunable)
    scores = tg.tg_gate_score(resid, prunable, to_dev(g.w1, dt), to_dev(g.w2), b2=g.b2,
                              rms_weight=to_dev(g.gamma), b1=to_dev(g.b1), eps=g.eps)
    if planted is not None:                 # the planted block overwrites real scores
        p0, vals = planted
        scores[p0:p0 + 64] = to_dev(vals)
    kept, n_kept = tg.tg_topk_select(scores, prunable, w.K)
    N = w.n_kept
    resid_kept, pos_kept, score_kept = tg.tg_compact_gather(resid, scores, kept, N)
    key_score = to_dev(a.drawn_scores) if w.drawn_key_scores else score_kept
    torch.cuda.synchronize()
    pos_host = pos_kept.cpu().numpy()
    q_scale = None
    if w.q_scale_recipe == "pos_rank":
        q_scale = to_dev(workloads.q_scale_pos_rank(pos_host))
    q, k, v, gain = to_dev(a.q, dt), to_dev(a.k, dt), to_dev(a.v, dt), to_dev(a.gain)
    split = False
    if entry == "ws":
        nb = tg.tg_bias_attn_workspace_size(N, w.Hq, w.Hkv, w.D, True, q.dtype)
        ws = torch.empty(nb, dtype=torch.uint8, device=q.device) if nb else None
        split = ws is not None
        out, lse = tg.tg_bias_attn_fwd_ws(q, k, v, key_score, gain, ws, q_scale)
    else:
        out, lse = tg.tg_bias_attn_fwd(q, k, v, key_score, gain, q_scale)
    torch.cuda.synchronize()
    rk = bf16_bits(resid_kept) if dt == "bf16" else resid_kept.cpu().numpy()
    return dict(scores=scores.cpu().numpy(), n_kept=int(n_kept.item()),
                kept=kept.cpu().numpy()[:N], resid_kept=rk, pos=pos_host,
                score_kept=score_kept.cpu().numpy(), key_score=key_score.cpu().numpy(),
                q_scale=None if q_scale is None else q_scale.cpu().numpy(),
                out=as_f64(out), lse=lse.cpu().numpy(), split=split)


CASES = [(n, "ws") for n in ALL] + [("t16k", "unsplit"), ("t16k-d256", "unsplit")]


@pytest.mark.parametrize("name,entry", CASES)
def test_chain(name, entry):
    w = workloads.get(name)
    g, a = workloads.generate(w)
    planted = workloads.planted_block(w, g) if w.planted_block else None
    r = run_chain(w, g, a, planted, entry)
    if name in ("t16k", "t16k-d256") and entry == "ws":
        assert r["split"], "the 16k prompt's attention is expected to take the split"
    check_chain(w, g.resid, g.prunable, g, a, r, "chain_%s_%s" % (name, entry), planted)
