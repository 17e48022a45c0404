"""Lower layers' KV cache gathered to the kept tokens (tg_kv_gather) vs the
oracle, bit for bit, also while tg_bias_attn_fwd runs on another stream.
(TokenGate pages: ai.info summary "Key Contributions" item 1 and
"Methodology in Plain English".)"""
import numpy as np
import pytest
import torch

import learned_token_pruning_gate_amd as tg
import oracle
import workloads
from gpu_util import dev, report, to_dev

pytestmark = pytest.mark.gpu


def cache_bits(rng, L, T, Hkv, D):
    return rng.integers(0, 65536, size=(L, T, Hkv, D), dtype=np.uint16)


def u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("L,T,N,Hkv,D", [(1, 7, 3, 8, 128), (2, 1000, 333, 8, 128),
                                          (3, 4097, 1, 2, 64), (2, 16384, 2512, 8, 128)])
def test_kv_gather_matches_oracle(L, T, N, Hkv, D):
    rng = np.random.default_rng(L * 7 + T + N)
    kc, vc = cache_bits(rng, L, T, Hkv, D), cache_bits(rng, L, T, Hkv, D)
    idx = np.sort(rng.choice(T, size=N, replace=False)).astype(np.int32)
    k_kept, v_kept = tg.tg_kv_gather(to_dev(idx), N, to_dev(kc, "bf16"), to_dev(vc, "bf16"))
    torch.cuda.synchronize()
    assert np.array_equal(u16(k_kept), oracle.kv_gather(kc, idx))
    assert np.array_equal(u16(v_kept), oracle.kv_gather(vc, idx))
    report("kv_gather_L%d_T%d_N%d" % (L, T, N), bit_exact=True)


def test_kv_gather_edges():
    rng = np.random.default_rng(3)
    kc = cache_bits(rng, 2, 50, 2, 64)
    idx = np.array([0, 49, 7, -1, 50], np.int32)      # out-of-range -> zero rows
    k_kept, v_kept = tg.tg_kv_gather(to_dev(idx), 5, k_cache=to_dev(kc, "bf16"))
    torch.cuda.synchronize()
    assert v_kept is None
    got = u16(k_kept)
    assert np.array_equal(got[:, :3], oracle.kv_gather(kc, idx[:3]))
    assert not got[:, 3:].any()
    k0, _ = tg.tg_kv_gather(to_dev(idx), 0, k_cache=to_dev(kc, "bf16"))   # N = 0
    assert k0.shape == (2, 0, 2, 64)


def test_kv_gather_beside_attention_on_a_second_stream():
    """The serving order: after the top-K, the KV gather runs on a side stream
    while the bias attention runs on the main stream; both results exact."""
    w = workloads.get("t16k")
    g, a = workloads.generate(w)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()        # default priority
    resid, prunable = to_dev(g.resid, "bf16"), to_dev(g.prunable)
    scores = tg.tg_gate_score(resid, prunable, to_dev(g.w1, "bf16"), to_dev(g.w2))
    kept, n = tg.tg_topk_select(scores, prunable, w.K)
    N = w.n_kept
    rk, pos, sk = tg.tg_compact_gather(resid, scores, kept, N)
    rng = np.random.default_rng(9)
    kc, vc = cache_bits(rng, 2, w.T, w.Hkv, w.D), cache_bits(rng, 2, w.T, w.Hkv, w.D)
    kcd, vcd = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    torch.cuda.synchronize()
    ready = torch.cuda.Event()
    ready.record(main)
    side.wait_event(ready)
    k_kept, v_kept = tg.tg_kv_gather(kept, N, kcd, vcd, stream=side)
    q, k, v = to_dev(a.q, "bf16"), to_dev(a.k, "bf16"), to_dev(a.v, "bf16")
    out, lse = tg.tg_bias_attn_fwd(q, k, v, sk, to_dev(a.gain))
    done = torch.cuda.Event()
    done.record(side)
    main.wait_event(done)
    torch.cuda.synchronize()
    idx = kept.cpu().numpy()[:N]
    assert np.array_equal(u16(k_kept), oracle.kv_gather(kc, idx))
    assert np.array_equal(u16(v_kept), oracle.kv_gather(vc, idx))
    # attention ran beside it: same bits as a lone run
    out2, _ = tg.tg_bias_attn_fwd(q, k, v, sk, to_dev(a.gain))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
