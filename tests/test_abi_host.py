"""C-ABI host checks (CPU only; no kernel is launched).

* libtokengate.so loads and exports every function include/tokengate.h
  declares;
* status strings and the workspace size query;
* every argument-validation path returns its status code before any device
  work (the pointers passed are never dereferenced, because validation
  fails first).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokengate.h")
LIB = os.path.join(ROOT, "learned_token_pruning_gate_amd", "libtokengate.so")

OK, INVAL, UNSUP, WS = 0, 1, 2, 3
F32, BF16 = 0, 1
P = ctypes.c_void_p
FAKE = P(0x1000)          # 16-byte aligned, never dereferenced
FAKE_ODD = P(0x1002)      # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import learned_token_pruning_gate_amd.build as b
        b.build()
    import learned_token_pruning_gate_amd as tg
    return tg.load()


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("tg_gate_score", "tg_topk_select", "tg_compact_gather", "tg_bias_attn_fwd",
              "tg_topk_workspace_size", "tg_status_str", "tg_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    names = [lib.tg_status_str(i).decode() for i in range(5)]
    assert names == ["TG_OK", "TG_ERR_INVALID_ARGUMENT", "TG_ERR_UNSUPPORTED",
                     "TG_ERR_WORKSPACE", "TG_ERR_LAUNCH"]
    assert lib.tg_status_str(99).decode() == "TG_ERR_UNKNOWN"


def test_workspace_size(lib):
    sizes = [lib.tg_topk_workspace_size(T) for T in (0, 1, 1000, 131072, 2**31 - 1)]
    assert all(s % 256 == 0 and s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    assert sizes[-1] < 1 << 20     # bounded by the workgroup cap


def _gate(lib, dt=BF16, T=64, d=64, h=64, resid=FAKE, stride=None, prunable=FAKE, eps=1e-6,
          w1=FAKE, w2=FAKE, scores=FAKE):
    return lib.tg_gate_score(dt, T, d, h, resid, d if stride is None else stride, prunable,
                             None, ctypes.c_float(eps), w1, None, w2, ctypes.c_float(0.0),
                             scores, None)


def test_gate_validation(lib):
    assert _gate(lib, dt=7) == INVAL
    assert _gate(lib, T=-1) == INVAL
    assert _gate(lib, d=0) == INVAL
    assert _gate(lib, h=0) == INVAL
    assert _gate(lib, eps=-1.0) == INVAL
    assert _gate(lib, T=0) == OK                      # empty input: nothing to do
    assert _gate(lib, resid=None) == INVAL
    assert _gate(lib, prunable=None) == INVAL
    assert _gate(lib, w1=None) == INVAL
    assert _gate(lib, w2=None) == INVAL
    assert _gate(lib, scores=None) == INVAL
    assert _gate(lib, stride=32) == INVAL             # stride < d
    assert _gate(lib, d=60) == UNSUP                  # bf16 needs d % 8 == 0
    assert _gate(lib, h=96) == UNSUP                  # bf16 needs h in {64,...,256}
    assert _gate(lib, h=320) == UNSUP
    assert _gate(lib, resid=FAKE_ODD) == INVAL        # misaligned bf16 resid
    assert _gate(lib, stride=68) == INVAL             # bf16 stride % 8 != 0
    assert "d % 8" in lib.tg_last_error().decode() or True


def test_gate_packed_validation(lib):
    assert lib.tg_gate_w1_packed_bytes(BF16, 256, 2048) == 256 * 2048 * 2
    assert lib.tg_gate_w1_packed_bytes(BF16, 64, 128) == 64 * 128 * 2
    assert lib.tg_gate_w1_packed_bytes(F32, 256, 2048) == 0      # a bf16 layout
    assert lib.tg_gate_w1_packed_bytes(BF16, 96, 2048) == 0      # h not a multiple of 64
    assert lib.tg_gate_w1_packed_bytes(BF16, 256, 2000) == 0     # d % 64 != 0
    assert lib.tg_gate_w1_packed_bytes(BF16, 256, 64) == 0       # d < 128
    assert lib.tg_gate_pack_w1(BF16, 256, 2000, FAKE, FAKE, None) == UNSUP
    assert lib.tg_gate_pack_w1(F32, 256, 2048, FAKE, FAKE, None) == UNSUP
    assert lib.tg_gate_pack_w1(BF16, 256, 2048, None, FAKE, None) == INVAL
    assert lib.tg_gate_pack_w1(BF16, 256, 2048, FAKE, None, None) == INVAL
    assert lib.tg_gate_pack_w1(BF16, 256, 2048, FAKE_ODD, FAKE, None) == INVAL

    def packed(dt=BF16, T=64, d=2048, h=256, gamma=None, w1=FAKE):
        return lib.tg_gate_score_packed(dt, T, d, h, FAKE, d, FAKE, gamma,
                                        ctypes.c_float(1e-6), w1, None, FAKE,
                                        ctypes.c_float(0.0), FAKE, None)
    assert packed(dt=F32) == UNSUP
    assert packed(d=2000) == UNSUP
    assert packed(h=96) == UNSUP
    assert packed(gamma=FAKE) == UNSUP          # unit RMSNorm weight only
    assert packed(w1=None) == INVAL
    assert packed(T=0) == OK
    assert "packed" in lib.tg_last_error().decode() or True


def _select(lib, T=100, scores=FAKE, prunable=FAKE, K=10, kept=FAKE, cap=100, n_kept=FAKE,
            ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.tg_topk_workspace_size(T)
    return lib.tg_topk_select(T, scores, prunable, K, kept, cap, n_kept, ws, ws_bytes, None)


def test_select_validation(lib):
    assert _select(lib, T=-1) == INVAL
    assert _select(lib, T=2**31) == INVAL
    assert _select(lib, K=-1) == INVAL
    assert _select(lib, cap=-1) == INVAL
    assert _select(lib, n_kept=None) == INVAL
    assert _select(lib, scores=None) == INVAL
    assert _select(lib, prunable=None) == INVAL
    assert _select(lib, kept=None) == INVAL
    assert _select(lib, scores=FAKE_ODD) == INVAL
    assert _select(lib, ws=None) == WS
    assert _select(lib, ws_bytes=16) == WS
    assert _select(lib, ws=P(0x1010)) == WS          # not 256-byte aligned
    assert "workspace" in lib.tg_last_error().decode()


def test_select_noalloc_validation(lib):
    """The allocation-free variant checks its arguments as tg_topk_select
    does, before it touches a device (no workspace argument to check)."""
    def sel(T=100, scores=FAKE, prunable=FAKE, K=10, kept=FAKE, cap=100, n_kept=FAKE):
        return lib.tg_topk_select_noalloc(T, scores, prunable, K, kept, cap, n_kept, None)
    assert sel(T=-1) == INVAL
    assert sel(T=2**31) == INVAL
    assert sel(K=-1) == INVAL
    assert sel(cap=-1) == INVAL
    assert sel(n_kept=None) == INVAL
    assert sel(scores=None) == INVAL
    assert sel(prunable=None) == INVAL
    assert sel(kept=None) == INVAL
    assert sel(scores=FAKE_ODD) == INVAL
    assert "tg_topk_select_noalloc" in lib.tg_last_error().decode()
    # the static scratch (64 KiB) covers the workspace of every valid T
    assert lib.tg_topk_workspace_size(2**31 - 1) <= 64 * 1024


def _gather(lib, dt=BF16, T=100, N=10, d=64, resid=FAKE, sstride=64, scores=FAKE,
            idx=FAKE, out=FAKE, dstride=64, pos=FAKE, sk=FAKE):
    return lib.tg_compact_gather(dt, T, N, d, resid, sstride, scores, idx, out, dstride, pos,
                                 sk, None)


def test_gather_validation(lib):
    assert _gather(lib, dt=5) == INVAL
    assert _gather(lib, T=-1) == INVAL
    assert _gather(lib, N=-1) == INVAL
    assert _gather(lib, d=0) == INVAL
    assert _gather(lib, N=0) == OK                    # empty gather
    assert _gather(lib, idx=None) == INVAL
    assert _gather(lib, scores=None) == INVAL         # score_kept needs scores
    assert _gather(lib, resid=None) == INVAL
    assert _gather(lib, sstride=10) == INVAL
    assert _gather(lib, dstride=10) == INVAL
    assert _gather(lib, resid=P(0x1001)) == INVAL


def _attn(lib, dt=BF16, N=64, Hq=4, Hkv=2, D=128, q=FAKE, k=FAKE, v=FAKE, ks=FAKE,
          gain=FAKE, out=FAKE):
    return lib.tg_bias_attn_fwd(dt, N, Hq, Hkv, D, q, k, v, ks, gain, None,
                                ctypes.c_float(0.0), 1, out, None, None)


def test_attn_validation(lib):
    assert _attn(lib, dt=3) == INVAL
    assert _attn(lib, N=-1) == INVAL
    assert _attn(lib, Hq=0) == INVAL
    assert _attn(lib, Hkv=0) == INVAL
    assert _attn(lib, Hq=6, Hkv=4) == INVAL           # Hq % Hkv != 0
    assert _attn(lib, D=96) == UNSUP
    assert _attn(lib, D=512) == UNSUP
    assert _attn(lib, N=0) == OK
    assert _attn(lib, q=None) == INVAL
    assert _attn(lib, out=None) == INVAL
    assert _attn(lib, gain=None) == INVAL             # bias without gain
    assert _attn(lib, k=P(0x1008)) == INVAL           # misaligned
    assert _attn(lib, N=2**30, Hq=4, Hkv=2) == UNSUP  # N * Hq beyond int32


def _attn_ws(lib, ws, nbytes, dt=BF16, N=2512, Hq=16, Hkv=8, D=128, q=FAKE, out=FAKE):
    return lib.tg_bias_attn_fwd_ws(dt, N, Hq, Hkv, D, q, FAKE, FAKE, FAKE, FAKE, None,
                                   ctypes.c_float(0.0), 0, out, None, ws, nbytes, None)


def test_attn_workspace_size(lib):
    size = lambda *a: lib.tg_bias_attn_workspace_size(*a)
    # N = 2512, 8/2 heads, D = 256, causal: 4 query heads per KV head, so 79
    # rows of 32 queries (row p has ceil(32 (p + 1) / 64) key tiles) x 2 head
    # groups; the plan cuts rows into chunks of 14 tiles, so rows 28..78 (51
    # rows) are split, with state slots for 3 chunks per head group: 51 x 3 x
    # 2 slots of 4 waves x (8 x 16 x 64 fp16 of O^T + 128 floats of max, sum)
    assert size(BF16, 2512, 8, 2, 256, 1) == 51 * 3 * 2 * 4 * (8 * 16 * 64 * 2 + 128 * 4)
    # the same prompt at 16/8 heads, D = 128: with fp16 chunk states the split
    # is priced below the two-stream launch
    assert size(BF16, 2512, 16, 8, 128, 1) > 0
    assert size(F32, 2512, 16, 8, 128, 1) == 0          # fp32 path never splits
    assert size(BF16, 32768, 16, 8, 128, 1) == 0        # grid fills the chip
    assert size(BF16, 100, 16, 8, 128, 1) == 0          # rows too short to cut
    assert size(BF16, 0, 16, 8, 128, 1) == 0
    assert size(BF16, 2512, 6, 4, 128, 1) == 0          # invalid: Hq % Hkv != 0
    assert size(BF16, 2512, 16, 8, 96, 1) == 0          # invalid head dim
    assert size(BF16, 2512, 16, 8, 128, 0) > 0          # non-causal rows split too


def test_attn_plan_cache_is_bounded(lib):
    # the kept-token count changes from prompt to prompt: 300 distinct shapes
    # overflow the plan cache (256 shapes), and a plan computed again after
    # its eviction sizes the workspace the same way
    size = lambda n: lib.tg_bias_attn_workspace_size(BF16, n, 16, 8, 128, 1)
    first = {n: size(n) for n in range(1200, 4200, 10)}
    assert any(v > 0 for v in first.values())
    for n in (1200, 2510, 4190):
        assert size(n) == first[n]


def test_attn_ws_validation(lib):
    need = lib.tg_bias_attn_workspace_size(BF16, 2512, 16, 8, 128, 0)   # non-causal splits
    assert _attn_ws(lib, FAKE, 0) == WS
    assert b"workspace" in lib.tg_last_error()
    assert _attn_ws(lib, FAKE, need - 1) == WS
    assert _attn_ws(lib, FAKE_ODD, need) == INVAL
    assert _attn_ws(lib, FAKE, need, q=None) == INVAL
    assert _attn_ws(lib, None, 0, q=None) == INVAL      # NULL workspace: unsplit checks
    assert _attn_ws(lib, FAKE, need, D=96) == UNSUP
    assert _attn_ws(lib, FAKE, 0, N=0) == OK            # nothing to do, nothing needed


def _bwd(lib, ws=FAKE, nbytes=1 << 30, dt=BF16, N=64, Hq=4, Hkv=2, D=128, q=FAKE, ks=FAKE,
         dscore=FAKE, lse=FAKE):
    return lib.tg_bias_attn_bwd(dt, N, Hq, Hkv, D, q, FAKE, FAKE, ks, FAKE, None,
                                ctypes.c_float(0.0), 1, FAKE, FAKE, lse, FAKE, FAKE, FAKE,
                                dscore, FAKE, ws, nbytes, None)


def test_attn_bwd_workspace_size(lib):
    # N = 2512, 16/8 heads, D = 128: 20 key blocks of 128 x 8 KV heads = 160
    # dK/dV workgroups, split 5 ways (768 / 160 rounded up) into chunks of
    # 8 of the 40 query tiles: 800 slots.  Delta and lse2 [Hq][N], dscore
    # partials [slot][128 keys], dgain partials [slot][4 waves][2 heads],
    # dK and dV partials [slot][2][128][D], all f32
    slots = 5 * 20 * 8
    assert lib.tg_bias_attn_bwd_workspace_size(2512, 16, 8, 128) == \
        (2 * 16 * 2512 + slots * 128 + slots * 4 * 2 + slots * 2 * 128 * 128) * 4
    assert lib.tg_bias_attn_bwd_workspace_size(0, 16, 8, 128) == 0
    assert lib.tg_bias_attn_bwd_workspace_size(100, 6, 4, 128) == 0   # Hq % Hkv != 0
    # head dim 256: the same layout with [slot][2][128][256] dK/dV partials
    # (N = 1000, 4/2 heads: 8 key blocks x 2 KV heads = 16 workgroups, split
    # 8 ways into chunks of 2 of the 16 query tiles: 128 slots)
    slots = 8 * 8 * 2
    assert lib.tg_bias_attn_bwd_workspace_size(1000, 4, 2, 256) == \
        (2 * 4 * 1000 + slots * 128 + slots * 4 * 2 + slots * 2 * 128 * 256) * 4
    assert lib.tg_bias_attn_bwd_workspace_size(100, 8, 4, 96) == 0    # head dim 96
    assert lib.tg_bias_attn_bwd_workspace_size(100, 8, 4, 512) == 0   # head dim 512


def test_attn_bwd_validation(lib):
    assert _bwd(lib, dt=3) == INVAL
    assert _bwd(lib, dt=F32) == UNSUP
    assert _bwd(lib, D=96) == UNSUP
    assert _bwd(lib, D=512) == UNSUP
    assert _bwd(lib, Hq=6, Hkv=4) == INVAL
    assert _bwd(lib, ws=None, nbytes=0) == WS
    assert _bwd(lib, nbytes=16) == WS
    assert _bwd(lib, ws=FAKE_ODD) == INVAL
    assert _bwd(lib, q=None) == INVAL
    assert _bwd(lib, lse=None) == INVAL
    assert _bwd(lib, dscore=None) == INVAL          # scores given, no dscore output
    assert _bwd(lib, N=0, ws=None, nbytes=0) == OK


def test_product_binding_refuses_cpu_tensors():
    import torch
    import learned_token_pruning_gate_amd as tg
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        tg.tg_gate_score(x, torch.ones(4, dtype=torch.uint8), x, torch.zeros(4))


def test_product_binding_fails_loudly_without_the_library():
    # no fallback: with the library missing, loading raises and says how to build
    code = ("import learned_token_pruning_gate_amd as tg\n"
            "tg.lib_path = '/nonexistent/libtokengate.so'\n"
            "tg._lib = None\n"
            "try:\n"
            "    tg.load()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    import subprocess
    import sys
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert "raised: libtokengate.so is not built" in r.stdout


def test_product_package_does_not_import_the_oracle():
    src_dir = os.path.join(ROOT, "learned_token_pruning_gate_amd")
    for dirpath, _, files in os.walk(src_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "tg_oracle" not in text, f
                assert "liboracle" not in text, f


def test_chain_null_arguments(lib):
    """tg_chain_create validates its own pointers before any HIP call."""
    import learned_token_pruning_gate_amd as tg
    h = ctypes.c_void_p()
    desc = tg.ChainDesc()
    assert lib.tg_chain_create(None, ctypes.byref(h)) == INVAL
    assert lib.tg_chain_create(ctypes.byref(desc), None) == INVAL
    assert lib.tg_chain_launch(None, None) == INVAL
    lib.tg_chain_destroy(None)          # a no-op


def test_chain_desc_layout_matches_header():
    """The ctypes mirror names the header's fields in the header's order."""
    import learned_token_pruning_gate_amd as tg
    src = open(HEADER).read()
    body = src[src.index("typedef struct tg_chain_desc {"):src.index("} tg_chain_desc;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = []
    for decl in body.split(";")[:-1]:
        decl = decl.split("{")[-1].strip()
        if not decl:
            continue
        # "int64_t T, d, h" -> T, d, h ; "const void* resid" -> resid
        parts = decl.replace("*", " ").split(",")
        first = parts[0].split()[-1]
        names.append(first)
        names.extend(p.strip() for p in parts[1:])
    assert [f[0] for f in tg.ChainDesc._fields_] == names


def test_kv_gather_validation(lib):
    def kv(dt=BF16, L=2, T=100, N=10, Hkv=8, D=128, kc=FAKE, vc=FAKE, idx=FAKE, ko=FAKE, vo=FAKE):
        return lib.tg_kv_gather(dt, L, T, N, Hkv, D, kc, vc, idx, ko, vo, None)
    assert kv(dt=9) == INVAL
    assert kv(L=-1) == INVAL
    assert kv(N=-1) == INVAL
    assert kv(Hkv=0) == INVAL
    assert kv(Hkv=1, D=3) == UNSUP     # a row of 3 * 2 bytes is not a multiple of 16
    assert kv(L=0) == OK and kv(N=0) == OK
    assert kv(idx=None) == INVAL
    assert kv(kc=None) == INVAL        # cache and output must come together
    assert kv(kc=None, ko=None, vc=None, vo=None) == OK   # nothing to gather, nothing launched
    assert kv(ko=FAKE_ODD) == INVAL
