"""Token-gated prefill path for AMD Instinct MI355X (gfx950).

Thin Python binding over ``libtokengate.so`` (C ABI in ``include/tokengate.h``).
This module only marshals arguments: PyTorch supplies device memory and the
stream, and every step of the path runs in the library's HIP kernels.  There
is no CPU fallback: if the library is missing, or a tensor is not on the
GPU, the call raises.

Entry points (same names as the C ABI):

* ``tg_gate_score``       -- RMSNorm + MLP scorer over the residual rows
* ``tg_gate_w1_packed_bytes`` / ``tg_gate_pack_w1`` / ``tg_gate_score_packed``
                          -- the same scorer with W1 packed once, at weight
                             load, into the MFMA fragment order
* ``tg_topk_workspace_size`` / ``tg_topk_select`` -- top-K + compaction
* ``tg_topk_select_noalloc`` -- the same with the library's static scratch
                          (for callers that cannot allocate device memory)
* ``tg_compact_gather``   -- gather of rows, positions and scores
* ``tg_bias_attn_fwd``    -- causal GQA attention with the gate bias
* ``tg_bias_attn_workspace_size`` / ``tg_bias_attn_fwd_ws`` -- the same with
                          long rows' keys split over workgroups (short prompts)
* ``tg_bias_attn_bwd_workspace_size`` / ``tg_bias_attn_bwd`` -- its gradients
                          (dQ, dK, dV, dscore, dgain)
* ``tg_kv_gather``        -- lower layers' KV cache gathered to the kept tokens
* ``tg_chain_create`` / ``TgChain.launch`` -- the four calls captured once as
                          a HIP graph and replayed
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "TokenGateError", "lib_path", "load", "kept_count",
    "tg_status_str", "tg_last_error", "tg_gate_score", "tg_gate_w1_packed_bytes",
    "tg_gate_pack_w1", "tg_gate_score_packed", "tg_topk_workspace_size",
    "tg_topk_select", "tg_topk_select_noalloc", "tg_compact_gather", "tg_bias_attn_fwd",
    "tg_bias_attn_workspace_size",
    "tg_bias_attn_fwd_ws", "tg_bias_attn_bwd_workspace_size", "tg_bias_attn_bwd",
    "tg_kv_gather", "tg_chain_create", "TgChain",
    "TG_OK", "TG_ERR_INVALID_ARGUMENT", "TG_ERR_UNSUPPORTED", "TG_ERR_WORKSPACE",
    "TG_ERR_LAUNCH", "TG_DTYPE_F32", "TG_DTYPE_BF16",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libtokengate.so")

TG_OK, TG_ERR_INVALID_ARGUMENT, TG_ERR_UNSUPPORTED, TG_ERR_WORKSPACE, TG_ERR_LAUNCH = range(5)
TG_DTYPE_F32, TG_DTYPE_BF16 = 0, 1

EXPORTED = ("tg_status_str", "tg_last_error", "tg_gate_score", "tg_gate_w1_packed_bytes",
            "tg_gate_pack_w1", "tg_gate_score_packed", "tg_topk_workspace_size",
            "tg_topk_select", "tg_topk_select_noalloc", "tg_compact_gather", "tg_bias_attn_fwd",
            "tg_bias_attn_workspace_size", "tg_bias_attn_fwd_ws",
            "tg_bias_attn_bwd_workspace_size", "tg_bias_attn_bwd", "tg_kv_gather",
            "tg_chain_create",
            "tg_chain_launch", "tg_chain_destroy")


class TokenGateError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s: %s: %s" % (where, _status_name(status), detail))


_lib = None


class ChainDesc(ctypes.Structure):
    """Mirror of tg_chain_desc (include/tokengate.h), field for field."""
    _P, _I64, _F, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    _fields_ = [
        ("dt", _I), ("T", _I64), ("d", _I64), ("h", _I64), ("resid", _P),
        ("resid_row_stride", _I64), ("prunable", _P), ("rms_weight", _P), ("eps", _F),
        ("w1", _P), ("w1_packed", _I), ("b1", _P), ("w2", _P), ("b2", _F), ("scores", _P),
        ("K", _I64), ("kept_idx", _P), ("kept_capacity", _I64), ("n_kept", _P),
        ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
        ("N", _I64), ("resid_kept", _P), ("kept_row_stride", _I64), ("pos_kept", _P),
        ("score_kept", _P),
        ("Hq", _I64), ("Hkv", _I64), ("D", _I64), ("q", _P), ("k", _P), ("v", _P),
        ("attn_key_score", _P), ("gain", _P), ("q_scale", _P), ("softmax_scale", _F),
        ("causal", _I), ("out", _P), ("lse", _P),
        ("kv_L", _I64), ("kv_k_cache", _P), ("kv_v_cache", _P), ("kv_k_kept", _P),
        ("kv_v_kept", _P), ("attn_workspace", _P), ("attn_workspace_bytes", ctypes.c_size_t),
        ("prompt_len", _P),
    ]


def load():
    """Load libtokengate.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(
            "libtokengate.so is not built (%s); run "
            "`python learned_token_pruning_gate_amd/build.py`" % lib_path)
    lib = ctypes.CDLL(lib_path)
    P, I64, F, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.tg_status_str.argtypes = [I]
    lib.tg_status_str.restype = ctypes.c_char_p
    lib.tg_last_error.argtypes = []
    lib.tg_last_error.restype = ctypes.c_char_p
    lib.tg_gate_score.argtypes = [I, I64, I64, I64, P, I64, P, P, F, P, P, P, F, P, P]
    lib.tg_gate_score.restype = I
    lib.tg_gate_score_packed.argtypes = [I, I64, I64, I64, P, I64, P, P, F, P, P, P, F, P, P]
    lib.tg_gate_score_packed.restype = I
    lib.tg_gate_w1_packed_bytes.argtypes = [I, I64, I64]
    lib.tg_gate_w1_packed_bytes.restype = ctypes.c_size_t
    lib.tg_gate_pack_w1.argtypes = [I, I64, I64, P, P, P]
    lib.tg_gate_pack_w1.restype = I
    lib.tg_topk_workspace_size.argtypes = [I64]
    lib.tg_topk_workspace_size.restype = ctypes.c_size_t
    lib.tg_topk_select.argtypes = [I64, P, P, I64, P, I64, P, P, ctypes.c_size_t, P]
    lib.tg_topk_select.restype = I
    lib.tg_topk_select_noalloc.argtypes = [I64, P, P, I64, P, I64, P, P]
    lib.tg_topk_select_noalloc.restype = I
    lib.tg_compact_gather.argtypes = [I, I64, I64, I64, P, I64, P, P, P, I64, P, P, P]
    lib.tg_compact_gather.restype = I
    lib.tg_bias_attn_fwd.argtypes = [I, I64, I64, I64, I64, P, P, P, P, P, P, F, I, P, P, P]
    lib.tg_bias_attn_fwd.restype = I
    lib.tg_bias_attn_workspace_size.argtypes = [I, I64, I64, I64, I64, I]
    lib.tg_bias_attn_workspace_size.restype = ctypes.c_size_t
    lib.tg_bias_attn_fwd_ws.argtypes = [I, I64, I64, I64, I64, P, P, P, P, P, P, F, I, P, P, P,
                                        ctypes.c_size_t, P]
    lib.tg_bias_attn_fwd_ws.restype = I
    lib.tg_bias_attn_bwd_workspace_size.argtypes = [I64, I64, I64, I64]
    lib.tg_bias_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.tg_bias_attn_bwd.argtypes = [I, I64, I64, I64, I64, P, P, P, P, P, P, F, I, P, P, P, P, P,
                                     P, P, P, P, ctypes.c_size_t, P]
    lib.tg_bias_attn_bwd.restype = I
    lib.tg_kv_gather.argtypes = [I, I64, I64, I64, I64, I64, P, P, P, P, P, P]
    lib.tg_kv_gather.restype = I
    lib.tg_chain_create.argtypes = [ctypes.POINTER(ChainDesc), ctypes.POINTER(P)]
    lib.tg_chain_create.restype = I
    lib.tg_chain_launch.argtypes = [P, P]
    lib.tg_chain_launch.restype = I
    lib.tg_chain_destroy.argtypes = [P]
    lib.tg_chain_destroy.restype = None
    _lib = lib
    return lib


def _status_name(s: int) -> str:
    return load().tg_status_str(int(s)).decode()


def tg_status_str(status: int) -> str:
    return _status_name(status)


def tg_last_error() -> str:
    return load().tg_last_error().decode()


def _check(status: int, where: str):
    if status != TG_OK:
        raise TokenGateError(status, where, tg_last_error())


def _dev(t, name, dtype=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _addr(t):
    return 0 if t is None else int(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return TG_DTYPE_BF16
    if t.dtype == torch.float32:
        return TG_DTYPE_F32
    raise TypeError("unsupported dtype %s (bf16 or f32)" % t.dtype)


def kept_count(n_prunable: int, T: int, K: int) -> int:
    """N = min(K, |P|) + |not P|: the number of kept tokens."""
    return min(int(K), int(n_prunable)) + (int(T) - int(n_prunable))


# ---------------------------------------------------------------------------
def tg_gate_score(resid, prunable, w1, w2, b2=0.0, rms_weight=None, b1=None, eps=1e-6,
                  scores=None, stream=None):
    """scores[T] (f32) for resid [T, d] (bf16 or f32, row stride >= d)."""
    lib = load()
    _dev(resid, "resid")
    T, d = resid.shape
    if resid.stride(1) != 1:
        raise ValueError("resid rows must be contiguous")
    _dev(prunable, "prunable", torch.uint8)
    _dev(w1, "w1", resid.dtype)
    h = w1.shape[0]
    if tuple(w1.shape) != (h, d) or not w1.is_contiguous():
        raise ValueError("w1 must be a contiguous [h, d] tensor")
    _dev(w2, "w2", torch.float32)
    _dev(rms_weight, "rms_weight", torch.float32, allow_none=True)
    _dev(b1, "b1", torch.float32, allow_none=True)
    if scores is None:
        scores = torch.empty(T, dtype=torch.float32, device=resid.device)
    _dev(scores, "scores", torch.float32)
    st = lib.tg_gate_score(_dt(resid), T, d, h, _ptr(resid), resid.stride(0), _ptr(prunable),
                           _ptr(rms_weight), float(eps), _ptr(w1), _ptr(b1), _ptr(w2),
                           float(b2), _ptr(scores), _stream(stream))
    _check(st, "tg_gate_score")
    return scores


def tg_gate_w1_packed_bytes(dtype, h: int, d: int) -> int:
    """Bytes of the packed W1 layout (0 if that layout does not cover h, d)."""
    dt = TG_DTYPE_BF16 if dtype == torch.bfloat16 else TG_DTYPE_F32
    return int(load().tg_gate_w1_packed_bytes(dt, int(h), int(d)))


def tg_gate_pack_w1(w1, out=None, stream=None):
    """Packed copy of a contiguous bf16 W1 [h, d] (a flat bf16 tensor)."""
    lib = load()
    _dev(w1, "w1", torch.bfloat16)
    if w1.dim() != 2 or not w1.is_contiguous():
        raise ValueError("w1 must be a contiguous [h, d] tensor")
    h, d = w1.shape
    if out is None:
        out = torch.empty(h * d, dtype=torch.bfloat16, device=w1.device)
    _dev(out, "out", torch.bfloat16)
    if out.numel() * 2 < tg_gate_w1_packed_bytes(torch.bfloat16, h, d):
        raise ValueError("out holds fewer bytes than the packed layout")
    _check(lib.tg_gate_pack_w1(TG_DTYPE_BF16, h, d, _ptr(w1), _ptr(out), _stream(stream)),
           "tg_gate_pack_w1")
    return out


def tg_gate_score_packed(resid, prunable, w1_packed, w2, b2=0.0, b1=None, eps=1e-6,
                         scores=None, stream=None):
    """tg_gate_score with W1 from tg_gate_pack_w1; h is w2's length."""
    lib = load()
    _dev(resid, "resid", torch.bfloat16)
    T, d = resid.shape
    if resid.stride(1) != 1:
        raise ValueError("resid rows must be contiguous")
    _dev(prunable, "prunable", torch.uint8)
    _dev(w2, "w2", torch.float32)
    h = w2.shape[0]
    _dev(w1_packed, "w1_packed", torch.bfloat16)
    if w1_packed.numel() != h * d or not w1_packed.is_contiguous():
        raise ValueError("w1_packed must be the contiguous output of tg_gate_pack_w1")
    _dev(b1, "b1", torch.float32, allow_none=True)
    if scores is None:
        scores = torch.empty(T, dtype=torch.float32, device=resid.device)
    _dev(scores, "scores", torch.float32)
    st = lib.tg_gate_score_packed(TG_DTYPE_BF16, T, d, h, _ptr(resid), resid.stride(0),
                                  _ptr(prunable), None, float(eps), _ptr(w1_packed), _ptr(b1),
                                  _ptr(w2), float(b2), _ptr(scores), _stream(stream))
    _check(st, "tg_gate_score_packed")
    return scores


def tg_kv_gather(kept_idx, N, k_cache=None, v_cache=None, k_kept=None, v_kept=None,
                 stream=None):
    """(k_kept, v_kept) [L, N, Hkv, D] from caches [L, T, Hkv, D] (either may
    be None); kept_idx is tg_topk_select's output (its first N entries)."""
    lib = load()
    ref = k_cache if k_cache is not None else v_cache
    if ref is None:
        raise ValueError("give k_cache and/or v_cache")
    _dev(kept_idx, "kept_idx", torch.int32)
    L, T, Hkv, D = ref.shape
    outs = []
    for c, o, name in ((k_cache, k_kept, "k"), (v_cache, v_kept, "v")):
        if c is None:
            outs.append(None)
            continue
        _dev(c, name + "_cache", ref.dtype)
        if tuple(c.shape) != (L, T, Hkv, D) or not c.is_contiguous():
            raise ValueError(name + "_cache must be a contiguous [L, T, Hkv, D] tensor")
        if o is None:
            o = torch.empty((L, int(N), Hkv, D), dtype=c.dtype, device=c.device)
        _dev(o, name + "_kept", c.dtype)
        if tuple(o.shape) != (L, int(N), Hkv, D) or not o.is_contiguous():
            raise ValueError(name + "_kept must be a contiguous [L, N, Hkv, D] tensor")
        outs.append(o)
    st = lib.tg_kv_gather(_dt(ref), L, T, int(N), Hkv, D, _ptr(k_cache), _ptr(v_cache),
                          _ptr(kept_idx), _ptr(outs[0]), _ptr(outs[1]), _stream(stream))
    _check(st, "tg_kv_gather")
    return outs[0], outs[1]


class TgChain:
    """A captured chain (tg_chain_create); keeps its tensors alive."""

    def __init__(self, handle, keep):
        self._h = handle
        self._keep = keep

    def launch(self, stream=None):
        if self._h is None:
            raise ValueError("chain was closed")
        _check(load().tg_chain_launch(self._h, _stream(stream)), "tg_chain_launch")

    def close(self):
        if self._h is not None:
            load().tg_chain_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tg_chain_create(*, resid, prunable, w1, w2, scores, K, kept_idx, n_kept, workspace,
                    N, resid_kept, pos_kept, score_kept, q, k, v, attn_key_score, gain,
                    out, w1_packed=False, b2=0.0, rms_weight=None, b1=None, eps=1e-6,
                    q_scale=None, softmax_scale=0.0, causal=True, lse=None,
                    kv_k_cache=None, kv_v_cache=None, kv_k_kept=None, kv_v_kept=None,
                    attn_workspace=None, prompt_len=None):
    """Capture gate -> top-K -> gather -> bias attention into one HIP graph.
    Every argument is the tensor the corresponding call would take; the graph
    keeps their addresses, so refill inputs in place between launches.  N is
    a capacity (rows past the device kept count are padding); ``prompt_len``
    (a 1-element int32 device tensor, or None) makes T a capacity too: the
    replay reads the prompt's length from it."""
    lib = load()
    _dev(prompt_len, "prompt_len", torch.int32, allow_none=True)
    T, d = resid.shape
    h = w2.shape[0]
    Nq, Hq, D = q.shape
    desc = ChainDesc(
        dt=_dt(resid), T=T, d=d, h=h, resid=_addr(resid), resid_row_stride=resid.stride(0),
        prunable=_addr(prunable), rms_weight=_addr(rms_weight), eps=float(eps), w1=_addr(w1),
        w1_packed=1 if w1_packed else 0, b1=_addr(b1), w2=_addr(w2), b2=float(b2),
        scores=_addr(scores), K=int(K), kept_idx=_addr(kept_idx), kept_capacity=kept_idx.numel(),
        n_kept=_addr(n_kept), workspace=_addr(workspace), workspace_bytes=workspace.numel(),
        N=int(N), resid_kept=_addr(resid_kept), kept_row_stride=resid_kept.stride(0),
        pos_kept=_addr(pos_kept), score_kept=_addr(score_kept), Hq=Hq, Hkv=k.shape[1], D=D,
        q=_addr(q), k=_addr(k), v=_addr(v), attn_key_score=_addr(attn_key_score), gain=_addr(gain),
        q_scale=_addr(q_scale), softmax_scale=float(softmax_scale), causal=1 if causal else 0,
        out=_addr(out), lse=_addr(lse),
        kv_L=(kv_k_cache if kv_k_cache is not None else kv_v_cache).shape[0]
        if (kv_k_cache is not None or kv_v_cache is not None) else 0,
        kv_k_cache=_addr(kv_k_cache), kv_v_cache=_addr(kv_v_cache),
        kv_k_kept=_addr(kv_k_kept), kv_v_kept=_addr(kv_v_kept),
        attn_workspace=_addr(attn_workspace),
        attn_workspace_bytes=0 if attn_workspace is None else attn_workspace.numel(),
        prompt_len=_addr(prompt_len))
    h_out = ctypes.c_void_p()
    _check(lib.tg_chain_create(ctypes.byref(desc), ctypes.byref(h_out)), "tg_chain_create")
    keep = [resid, prunable, w1, w2, scores, kept_idx, n_kept, workspace, resid_kept,
            pos_kept, score_kept, q, k, v, attn_key_score, gain, out, rms_weight, b1,
            q_scale, lse, kv_k_cache, kv_v_cache, kv_k_kept, kv_v_kept, attn_workspace,
            prompt_len]
    return TgChain(h_out, keep)


def tg_topk_workspace_size(T: int) -> int:
    return int(load().tg_topk_workspace_size(int(T)))


def tg_topk_select(scores, prunable, K, kept_idx=None, n_kept=None, workspace=None,
                   stream=None):
    """(kept_idx, n_kept): kept_idx has capacity T unless given; its first N
    entries are the kept tokens in ascending order; n_kept is a 1-element
    int32 device tensor holding N.  ``workspace`` (uint8, zero-initialised
    once) may be reused across calls on one stream."""
    lib = load()
    _dev(scores, "scores", torch.float32)
    _dev(prunable, "prunable", torch.uint8)
    T = scores.shape[0]
    dev = scores.device
    if kept_idx is None:
        kept_idx = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    _dev(kept_idx, "kept_idx", torch.int32)
    if n_kept is None:
        n_kept = torch.empty(1, dtype=torch.int32, device=dev)
    _dev(n_kept, "n_kept", torch.int32)
    need = tg_topk_workspace_size(T)
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8)
    st = lib.tg_topk_select(T, _ptr(scores), _ptr(prunable), int(K), _ptr(kept_idx),
                            kept_idx.numel(), _ptr(n_kept), _ptr(workspace),
                            workspace.numel(), _stream(stream))
    _check(st, "tg_topk_select")
    return kept_idx, n_kept


def tg_topk_select_noalloc(scores, prunable, K, kept_idx=None, n_kept=None, stream=None):
    """tg_topk_select with the library's static scratch (no workspace
    argument): (kept_idx, n_kept) as tg_topk_select returns them."""
    lib = load()
    _dev(scores, "scores", torch.float32)
    _dev(prunable, "prunable", torch.uint8)
    T = scores.shape[0]
    dev = scores.device
    if kept_idx is None:
        kept_idx = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    _dev(kept_idx, "kept_idx", torch.int32)
    if n_kept is None:
        n_kept = torch.empty(1, dtype=torch.int32, device=dev)
    _dev(n_kept, "n_kept", torch.int32)
    st = lib.tg_topk_select_noalloc(T, _ptr(scores), _ptr(prunable), int(K), _ptr(kept_idx),
                                    kept_idx.numel(), _ptr(n_kept), _stream(stream))
    _check(st, "tg_topk_select_noalloc")
    return kept_idx, n_kept


def tg_compact_gather(resid, scores, kept_idx, N, resid_kept=None, pos_kept=None,
                      score_kept=None, stream=None):
    """(resid_kept [N, d], pos_kept [N] int32, score_kept [N] f32)."""
    lib = load()
    _dev(resid, "resid")
    T, d = resid.shape
    _dev(scores, "scores", torch.float32)
    _dev(kept_idx, "kept_idx", torch.int32)
    N = int(N)
    if N > kept_idx.numel():
        raise ValueError("N exceeds kept_idx")
    dev = resid.device
    if resid_kept is None:
        resid_kept = torch.empty((N, d), dtype=resid.dtype, device=dev)
    if pos_kept is None:
        pos_kept = torch.empty(N, dtype=torch.int32, device=dev)
    if score_kept is None:
        score_kept = torch.empty(N, dtype=torch.float32, device=dev)
    _dev(resid_kept, "resid_kept", resid.dtype)
    _dev(pos_kept, "pos_kept", torch.int32)
    _dev(score_kept, "score_kept", torch.float32)
    st = lib.tg_compact_gather(_dt(resid), T, N, d, _ptr(resid), resid.stride(0),
                               _ptr(scores), _ptr(kept_idx), _ptr(resid_kept),
                               resid_kept.stride(0), _ptr(pos_kept), _ptr(score_kept),
                               _stream(stream))
    _check(st, "tg_compact_gather")
    return resid_kept, pos_kept, score_kept


def tg_bias_attn_workspace_size(N: int, Hq: int, Hkv: int, D: int, causal=True,
                                dtype=torch.bfloat16) -> int:
    """Bytes of the split-key workspace for this shape (0: runs unsplit)."""
    dt = TG_DTYPE_BF16 if dtype == torch.bfloat16 else TG_DTYPE_F32
    return int(load().tg_bias_attn_workspace_size(dt, int(N), int(Hq), int(Hkv), int(D),
                                                  1 if causal else 0))


def tg_bias_attn_fwd_ws(q, k, v, key_score, gain, workspace, q_scale=None, softmax_scale=0.0,
                        causal=True, out=None, lse=None, want_lse=True, stream=None):
    """tg_bias_attn_fwd with a split-key workspace (a uint8 device tensor of
    tg_bias_attn_workspace_size bytes, or None)."""
    return _bias_attn(q, k, v, key_score, gain, q_scale, softmax_scale, causal, out, lse,
                      want_lse, stream, True, workspace)


def tg_bias_attn_bwd_workspace_size(N: int, Hq: int, Hkv: int, D: int) -> int:
    return int(load().tg_bias_attn_bwd_workspace_size(int(N), int(Hq), int(Hkv), int(D)))


def tg_bias_attn_bwd(q, k, v, key_score, gain, out, dout, lse, q_scale=None, softmax_scale=0.0,
                     causal=True, workspace=None, stream=None):
    """(dq, dk, dv, dscore, dgain); dscore/dgain are None without key_score."""
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _dev(t, n, q.dtype)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    N, Hq, D = q.shape
    Hkv = k.shape[1]
    if tuple(out.shape) != (N, Hq, D) or tuple(dout.shape) != (N, Hq, D):
        raise ValueError("out and dout must be [N, Hq, D]")
    _dev(lse, "lse", torch.float32)
    _dev(key_score, "key_score", torch.float32, allow_none=True)
    _dev(gain, "gain", torch.float32, allow_none=True)
    _dev(q_scale, "q_scale", torch.float32, allow_none=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dscore = dgain = None
    if key_score is not None:
        dscore = torch.empty(N, dtype=torch.float32, device=q.device)
        dgain = torch.empty(Hq, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(tg_bias_attn_bwd_workspace_size(N, Hq, Hkv, D), 16),
                                dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    st = lib.tg_bias_attn_bwd(_dt(q), N, Hq, Hkv, D, _ptr(q), _ptr(k), _ptr(v), _ptr(key_score),
                              _ptr(gain), _ptr(q_scale), float(softmax_scale),
                              1 if causal else 0, _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                              _ptr(dk), _ptr(dv), _ptr(dscore), _ptr(dgain), _ptr(workspace),
                              workspace.numel(), _stream(stream))
    _check(st, "tg_bias_attn_bwd")
    return dq, dk, dv, dscore, dgain


def tg_bias_attn_fwd(q, k, v, key_score, gain, q_scale=None, softmax_scale=0.0, causal=True,
                     out=None, lse=None, want_lse=True, stream=None):
    """(out [N, Hq, D], lse [Hq, N] or None)."""
    return _bias_attn(q, k, v, key_score, gain, q_scale, softmax_scale, causal, out, lse,
                      want_lse, stream, False, None)


def _bias_attn(q, k, v, key_score, gain, q_scale, softmax_scale, causal, out, lse, want_lse,
               stream, ws_entry, workspace):
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, q.dtype)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    N, Hq, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (N, Hkv, D) or tuple(v.shape) != (N, Hkv, D):
        raise ValueError("k and v must be [N, Hkv, D]")
    _dev(key_score, "key_score", torch.float32, allow_none=True)
    _dev(gain, "gain", torch.float32, allow_none=True)
    _dev(q_scale, "q_scale", torch.float32, allow_none=True)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    if lse is None and want_lse:
        lse = torch.empty((Hq, N), dtype=torch.float32, device=q.device)
    _dev(lse, "lse", torch.float32, allow_none=True)
    if ws_entry:
        if workspace is not None:
            _dev(workspace, "workspace", torch.uint8)
        st = lib.tg_bias_attn_fwd_ws(_dt(q), N, Hq, Hkv, D, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(key_score), _ptr(gain), _ptr(q_scale),
                                     float(softmax_scale), 1 if causal else 0, _ptr(out),
                                     _ptr(lse), _ptr(workspace),
                                     0 if workspace is None else workspace.numel(),
                                     _stream(stream))
        _check(st, "tg_bias_attn_fwd_ws")
        return out, lse
    st = lib.tg_bias_attn_fwd(_dt(q), N, Hq, Hkv, D, _ptr(q), _ptr(k), _ptr(v),
                              _ptr(key_score), _ptr(gain), _ptr(q_scale),
                              float(softmax_scale), 1 if causal else 0, _ptr(out), _ptr(lse),
                              _stream(stream))
    _check(st, "tg_bias_attn_fwd")
    return out, lse
