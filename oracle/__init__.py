"""Plain fp64 CPU oracle for the token-gated prefill path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``learned_token_pruning_gate_amd`` and neither
imports the other.

The arithmetic lives in ``tg_oracle.c`` (plain C, fp64, one output at a
time); this module only marshals numpy arrays into it.  Each wrapper names
the passage of the TokenGate pages its step follows:

* ``gate_score``   -- ai.info summary "Key Contributions" item 1; techbycountry
  "how the gate works"; README mirror "How it works": RMSNorm of the
  post-attention residual, then an MLP d -> h (SiLU) -> 1 per prunable token.
* ``topk_select``  -- ai.info summary "Key Contributions" item 1 and
  "Methodology in Plain English": keep the top-K prunable tokens plus every
  non-prunable token.
* ``compact_gather`` -- same passages: upper layers process only kept tokens.
* ``bias_attn``    -- ai.info summary "Key Contributions" items 2-3 and
  "Methodology in Plain English": a per-key, per-head gate bias is added to
  the attention logits before the softmax, scaled by a per-head gain, with
  a per-query temperature.

Parity pins for every function are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "tg_oracle.c")


def build(force: bool = True, src: str = SRC_PATH, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fast-math, no FMA
    contraction) into ``oracle/liboracle.so`` (or ``out``)."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-I", _HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    D = ctypes.c_double
    lib.tgo_gate_score.argtypes = [I64, I64, I64, P, P, P, D, P, P, P, D, P]
    lib.tgo_gate_score.restype = None
    lib.tgo_topk_select.argtypes = [I64, P, P, I64, P]
    lib.tgo_topk_select.restype = I64
    lib.tgo_compact_gather.argtypes = [I64, I64, P, I64, P, P, P, P, P]
    lib.tgo_compact_gather.restype = None
    lib.tgo_kv_gather.argtypes = [I64, I64, I64, I64, P, P, P]
    lib.tgo_kv_gather.restype = None
    lib.tgo_bias_attn.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, D,
                                  ctypes.c_int, P, I64, P, P]
    lib.tgo_bias_attn.restype = None
    lib.tgo_bias_attn_bwd.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, D, ctypes.c_int,
                                      P, P, P, P, P, P]
    lib.tgo_bias_attn_bwd.restype = None
    lib.tgo_num_threads.argtypes = []
    lib.tgo_num_threads.restype = ctypes.c_int
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


class Oracle:
    """The oracle's functions bound to one compiled library: the default
    ``oracle/liboracle.so`` unless another path is given."""

    def __init__(self, lib_path: str | None = None):
        if lib_path is None:
            if not os.path.exists(LIB_PATH):
                build()
            lib_path = LIB_PATH
        self._lib = _bind(lib_path)

    def num_threads(self) -> int:
        return int(self._lib.tgo_num_threads())

    def gate_score(self, resid, prunable, w1, w2, b2=0.0, gamma=None, b1=None,
                   eps=1e-6) -> np.ndarray:
        """fp64 gate scores [T]; 0 for non-prunable tokens."""
        resid = _f64(resid)
        T, d = resid.shape
        w1 = _f64(w1)
        h = w1.shape[0]
        assert w1.shape == (h, d)
        prunable = np.ascontiguousarray(prunable, dtype=np.uint8)
        assert prunable.shape == (T,)
        w2 = _f64(w2)
        assert w2.shape == (h,)
        gamma = _f64(gamma)
        b1 = _f64(b1)
        out = np.empty(T, dtype=np.float64)
        self._lib.tgo_gate_score(T, d, h, _ptr(resid), _ptr(prunable),
                                 _ptr(gamma), float(eps), _ptr(w1), _ptr(b1),
                                 _ptr(w2), float(b2), _ptr(out))
        return out

    def topk_select(self, scores, prunable, K) -> np.ndarray:
        """Kept token indices (int32, ascending).  ``scores`` are taken as
        fp32, the precision the selection is made in."""
        scores = np.ascontiguousarray(scores, dtype=np.float32)
        prunable = np.ascontiguousarray(prunable, dtype=np.uint8)
        T = scores.shape[0]
        assert prunable.shape == (T,)
        out = np.empty(max(T, 1), dtype=np.int32)
        n = self._lib.tgo_topk_select(T, _ptr(scores), _ptr(prunable), int(K),
                                      _ptr(out))
        if n < 0:
            raise ValueError("topk_select: K must be >= 0")
        return out[:n].copy()

    def compact_gather(self, resid, scores, kept_idx):
        """(resid_kept, pos_kept, score_kept): byte-exact row gather."""
        resid = np.ascontiguousarray(resid)
        scores = np.ascontiguousarray(scores, dtype=np.float32)
        kept_idx = np.ascontiguousarray(kept_idx, dtype=np.int32)
        N = kept_idx.shape[0]
        T = resid.shape[0]
        if N and (kept_idx.min() < 0 or kept_idx.max() >= T):
            raise IndexError("kept index out of range")
        row_bytes = resid.strides[0]
        out = np.empty((N,) + resid.shape[1:], dtype=resid.dtype)
        pos = np.empty(N, dtype=np.int32)
        sk = np.empty(N, dtype=np.float32)
        self._lib.tgo_compact_gather(N, row_bytes, _ptr(resid), row_bytes,
                                     _ptr(scores), _ptr(kept_idx), _ptr(out),
                                     _ptr(pos), _ptr(sk))
        return out, pos, sk

    def kv_gather(self, cache, kept_idx):
        """cache [L, T, ...] -> [L, N, ...]: byte-exact gather of token rows."""
        cache = np.ascontiguousarray(cache)
        kept_idx = np.ascontiguousarray(kept_idx, dtype=np.int32)
        L, T = cache.shape[:2]
        N = kept_idx.shape[0]
        if N and (kept_idx.min() < 0 or kept_idx.max() >= T):
            raise IndexError("kept index out of range")
        row_bytes = cache.strides[1]
        out = np.empty((L, N) + cache.shape[2:], dtype=cache.dtype)
        self._lib.tgo_kv_gather(L, T, N, row_bytes, _ptr(cache), _ptr(kept_idx), _ptr(out))
        return out

    def bias_attn(self, q, k, v, key_score, gain, q_scale=None, scale=None,
                  causal=True, rows=None):
        """(out, lse): out [n_rows, Hq, D] fp64, lse [Hq, n_rows] fp64.

        ``rows`` (optional) lists the query rows to compute; default all N."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        N, Hq, D = q.shape
        Hkv = k.shape[1]
        assert k.shape == (N, Hkv, D) and v.shape == (N, Hkv, D)
        assert Hkv > 0 and Hq % Hkv == 0
        key_score = _f64(key_score)
        gain = _f64(gain)
        assert key_score.shape == (N,) and gain.shape == (Hq,)
        q_scale = _f64(q_scale)
        if scale is None or scale <= 0:
            scale = 1.0 / np.sqrt(D)
        if rows is not None:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            assert rows.ndim == 1
            assert rows.size == 0 or (rows.min() >= 0 and rows.max() < N)
            n_rows = rows.shape[0]
        else:
            n_rows = N
        out = np.empty((n_rows, Hq, D), dtype=np.float64)
        lse = np.empty((Hq, n_rows), dtype=np.float64)
        self._lib.tgo_bias_attn(N, Hq, Hkv, D, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(key_score), _ptr(gain), _ptr(q_scale),
                                float(scale), 1 if causal else 0, _ptr(rows),
                                n_rows, _ptr(out), _ptr(lse))
        return out, lse


    def bias_attn_bwd(self, q, k, v, key_score, gain, dout, q_scale=None, scale=None,
                      causal=True):
        """(dq [N,Hq,D], dk [N,Hkv,D], dv [N,Hkv,D], dscore [N], dgain [Hq]),
        fp64: gradients of sum(out * dout) for the forward of bias_attn."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        N, Hq, D = q.shape
        Hkv = k.shape[1]
        assert k.shape == (N, Hkv, D) and v.shape == (N, Hkv, D) and dout.shape == q.shape
        assert Hkv > 0 and Hq % Hkv == 0
        key_score, gain, q_scale = _f64(key_score), _f64(gain), _f64(q_scale)
        assert key_score.shape == (N,) and gain.shape == (Hq,)
        if scale is None or scale <= 0:
            scale = 1.0 / np.sqrt(D)
        dq = np.empty((N, Hq, D)); dk = np.empty((N, Hkv, D)); dv = np.empty((N, Hkv, D))
        dscore = np.empty(N); dgain = np.empty(Hq)
        self._lib.tgo_bias_attn_bwd(N, Hq, Hkv, D, _ptr(q), _ptr(k), _ptr(v), _ptr(key_score),
                                    _ptr(gain), _ptr(q_scale), float(scale),
                                    1 if causal else 0, _ptr(dout), _ptr(dq), _ptr(dk),
                                    _ptr(dv), _ptr(dscore), _ptr(dgain))
        return dq, dk, dv, dscore, dgain


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def num_threads() -> int:
    return default().num_threads()


def gate_score(*args, **kwargs):
    return default().gate_score(*args, **kwargs)


def topk_select(*args, **kwargs):
    return default().topk_select(*args, **kwargs)


def compact_gather(*args, **kwargs):
    return default().compact_gather(*args, **kwargs)


def kv_gather(*args, **kwargs):
    return default().kv_gather(*args, **kwargs)


def bias_attn(*args, **kwargs):
    return default().bias_attn(*args, **kwargs)


def bias_attn_bwd(*args, **kwargs):
    return default().bias_attn_bwd(*args, **kwargs)
