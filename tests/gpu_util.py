"""Helpers shared by the GPU tests: host <-> device marshalling of the seeded
inputs, tolerances, and an optional JSON-lines report of observed errors."""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np
import torch

# Tolerances.  fp32 path: |gpu - ref| <= 1e-5 * max(1, |ref|) elementwise.
# bf16 path: max |gpu - ref| <= 2e-2 for gate scores and attention outputs
# (inputs are exact bf16 values, products accumulate in fp32; the attention
# rounds P and O to bf16, each a relative 2^-9 step).
F32_REL = 1e-5
BF16_ABS = 2e-2
LSE_ABS_BF16 = 2e-2


def dev():
    return torch.device("cuda", 0)


def to_dev(a, dtype: str | None = None):
    """numpy -> device tensor; uint16 arrays with dtype='bf16' become bf16."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(a).to(dev())


def bf16_bits(t) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def as_f64(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().float().cpu().numpy().astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def report(name, **kv):
    """Print (and optionally append to $TG_PARITY_REPORT) observed errors."""
    kv = {k: (float(v) if isinstance(v, (np.floating, float)) else v) for k, v in kv.items()}
    line = json.dumps(dict(test=name, **kv))
    print(line)
    sys.stdout.flush()
    path = os.environ.get("TG_PARITY_REPORT")
    if path:
        os.makedirs(os.path.dirname(path) or ".", exist_ok=True)
        with open(path, "a") as f:
            f.write(line + "\n")


def assert_close_f32(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bound = F32_REL * np.maximum(1.0, np.abs(ref))
    finite = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), finite), what + ": non-finite mismatch"
    worst = float(np.max((err / bound)[finite])) if finite.any() else 0.0
    report(what, max_abs=float(np.max(err[finite])) if finite.any() else 0.0,
           worst_ratio_to_tol=worst)
    assert worst <= 1.0, "%s: error %.3g x tolerance" % (what, worst)


def assert_close_abs(got, ref, tol, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), finite), what + ": non-finite mismatch"
    err = np.abs(got - ref)[finite]
    mx = float(err.max()) if err.size else 0.0
    report(what, max_abs=mx, mean_abs=float(err.mean()) if err.size else 0.0, tol=tol)
    assert mx <= tol, "%s: max |diff| %.3g > %.3g" % (what, mx, tol)


class Timer:
    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        self.s = time.time() - self.t
