"""Shared test helpers: tolerances and host/device conversions."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Acceptance for bf16 outputs against the fp64 oracle: max-abs 1e-2, widened to
# one bf16 ulp of the reference where that ulp is larger (|ref| >= 4, where even
# a correctly rounded bf16 value can be 1/2 ulp = 0.0156 away).
BF16_ABS_TOL = 1e-2
LSE_ABS_TOL = 1e-3


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(a)) - 7)


def check_bf16(got: torch.Tensor, ref: np.ndarray, name: str):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    err = np.abs(g - ref)
    tol = np.maximum(BF16_ABS_TOL, bf16_ulp(ref))
    bad = err > tol
    assert not bad.any(), (f"{name}: {bad.sum()} elements out of tolerance; max err {err.max():.3e} at "
                           f"{np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max())


def check_lse(got: torch.Tensor, ref: np.ndarray, name: str):
    g = got.detach().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    assert err.max() <= LSE_ABS_TOL, f"{name}: lse max err {err.max():.3e}"
    return float(err.max())


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
