"""Shared test helpers: tolerances and host/device conversions."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Acceptance for bf16 outputs against the fp64 oracle: max-abs 1e-2. Only where
# |ref| >= 4 is the bound one bf16 ulp of the reference instead (there half an
# ulp is already 0.0156, so even a correctly rounded bf16 value can miss 1e-2;
# below 4 half an ulp is at most 0.0078 and 1e-2 holds as it stands).
BF16_ABS_TOL = 1e-2
BF16_WIDEN_FROM = 4.0
LSE_ABS_TOL = 1e-3


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(a)) - 7)


def bf16_tolerance(ref: np.ndarray) -> np.ndarray:
    """Per-element bound on |got - ref| for a bf16 output whose fp64 reference is `ref`."""
    ref = np.asarray(ref, np.float64)
    return np.where(np.abs(ref) >= BF16_WIDEN_FROM, np.maximum(BF16_ABS_TOL, bf16_ulp(ref)), BF16_ABS_TOL)


def check_bf16(got: torch.Tensor, ref: np.ndarray, name: str):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    err = np.abs(g - ref)
    bad = err > bf16_tolerance(ref)
    assert not bad.any(), (f"{name}: {bad.sum()} elements out of tolerance; max err {err.max():.3e} at "
                           f"{np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max())


def check_lse(got: torch.Tensor, ref: np.ndarray, name: str):
    g = got.detach().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    assert err.max() <= LSE_ABS_TOL, f"{name}: lse max err {err.max():.3e}"
    return float(err.max())


def f32_ordinal(x: np.ndarray) -> np.ndarray:
    """fp32 values mapped to integers whose differences count representable fp32 steps (ulps); -0 == +0."""
    b = np.ascontiguousarray(x, np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF), b)


def f32_ulp_gap(a, b) -> np.ndarray:
    """Number of fp32 steps between a and b (0 when equal)."""
    return np.abs(f32_ordinal(np.asarray(a, np.float32)) - f32_ordinal(np.asarray(b, np.float32)))


CUT_GAP_ULP = 4


def f32_ulp(x) -> np.ndarray:
    """Spacing of fp32 values at |x| (the distance to the next fp32 value away from zero)."""
    a = np.abs(np.asarray(x, np.float32))
    return (np.nextafter(a, np.float32(np.inf)) - a).astype(np.float64)


def cut_gap(got: dict, ref: dict, i: int, k_local: int, k_global: int):
    """Request i of a beam top-K whose selection differs from the oracle's (computed with the oracle's own row
    log-sum-exp). A score s = cum + (x - lse) inherits the log-sum-exp's rounding at the log-sum-exp's
    magnitude, so distances are counted in fp32 ulps at max(|s|, |row lse|). Returns (gap, drift): the largest
    distance between the oracle's k_global-th score and the oracle score of any candidate that only one side
    selects, and the largest distance between a candidate's two stage-1 scores. `got` and `ref` hold numpy
    arrays (tokens, parents, scores [R, k_global]; local_tokens, local_scores [R, W_in, k_local]; ref also
    row_lse [R, W_in]); stage-1 ids must be identical."""
    lt = ref["local_tokens"][i]
    assert np.array_equal(got["local_tokens"][i], lt)
    so = ref["local_scores"][i].ravel().astype(np.float64)   # oracle scores by flat index f = b * k_local + j
    sg = got["local_scores"][i].ravel().astype(np.float64)
    lse = np.repeat(np.abs(ref["row_lse"][i]), k_local)        # the row lse of every flat index
    unit = f32_ulp(np.maximum(np.abs(so), lse))
    drift = float((np.abs(sg - so) / unit).max())

    def flat(tokens, parents):
        return np.array([p * k_local + int(np.flatnonzero(lt[p] == t)[0]) for t, p in zip(tokens, parents)])

    fg = flat(got["tokens"][i], got["parents"][i])
    fo = flat(ref["tokens"][i], ref["parents"][i])
    assert np.array_equal(so[fo], ref["scores"][i])
    cut = float(ref["scores"][i][k_global - 1])
    diff = np.setxor1d(fg, fo)
    gap = float((np.abs(so[diff] - cut) / unit[diff]).max()) if diff.size else 0.0
    return gap, drift


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
