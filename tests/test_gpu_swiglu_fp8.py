"""Fused SwiGLU + per-token E4M3 requantisation on the GPU against the oracle.

The kernel computes in fp32 (the article keeps SiLU * up, the amax reduction
and the scale in fp32), the oracle in fp64. The per-token scale must agree to
a few fp32 ulps. A code is an integer decided by floating point: wherever the
oracle's h / scale lies farther than 2e-6 (relative) from a rounding midpoint
between two E4M3 values, the GPU's code must equal the oracle's; within that
band either neighbour is correct (the count is printed). Rows built so that
every h / scale is exactly a midpoint (gate 32, where SiLU is the identity in
fp32, and up = midpoint / 32) check the hardware conversion's ties-to-even
directly, and an all-zero row gives zero codes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BAND = 2e-6


def bga():
    import attention_bga_packed_amd as m
    return m


def check(gate_up, name):
    codes, scale = bga().swiglu_quant_e4m3(gate_up)
    torch.cuda.synchronize()
    ref = oracle.swiglu_quant(gate_up.cpu())
    gs = scale.cpu().numpy().astype(np.float64)
    rel = np.abs(gs - ref["scale"]) / ref["scale"]
    assert rel.max() <= 4e-7, f"{name}: scale off by {rel.max():.2e}"
    x = ref["x"]
    lo, hi = oracle.e4m3_encode(x * (1 - BAND)), oracle.e4m3_encode(x * (1 + BAND))
    got = codes.cpu().numpy()
    unique = lo == hi
    assert np.array_equal(got[unique], ref["codes"][unique]), \
        f"{name}: {(got[unique] != ref['codes'][unique]).sum()} codes differ away from a rounding midpoint"
    assert np.all((got[~unique] == lo[~unique]) | (got[~unique] == hi[~unique])), f"{name}: code off a midpoint"
    say(f"    {name}: {got.size} codes, {int((~unique).sum())} within {BAND:g} of a midpoint "
        f"({int((got[~unique] != ref['codes'][~unique]).sum())} taken the other way); max scale error {rel.max():.1e}")
    return codes, scale


@pytest.mark.parametrize("t,i", [(7, 64), (33, 1000), (4228, 4096), (5, 16384), (1, 8)])
def test_random_rows(t, i):
    g = torch.Generator(device=DEV)
    g.manual_seed(t * 7 + i)
    say(f"[swiglu fp8] T={t} I={i}")
    check(wl.bf16_normal((t, 2 * i), g, DEV, 2.0), f"T={t} I={i}")


def test_exact_ties_and_zero_rows():
    vals = oracle.e4m3_decode([c for c in range(0x7F)])          # 0 .. 448, non-negative codes
    mids = (vals[:-1] + vals[1:]) / 2                               # every tie between neighbours
    i = 8 * ((len(mids) + 2 + 7) // 8)
    up = np.zeros(i)
    up[0] = 14.0                                                    # 32 * 14 = 448: amax, scale 1
    up[1:1 + len(mids)] = mids / 32
    rows = np.stack([np.concatenate([np.full(i, 32.0), up]), np.concatenate([np.full(i, 32.0), -up]),
                     np.zeros(2 * i)])
    gu = torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16)
    assert np.array_equal(gu.float().numpy(), rows)                 # every value exact in bf16
    codes, scale = bga().swiglu_quant_e4m3(gu.to(DEV))
    c = codes.cpu().numpy()
    want = oracle.e4m3_encode(rows[:2, i:] * 32)                    # exact ties: round to even
    assert np.array_equal(c[:2], want), np.flatnonzero(c[:2] != want)[:10]
    assert scale[0].item() == 1.0 and scale[1].item() == 1.0
    assert not (c[2] & 0x7F).any() and scale[2].item() == np.float32(1e-12) / np.float32(448)
