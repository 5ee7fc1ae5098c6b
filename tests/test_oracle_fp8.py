"""Pins for the oracle's selective-FP8 requantisation (article section 3.4), CPU.

  * the E4M3 encoder equals torch's float8_e4m3fn conversion (round to nearest
    even) on every representable value, every midpoint between neighbours
    (ties), and random values inside the finite range; encode(decode(c)) == c;
  * SwiGLU: h equals gate * scipy's expit(gate) * up; gate = 0 gives 0; an
    all-zero row gives zero codes; the row's largest |h| maps to +-448;
    every code is within half an E4M3 step of h / scale.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import workloads as wl

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def torch_e4m3(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_known_values():
    assert oracle.e4m3_decode([0x7E, 0xFE, 0x38, 0x01, 0x08, 0x00])[:5].tolist() == [448.0, -448.0, 1.0, 2.0 ** -9,
                                                                                     2.0 ** -6]
    assert np.isnan(oracle.e4m3_decode([0x7F])[0])


def test_encode_matches_torch_on_codes_midpoints_and_random():
    vals = oracle.e4m3_decode(FINITE)
    # every representable value round-trips (-0 keeps its sign bit)
    assert np.array_equal(oracle.e4m3_encode(vals), np.array(FINITE, np.uint8))
    pos = np.sort(np.unique(np.abs(vals)))
    mids = (pos[:-1] + pos[1:]) / 2               # exact ties: nearest even must win
    rnd = np.random.default_rng(0).uniform(-460, 460, 20000)
    small = np.random.default_rng(1).uniform(-0.05, 0.05, 20000)
    x = np.concatenate([vals, mids, -mids, rnd, small]).astype(np.float32).astype(np.float64)
    assert np.array_equal(oracle.e4m3_encode(x), torch_e4m3(x))


def test_encode_saturates_above_448():
    assert oracle.e4m3_encode([463.99, 464.0, 1e6, -1e6]).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


def gate_up(t, i, seed, std=2.0):
    g = torch.Generator().manual_seed(seed)
    return wl.bf16_normal((t, 2 * i), g, "cpu", std)


def test_swiglu_against_expit_and_codes_within_half_step():
    x = gate_up(9, 320, 3)
    r = oracle.swiglu_quant(x)
    f = x.double().numpy()
    g, u = f[:, :320], f[:, 320:]
    h = g * expit(g) * u
    assert np.allclose(r["h"], h, rtol=1e-14, atol=1e-300)
    amax = np.abs(h).max(1)
    assert np.allclose(r["scale"], amax / 448, rtol=1e-15)
    assert np.array_equal(r["x"], r["h"] / r["scale"][:, None])
    # the largest |h| of each row is +-448
    j = np.abs(h).argmax(1)
    assert set(r["codes"][np.arange(9), j].tolist()) <= {0x7E, 0xFE}
    # every code within half a step of h / scale
    dec = oracle.e4m3_decode(r["codes"])
    step = np.where(np.abs(r["x"]) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r["x"]),
                                                                                              1e-300))) - 3))
    assert np.all(np.abs(dec - r["x"]) <= step / 2 + 1e-12)


def test_swiglu_zero_gate_and_zero_rows():
    x = gate_up(3, 64, 4)
    x[0, :64] = 0.0                    # gate 0: SiLU(0) = 0
    x[1] = 0.0                         # the whole row
    r = oracle.swiglu_quant(x)
    # zero, with the sign of gate * up (-0 encodes as 0x80)
    assert not r["h"][0].any() and not (r["codes"][:2] & 0x7F).any()
    assert r["scale"][1] == 1e-12 / 448
