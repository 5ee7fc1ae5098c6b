"""Seeded synthetic inputs shaped like the workloads the bounded-generation engine
article describes (a Prefill-Only request of ~15 samples, long-prompt prefill
batches, short- and long-prompt beam search).

Recipe (the same for every consumer):
  * sequence lengths come from ``numpy.random.default_rng(seed)``:
    uniform integers (inclusive bounds) or round(exp(ln(median) + sigma * z)),
    clipped to the stated range;
  * tensor values come from a ``torch.Generator`` on the target device seeded
    with ``seed``, drawn as float32 N(0, 1) in the order q, k, v (prefill) or
    q, prefix_k, prefix_v, suffix_k, suffix_v (decode), multiplied by the
    stated standard deviation and rounded to bfloat16 (round to nearest even);
  * parent indices are uniform integers in [0, W) with replacement from
    ``numpy.random.default_rng(seed)``.

Large tensors are drawn on the GPU (drawing ~0.5 G normals on the host takes
minutes); host copies of the same buffers feed the oracle. Nothing here does any
attention, softmax, selection or reorder arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

# Named workloads: synthetic stand-ins with the shapes of the article's
# scenarios (its own business traffic and datasets are not public): a
# Prefill-Only request (15 sequences of 64..480 tokens, 28 layers), long
# packed prefill (lognormal lengths around 400, or 120 x 1024), short-prompt
# and long-prompt beam search.
CONFIGS = {
    "tiny_prefill": dict(kind="prefill", lengths=[5, 17, 40], nq=4, nkv=2, d=64, seed=0),
    "prefill_only": dict(kind="prefill", dist="uniform", n=15, lo=64, hi=480,
                         nq=16, nkv=8, d=128, seed=1, layers=28),
    "long_prefill": dict(kind="prefill", dist="lognormal", n=120, median=400.0, sigma=0.4,
                         lo=32, hi=1024, nq=14, nkv=2, d=64, seed=2),
    "long_prefill_1024": dict(kind="prefill", lengths=[1024] * 120, nq=14, nkv=2, d=64, seed=3),
    "short_decode": dict(kind="decode", r=32, lp=128, w=100, steps=4, ls_cap=4,
                         nq=16, nkv=8, d=64, seed=4),
    "long_beam": dict(kind="decode", r=8, lp=480, w=400, steps=5, ls_cap=5,
                      nq=16, nkv=8, d=128, seed=5, vocab=151936, logit_std=3.0),
    # the selective-FP8 SwiGLU requantisation over the Prefill-Only request's tokens; the pages give no model
    # dimensions, so the intermediate width is a synthetic 4096
    "swiglu_fp8": dict(kind="swiglu", tokens=4228, inter=4096, std=2.0, seed=6),
}


def lengths_uniform(n: int, lo: int, hi: int, seed: int) -> list[int]:
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def lengths_lognormal(n: int, median: float, sigma: float, lo: int, hi: int, seed: int) -> list[int]:
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(n)
    x = np.rint(np.exp(np.log(median) + sigma * z))
    return [int(v) for v in np.clip(x, lo, hi)]


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def bf16_normal(shape, gen: torch.Generator, device, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


@dataclass
class PrefillCase:
    lengths: list
    cu_seqlens: np.ndarray        # int32 [B+1]
    q: torch.Tensor               # bf16 [T, Nq, D]
    k: torch.Tensor               # bf16 [T, Nkv, D]
    v: torch.Tensor               # bf16 [T, Nkv, D]
    nq: int
    nkv: int
    d: int

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        return max(self.lengths) if self.lengths else 0


def prefill_lengths(cfg: dict) -> list[int]:
    if "lengths" in cfg:
        return list(cfg["lengths"])
    if cfg["dist"] == "uniform":
        return lengths_uniform(cfg["n"], cfg["lo"], cfg["hi"], cfg["seed"])
    return lengths_lognormal(cfg["n"], cfg["median"], cfg["sigma"], cfg["lo"], cfg["hi"], cfg["seed"])


def make_prefill_case(lengths, nq: int, nkv: int, d: int, seed: int, device="cpu") -> PrefillCase:
    cu = cu_seqlens_from_lengths(lengths)
    t = int(cu[-1])
    g = _gen(seed, device)
    q = bf16_normal((t, nq, d), g, device)
    k = bf16_normal((t, nkv, d), g, device)
    v = bf16_normal((t, nkv, d), g, device)
    return PrefillCase(list(lengths), cu, q, k, v, nq, nkv, d)


def make_named_prefill(name: str, device="cpu") -> PrefillCase:
    cfg = CONFIGS[name]
    return make_prefill_case(prefill_lengths(cfg), cfg["nq"], cfg["nkv"], cfg["d"], cfg["seed"], device)


@dataclass
class DecodeCase:
    q: torch.Tensor               # bf16 [R, W, Nq, D]
    prefix_k: torch.Tensor        # bf16 [R, Lp, Nkv, D]
    prefix_v: torch.Tensor
    suffix_k: torch.Tensor        # bf16 [R, W, Ls_cap, Nkv, D]
    suffix_v: torch.Tensor
    r: int
    w: int
    lp: int
    ls_cap: int
    nq: int
    nkv: int
    d: int


def make_decode_case(r, w, lp, ls_cap, nq, nkv, d, seed, device="cpu") -> DecodeCase:
    g = _gen(seed, device)
    q = bf16_normal((r, w, nq, d), g, device)
    pk = bf16_normal((r, lp, nkv, d), g, device)
    pv = bf16_normal((r, lp, nkv, d), g, device)
    sk = bf16_normal((r, w, ls_cap, nkv, d), g, device)
    sv = bf16_normal((r, w, ls_cap, nkv, d), g, device)
    return DecodeCase(q, pk, pv, sk, sv, r, w, lp, ls_cap, nq, nkv, d)


def make_named_decode(name: str, device="cpu") -> DecodeCase:
    c = CONFIGS[name]
    return make_decode_case(c["r"], c["w"], c["lp"], c["ls_cap"], c["nq"], c["nkv"], c["d"], c["seed"], device)


def make_parents(r: int, w_out: int, w_in: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, w_in, size=(r, w_out)).astype(np.int32)


def make_logits(r: int, w: int, vocab: int, std: float, seed: int, device="cpu") -> torch.Tensor:
    return bf16_normal((r, w, vocab), _gen(seed, device), device, std)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a (host) bfloat16 tensor as a uint16 array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
