"""The synthetic inputs follow their stated recipe (CPU only): seeded,
reproducible, with the sizes, bounds and value distributions of the named
workloads. These are the inputs both the kernels and the oracle receive."""
import numpy as np
import torch

import workloads as wl


def test_prefill_lengths_of_the_named_workloads():
    po = wl.prefill_lengths(wl.CONFIGS["prefill_only"])
    assert len(po) == 15 and min(po) >= 64 and max(po) <= 480 and sum(po) == 4228
    lp = wl.prefill_lengths(wl.CONFIGS["long_prefill"])
    assert len(lp) == 120 and min(lp) >= 32 and max(lp) <= 1024 and sum(lp) == 52348
    assert 340 <= np.median(lp) <= 460                       # lognormal around 400
    assert wl.prefill_lengths(wl.CONFIGS["long_prefill_1024"]) == [1024] * 120
    assert wl.prefill_lengths(wl.CONFIGS["tiny_prefill"]) == [5, 17, 40]
    assert po == wl.prefill_lengths(wl.CONFIGS["prefill_only"])   # seeded


def test_length_draws_follow_their_distributions():
    u = np.array(wl.lengths_uniform(20000, 64, 480, seed=7))
    assert u.min() == 64 and u.max() == 480 and abs(u.mean() - 272) < 3
    x = np.array(wl.lengths_lognormal(20000, 400.0, 0.4, 32, 1024, seed=7))
    assert x.min() >= 32 and x.max() <= 1024
    assert abs(np.median(x) - 400) < 8
    assert abs(np.std(np.log(x[(x > 32) & (x < 1024)])) - 0.4) < 0.02


def test_cu_seqlens_are_exclusive_prefix_sums():
    cu = wl.cu_seqlens_from_lengths([5, 0, 17, 40])
    assert cu.dtype == np.int32 and cu.tolist() == [0, 5, 5, 22, 62]


def test_values_are_seeded_bf16_normals():
    a = wl.make_prefill_case([300, 500], 4, 2, 64, seed=3)
    b = wl.make_prefill_case([300, 500], 4, 2, 64, seed=3)
    c = wl.make_prefill_case([300, 500], 4, 2, 64, seed=4)
    assert a.q.dtype == torch.bfloat16 and a.q.shape == (800, 4, 64) and a.k.shape == (800, 2, 64)
    assert torch.equal(a.q, b.q) and torch.equal(a.v, b.v) and not torch.equal(a.q, c.q)
    x = a.q.float()
    assert abs(x.mean().item()) < 0.02 and abs(x.std().item() - 1.0) < 0.02
    lg = wl.make_logits(2, 8, 20000, 3.0, seed=5).float()
    assert lg.shape == (2, 8, 20000) and abs(lg.std().item() - 3.0) < 0.03


def test_decode_case_shapes_and_parents():
    c = wl.make_decode_case(2, 5, 7, 3, 4, 2, 64, seed=1)
    assert c.q.shape == (2, 5, 4, 64) and c.prefix_k.shape == (2, 7, 2, 64)
    assert c.suffix_k.shape == (2, 5, 3, 2, 64) and c.suffix_v.dtype == torch.bfloat16
    p = wl.make_parents(4, 400, 400, seed=9)
    assert p.dtype == np.int32 and p.shape == (4, 400) and p.min() >= 0 and p.max() < 400
    assert len(np.unique(p[0])) < 400                        # drawn with replacement
