"""The measurement baselines (comparators/) compute the same attention as the
oracle: explicit padded and block-diagonal packed Torch prefill, per-beam full
K/V Torch decode. They use bf16 score products (the usual explicit form), so
their bound is looser than the kernels' (3e-2); the error is what it is, the
semantics must match."""
import numpy as np
import pytest
import torch

import comparators as C
import oracle
import workloads as wl

TOL = 3e-2


@pytest.mark.parametrize("lengths,nq,nkv,d", [([5, 17, 40, 1], 4, 2, 64), ([64, 3, 100], 14, 2, 64),
                                              ([9, 33], 8, 8, 128)])
def test_prefill_comparators_on_cpu(lengths, nq, nkv, d):
    c = wl.make_prefill_case(lengths, nq, nkv, d, 0)
    sc = 1 / np.sqrt(d)
    ro, _ = oracle.packed_prefill(c.q, c.k, c.v, c.cu_seqlens)
    o1 = C.padded_prefill(c.q, c.k, c.v, lengths, sc)
    o2 = C.packed_prefill(c.q, c.k, c.v, torch.from_numpy(c.cu_seqlens), sc)
    assert np.abs(o1.float().numpy() - ro).max() < TOL
    assert np.abs(o2.float().numpy() - ro).max() < TOL


@pytest.mark.parametrize("r,w,lp,ls,nq,nkv,d", [(2, 5, 33, 2, 4, 2, 64), (1, 3, 70, 3, 16, 8, 128)])
def test_per_beam_decode_comparator_on_cpu(r, w, lp, ls, nq, nkv, d):
    c = wl.make_decode_case(r, w, lp, 3, nq, nkv, d, 1)
    kt, vf = C.per_beam_kv(c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, ls)
    o = C.per_beam_decode(c.q, kt, vf, 1 / np.sqrt(d))
    ro, _ = oracle.shared_prefix_decode(c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, ls)
    assert np.abs(o.float().numpy() - ro).max() < TOL
    # the packed per-beam copies: beam (r, b) holds rows [prompt of r; suffix of (r, b)]
    pk, _ = C.per_beam_kv_packed(c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, ls)
    n = lp + ls
    for rr in range(r):
        for b in range(w):
            want = torch.cat([c.prefix_k[rr], c.suffix_k[rr, b, :ls]])
            assert torch.equal(pk[(rr * w + b) * n:(rr * w + b + 1) * n], want)


@pytest.mark.gpu
def test_comparators_on_the_gpu():
    """The same checks at workload sizes on the GPU, where the bench times them."""
    dev = "cuda:0"
    c = wl.make_named_prefill("prefill_only", device=dev)
    ro, _ = oracle.packed_prefill(c.q.cpu(), c.k.cpu(), c.v.cpu(), c.cu_seqlens)
    o1 = C.padded_prefill(c.q, c.k, c.v, c.lengths, 1 / np.sqrt(c.d))
    o2 = C.packed_prefill(c.q, c.k, c.v, torch.from_numpy(c.cu_seqlens).to(dev), 1 / np.sqrt(c.d))
    assert np.abs(o1.float().cpu().numpy() - ro).max() < TOL
    assert np.abs(o2.float().cpu().numpy() - ro).max() < TOL
    d = wl.make_decode_case(2, 400, 480, 5, 16, 8, 128, seed=5, device=dev)
    kt, vf = C.per_beam_kv(d.prefix_k, d.prefix_v, d.suffix_k, d.suffix_v, 5)
    o = C.per_beam_decode(d.q, kt, vf, 1 / np.sqrt(128))
    host = [t.cpu() for t in (d.q, d.prefix_k, d.prefix_v, d.suffix_k, d.suffix_v)]
    r3, _ = oracle.shared_prefix_decode(*host, 5)
    assert np.abs(o.float().cpu().numpy() - r3).max() < TOL
