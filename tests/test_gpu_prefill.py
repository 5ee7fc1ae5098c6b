"""Packed causal GQA prefill on the GPU against the fp64 oracle.

Every case, the full-size workloads included (the 120-sequence lognormal batch
and the 120 x 1024 batch), is compared element by element against the oracle
over all of its sequences. Sequence isolation, packed == separate launches and
run-to-run determinism are checked on the GPU's own outputs for a six-sequence
batch of mixed lengths (d 64, group 7) and the tiny workload.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import check_bf16, check_lse, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bga():
    import attention_bga_packed_amd as m
    return m


def to_dev(case):
    cu = torch.from_numpy(case.cu_seqlens).to(DEV)
    return case.q.to(DEV), case.k.to(DEV), case.v.to(DEV), cu


def run_and_check(case, scale=None, name=""):
    """GPU prefill of the whole batch, then the oracle over every sequence, element by element."""
    q, k, v, cu = to_dev(case)
    say(f"[prefill] {name} T={case.total_tokens} B={len(case.lengths)} nq={case.nq} nkv={case.nkv} d={case.d}")
    out, lse = bga().packed_gqa_prefill(q, k, v, cu, case.max_seqlen, scale)
    torch.cuda.synchronize()
    scale = scale if scale is not None else 1.0 / np.sqrt(case.d)
    ro, rl = oracle.packed_prefill(case.q.cpu(), case.k.cpu(), case.v.cpu(), case.cu_seqlens, scale)
    emax = check_bf16(out, ro, f"{name} out")
    lmax = check_lse(lse, rl, f"{name} lse")
    say(f"    {len(case.lengths)} sequences: max |out err| {emax:.2e}  max |lse err| {lmax:.2e}")
    return out, lse


def test_tiny_config():
    case = wl.make_named_prefill("tiny_prefill")
    run_and_check(case, name="tiny")


@pytest.mark.parametrize("nq,nkv,d", [(4, 2, 64), (16, 8, 128), (14, 2, 64), (8, 8, 64), (16, 1, 128),
                                      (3, 1, 64), (12, 4, 128), (9, 1, 64)])
def test_boundary_lengths(nq, nkv, d):
    lengths = [1, 31, 32, 33, 0, 63, 64, 65, 127, 128, 129, 200, 0, 2]
    case = wl.make_prefill_case(lengths, nq, nkv, d, seed=100 + nq + d)
    run_and_check(case, name=f"boundary {nq}/{nkv}/{d}")


def test_single_long_sequence_and_scale():
    case = wl.make_prefill_case([777], 4, 2, 128, seed=7)
    run_and_check(case, scale=0.05, name="single 777 scale 0.05")


def test_prefill_only_config_full():
    case = wl.make_named_prefill("prefill_only")
    run_and_check(case, name="prefill_only")


def test_long_prefill_config_full():
    case = wl.make_named_prefill("long_prefill", device=DEV)
    run_and_check(case, name="long_prefill")


def test_long_prefill_1024_full():
    case = wl.make_named_prefill("long_prefill_1024", device=DEV)
    run_and_check(case, name="long_prefill_1024")


def test_sequence_isolation_and_separate_launches():
    case = wl.make_prefill_case([70, 5, 130, 64, 1, 99], 14, 2, 64, seed=3)
    q, k, v, cu = to_dev(case)
    out, lse = bga().packed_gqa_prefill(q, k, v, cu, case.max_seqlen)
    # separate launches, one sequence each
    for i, n in enumerate(case.lengths):
        s = int(case.cu_seqlens[i])
        cu1 = torch.tensor([0, n], dtype=torch.int32, device=DEV)
        o1, l1 = bga().packed_gqa_prefill(q[s:s + n].contiguous(), k[s:s + n].contiguous(), v[s:s + n].contiguous(),
                                          cu1, n)
        assert torch.equal(o1, out[s:s + n]) and torch.equal(l1, lse[s:s + n])
    # perturb sequence 2: every other row stays bit-identical
    s, n = int(case.cu_seqlens[2]), case.lengths[2]
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for t in (q2, k2, v2):
        t[s:s + n] = -t[s:s + n] * 0.5 + 0.25
    o2, l2 = bga().packed_gqa_prefill(q2, k2, v2, cu, case.max_seqlen)
    keep = torch.ones(case.total_tokens, dtype=torch.bool, device=DEV)
    keep[s:s + n] = False
    assert torch.equal(o2[keep], out[keep]) and torch.equal(l2[keep], lse[keep])
    assert not torch.equal(o2[~keep], out[~keep])


def test_determinism_and_guard_bands():
    case = wl.make_named_prefill("tiny_prefill")
    q, k, v, cu = to_dev(case)
    t, nq, d = q.shape
    guard = 4096
    buf = torch.full((t * nq * d + 2 * guard,), 12345, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    out = buf[guard:guard + t * nq * d].view(t, nq, d)
    lbuf = torch.full((t * nq + 2 * guard,), -7.0, dtype=torch.float32, device=DEV)
    lse = lbuf[guard:guard + t * nq].view(t, nq)
    bga().packed_gqa_prefill(q, k, v, cu, case.max_seqlen, out=out, lse=lse)
    o1, l1 = out.clone(), lse.clone()
    bga().packed_gqa_prefill(q, k, v, cu, case.max_seqlen, out=out, lse=lse)
    assert torch.equal(o1, out) and torch.equal(l1, lse)
    assert torch.all(buf[:guard].view(torch.int16) == 12345) and torch.all(buf[-guard:].view(torch.int16) == 12345)
    assert torch.all(lbuf[:guard] == -7.0) and torch.all(lbuf[-guard:] == -7.0)


def test_no_lse_and_empty_batch():
    case = wl.make_prefill_case([10, 20], 4, 2, 64, seed=9)
    q, k, v, cu = to_dev(case)
    out, lse = bga().packed_gqa_prefill(q, k, v, cu, 20, want_lse=False)
    assert lse is None
    ro, _ = oracle.packed_prefill(case.q, case.k, case.v, case.cu_seqlens)
    check_bf16(out, ro, "no-lse")
    # all sequences empty: nothing to do, nothing written
    cu0 = torch.zeros(4, dtype=torch.int32, device=DEV)
    e = torch.empty((0, 4, 64), dtype=torch.bfloat16, device=DEV)
    ek = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    bga().packed_gqa_prefill(e, ek, ek, cu0, 0)


@pytest.mark.parametrize("lengths,nq,nkv,d", [([8192, 5], 4, 2, 64), ([8192], 16, 1, 128)])
def test_longest_sequence_cap(lengths, nq, nkv, d):
    """Sequences at BGA_MAX_SEQLEN (8192 tokens), in full against the oracle."""
    case = wl.make_prefill_case(lengths, nq, nkv, d, seed=8192 + d, device=DEV)
    run_and_check(case, name=f"cap {lengths} {nq}/{nkv}/{d}")
