"""Packed causal GQA prefill on the GPU against the fp64 oracle.

Small cases are compared element by element in full. At the full workload
sizes the oracle recomputes a fixed subset of sequences (the oracle's per-
sequence independence is pinned on the CPU), always including the shortest and
longest, and the GPU's own invariants (sequence isolation, packed == separate
launches, run-to-run determinism) are checked on the whole batch.
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


def run_and_check(case, seqs=None, scale=None, name=""):
    q, k, v, cu = to_dev(case)
    say(f"[prefill] {name} T={case.total_tokens} B={len(case.lengths)} nq={case.nq} nkv={case.nkv} d={case.d}")
    out, lse = bga().packed_gqa_prefill(q, k, v, cu, case.max_seqlen, scale)
    torch.cuda.synchronize()
    scale = scale if scale is not None else 1.0 / np.sqrt(case.d)
    seqs = range(len(case.lengths)) if seqs is None else seqs
    emax = lmax = 0.0
    for i in seqs:
        s, n = int(case.cu_seqlens[i]), case.lengths[i]
        if n == 0:
            continue
        ro, rl = oracle.packed_prefill(case.q[s:s + n], case.k[s:s + n], case.v[s:s + n],
                                       np.array([0, n], np.int32), scale)
        emax = max(emax, check_bf16(out[s:s + n], ro, f"{name} seq {i} out"))
        lmax = max(lmax, check_lse(lse[s:s + n], rl, f"{name} seq {i} lse"))
    say(f"    max |out err| {emax:.2e}  max |lse err| {lmax:.2e}")
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


def subset(lengths, extra=4):
    order = np.argsort(lengths)
    pick = {int(order[0]), int(order[-1])}
    rng = np.random.default_rng(0)
    pick.update(int(i) for i in rng.choice(len(lengths), size=extra, replace=False))
    return sorted(pick)


def test_long_prefill_config_sampled():
    case = wl.make_named_prefill("long_prefill", device=DEV)
    case.q, case.k, case.v = case.q.cpu(), case.k.cpu(), case.v.cpu()
    run_and_check(case, seqs=subset(case.lengths), name="long_prefill")


def test_long_prefill_1024_sampled():
    case = wl.make_named_prefill("long_prefill_1024", device=DEV)
    case.q, case.k, case.v = case.q.cpu(), case.k.cpu(), case.v.cpu()
    run_and_check(case, seqs=[0, 57, 119], name="long_prefill_1024")


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
