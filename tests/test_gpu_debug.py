"""The debug library (libbga_debug.so) on the GPU: device-side preconditions.

Each bad input is caught by the debug build's check kernel, which reads only
inside the host-validated extents; the entry point then returns
BGA_ERR_PRECONDITION with the matching violation bit and launches nothing. On
good inputs the debug build's results are bit-identical to the release build's.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CU, MAXLEN, PARENT, LOGITS = 1, 2, 4, 8   # BGA_VIOLATION_* bits


@pytest.fixture()
def dbg(monkeypatch):
    """The package's entry points routed through the debug library."""
    import attention_bga_packed_amd as m
    from attention_bga_packed_amd import _binding
    lib = _binding.load_library(_binding.DEBUG_LIB_PATH)
    assert lib.bga_debug_build() == 1
    monkeypatch.setattr(_binding, "lib", lib)
    return m


def expect_violation(fn, bits):
    import attention_bga_packed_amd as m
    with pytest.raises(m.BgaError) as e:
        fn()
    assert e.value.status == 8, e.value
    from attention_bga_packed_amd import _binding
    assert _binding.lib.bga_last_violations() == bits, hex(_binding.lib.bga_last_violations())


def prefill_inputs(lengths, nq=4, nkv=2, d=64, seed=1):
    c = wl.make_prefill_case(lengths, nq, nkv, d, seed)
    return c, c.q.to(DEV), c.k.to(DEV), c.v.to(DEV)


def test_prefill_preconditions(dbg):
    say("[debug] prefill: non-monotone cu_seqlens, cu[B] != T, a sequence longer than max_seqlen")
    c, q, k, v = prefill_inputs([10, 30, 5])
    bad_cu = torch.tensor([0, 10, 5, 45], dtype=torch.int32, device=DEV)
    expect_violation(lambda: dbg.packed_gqa_prefill(q, k, v, bad_cu, 40), CU)
    short_end = torch.tensor([0, 10, 40, 44], dtype=torch.int32, device=DEV)
    expect_violation(lambda: dbg.packed_gqa_prefill(q, k, v, short_end, 30), CU)
    cu = torch.from_numpy(c.cu_seqlens).to(DEV)
    expect_violation(lambda: dbg.packed_gqa_prefill(q, k, v, cu, 16), MAXLEN)
    nonzero_start = torch.tensor([2, 10, 40, 45], dtype=torch.int32, device=DEV)
    expect_violation(lambda: dbg.packed_gqa_prefill(q, k, v, nonzero_start, 8), CU | MAXLEN)
    # good input: bit-identical to the release build
    out_d, lse_d = dbg.packed_gqa_prefill(q, k, v, cu, 30)
    from attention_bga_packed_amd import _binding
    rel = _binding.load_library(_binding.RELEASE_LIB_PATH)
    import attention_bga_packed_amd as m
    _binding.lib, saved = rel, _binding.lib
    try:
        out_r, lse_r = m.packed_gqa_prefill(q, k, v, cu, 30)
    finally:
        _binding.lib = saved
    assert torch.equal(out_d, out_r) and torch.equal(lse_d, lse_r)


def test_reorder_preconditions(dbg):
    say("[debug] reorder: parents outside [0, W)")
    c = wl.make_decode_case(2, 4, 3, 2, 4, 2, 64, seed=3)
    sk, sv = c.suffix_k.to(DEV), c.suffix_v.to(DEV)
    for bad in (4, -1, 1 << 30):
        par = torch.tensor([[0, 1, 2, 3], [3, 2, bad, 0]], dtype=torch.int32, device=DEV)
        dk = torch.full_like(sk, 7.0)
        expect_violation(lambda: dbg.suffix_reorder(sk, sv, par, 2, dst_k=dk), PARENT)
        assert torch.all(dk == 7.0)   # nothing launched, nothing written
    par = torch.tensor([[3, 3, 0, 1], [2, 2, 2, 0]], dtype=torch.int32, device=DEV)
    dk, dv = dbg.suffix_reorder(sk, sv, par, 2)
    assert torch.equal(dk[:, :, :2], sk[torch.arange(2)[:, None], par.cpu().long()][:, :, :2])


def test_topk_preconditions(dbg):
    say("[debug] top-K: an inf and a NaN logit")
    x = wl.make_logits(2, 3, 5000, 3.0, seed=4).to(DEV)
    for val in (float("inf"), float("-inf"), float("nan")):
        xb = x.clone()
        xb[1, 2, 4321] = val
        expect_violation(lambda: dbg.beam_topk(xb, None, 10, 5), LOGITS)
    r = dbg.beam_topk(x, None, 10, 5, want_local=True)
    import oracle
    ref = oracle.beam_topk(x.cpu(), None, 10, 5)
    assert np.array_equal(r["local_tokens"].cpu().numpy(), ref["local_tokens"])


def test_packed_prompt_preconditions(dbg):
    say("[debug] packed prompts: bad offsets, an empty prompt without a suffix")
    c = wl.make_decode_case(3, 4, 1, 2, 4, 2, 64, seed=6, device=DEV)
    pk = torch.zeros((20, 2, 64), dtype=torch.bfloat16, device=DEV)
    bad = torch.tensor([0, 12, 8, 20], dtype=torch.int32, device=DEV)
    expect_violation(lambda: dbg.shared_prefix_decode_packed(c.q, pk, pk, bad, c.suffix_k, c.suffix_v, 1), CU)
    empty = torch.tensor([0, 12, 12, 20], dtype=torch.int32, device=DEV)
    expect_violation(lambda: dbg.shared_prefix_decode_packed(c.q, pk, pk, empty, c.suffix_k, c.suffix_v, 0), 16)
    dbg.shared_prefix_decode_packed(c.q, pk, pk, empty, c.suffix_k, c.suffix_v, 1)   # a suffix to attend to: fine
    x = torch.zeros((20, 8), dtype=torch.float32, device=DEV)
    expect_violation(lambda: dbg.last_token_gather(x, bad), CU)
