"""The Python binding rejects caller-provided tensors of the wrong shape, dtype or
device before anything reaches the library (an undersized output would otherwise
be written past its end)."""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bga():
    import attention_bga_packed_amd as m
    return m


def test_prefill_output_shapes():
    c = wl.make_prefill_case([5, 9], 4, 2, 64, seed=1)
    q, k, v = c.q.to(DEV), c.k.to(DEV), c.v.to(DEV)
    cu = torch.from_numpy(c.cu_seqlens).to(DEV)
    with pytest.raises(ValueError):
        bga().packed_gqa_prefill(q, k, v, cu, 9, out=torch.empty((13, 4, 64), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        bga().packed_gqa_prefill(q, k, v, cu, 9, lse=torch.empty((14, 3), dtype=torch.float32, device=DEV))
    with pytest.raises(TypeError):
        bga().packed_gqa_prefill(q, k, v, cu, 9, lse=torch.empty((14, 4), dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):
        bga().packed_gqa_prefill(q, k, v, cu, 9, out=torch.empty((14, 4, 64), dtype=torch.bfloat16))


def test_decode_output_shapes():
    c = wl.make_decode_case(2, 3, 8, 2, 4, 2, 64, seed=2)
    args = [t.to(DEV) for t in (c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v)]
    with pytest.raises(ValueError):
        bga().shared_prefix_decode(*args, 1, out=torch.empty((2, 3, 4, 32), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        bga().shared_prefix_decode(*args, 1, lse=torch.empty((2, 3), dtype=torch.float32, device=DEV))


def test_reorder_shapes():
    c = wl.make_decode_case(2, 3, 8, 2, 4, 2, 64, seed=2)
    sk, sv = c.suffix_k.to(DEV), c.suffix_v.to(DEV)
    par = torch.zeros((2, 3), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        bga().suffix_reorder(sk, sv, torch.zeros((2, 2), dtype=torch.int32, device=DEV), 1)
    with pytest.raises(ValueError):
        bga().suffix_reorder(sk, sv, par, 1, dst_k=torch.empty((2, 3, 1, 2, 64), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        bga().suffix_reorder(sk, sv[:, :2].contiguous(), par, 1)
    tok = torch.zeros((2, 3, 4), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        bga().suffix_reorder(sk, sv, par, 1, src_tokens=tok, dst_tokens=torch.zeros((2, 3, 2), dtype=torch.int32,
                                                                                       device=DEV), num_tokens=1)
    with pytest.raises(ValueError):
        bga().suffix_reorder(sk, sv, par, 1, dst_tokens=tok)


def test_topk_shapes():
    x = wl.make_logits(2, 3, 1000, 3.0, seed=5).to(DEV)
    with pytest.raises(ValueError):
        bga().beam_topk(x, torch.zeros((2, 4), dtype=torch.float32, device=DEV), 8, 4)
    with pytest.raises(ValueError):
        bga().beam_topk(x, None, 8, 4, out={"tokens": torch.empty((2, 3), dtype=torch.int32, device=DEV)})
    with pytest.raises(TypeError):
        bga().beam_topk(x, None, 8, 4, out={"scores": torch.empty((2, 4), dtype=torch.float64, device=DEV)})
    with pytest.raises(ValueError):
        bga().beam_topk(x, None, 8, 4, out={"row_lse": torch.empty((2,), dtype=torch.float32, device=DEV)})
    with pytest.raises(ValueError):
        bga().beam_topk(x, None, 8, 4, out={"bogus": torch.empty(1, device=DEV)})
    r = bga().beam_topk(x, None, 8, 4)
    assert r["tokens"].shape == (2, 4)
