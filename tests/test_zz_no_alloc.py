"""bga_beam_topk_noalloc (the library's own per-device workspace, no allocation)
against bga_beam_topk (caller workspace) through the C-ABI: bit-identical
results on consecutive calls, the second and third smaller than the first, so
the shared workspace still holds the previous call's contents."""
import numpy as np
import pytest
import torch

import workloads as wl
from helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEYS = ("tokens", "parents", "scores", "local_tokens", "local_scores", "row_lse")


def bga():
    import attention_bga_packed_amd as m
    return m


def outputs(r, w_in, k_local, k_global):
    return {"tokens": torch.full((r, k_global), -5, dtype=torch.int32, device=DEV),
            "parents": torch.full((r, k_global), -5, dtype=torch.int32, device=DEV),
            "scores": torch.full((r, k_global), 7.0, dtype=torch.float32, device=DEV),
            "local_tokens": torch.full((r, w_in, k_local), -5, dtype=torch.int32, device=DEV),
            "local_scores": torch.full((r, w_in, k_local), 7.0, dtype=torch.float32, device=DEV),
            "row_lse": torch.full((r, w_in), 7.0, dtype=torch.float32, device=DEV)}


def test_noalloc_matches_workspace_entry_point():
    cases = [
        # (R, W_in, V, std, k_local, k_global, seed): the long-prompt step first, then smaller ones
        (8, 400, 151936, 3.0, 800, 400, 41),
        (3, 50, 30000, 3.0, 100, 50, 42),
        (2, 5, 333, 1.0, 10, 5, 43),
    ]
    for r, w_in, v, std, kl, kg, seed in cases:
        say(f"[noalloc] R={r} W_in={w_in} V={v} k_local={kl} k_global={kg}")
        x = wl.make_logits(r, w_in, v, std, seed=seed, device=DEV)
        cum = torch.from_numpy((np.random.default_rng(seed).standard_normal((r, w_in)) - 3).astype(np.float32)).to(DEV)
        ref = bga().beam_topk(x, cum, kl, kg, want_local=True, want_lse=True)
        out = outputs(r, w_in, kl, kg)
        torch.cuda.synchronize()
        got = bga().beam_topk_noalloc(x, cum, kl, kg, out=out, want_local=True, want_lse=True)
        torch.cuda.synchronize()
        assert got is out
        for key in KEYS:
            assert torch.equal(got[key], ref[key]), key
        say("    identical")


def test_noalloc_rejects_sizes_beyond_its_workspace():
    x = torch.zeros((8, 512, 8), dtype=torch.bfloat16, device=DEV)
    out = outputs(8, 512, 8, 8)
    with pytest.raises(ValueError):
        bga().beam_topk_noalloc(x, None, 8, 8, out={"tokens": out["tokens"]})   # outputs must be passed
    x = wl.make_logits(8, 512, 1024, 1.0, seed=1, device=DEV)
    out = outputs(8, 512, 1024, 1024)
    with pytest.raises(bga().BgaError) as e:
        bga().beam_topk_noalloc(x, None, 1024, 1024, out=out)
    assert e.value.status == 5
