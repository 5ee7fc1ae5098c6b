"""Shared-prefix beam decode and parent-index reorder on the GPU against the oracle."""
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


def dev(c):
    return [t.to(DEV) for t in (c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v)]


def check_decode(c, ls, name, scale=None):
    """GPU decode of every request, then the oracle over every request, beam and head, element by element."""
    q, pk, pv, sk, sv = dev(c)
    say(f"[decode] {name} R={c.r} W={c.w} Lp={c.lp} Ls={ls}/{c.ls_cap} nq={c.nq} nkv={c.nkv} d={c.d}")
    out, lse = bga().shared_prefix_decode(q, pk, pv, sk, sv, ls, scale)
    torch.cuda.synchronize()
    host = [t.cpu() for t in (c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v)]
    ro, rl = oracle.shared_prefix_decode(*host, ls, scale)
    e = check_bf16(out, ro, f"{name} out")
    l = check_lse(lse, rl, f"{name} lse")
    say(f"    max |out err| {e:.2e}  max |lse err| {l:.2e}")
    return out, lse


@pytest.mark.parametrize("ls", [1, 2, 3, 4])
def test_short_decode_config(ls):
    c = wl.make_named_decode("short_decode")
    check_decode(c, ls, "short_decode")


@pytest.mark.parametrize("ls", [1, 2, 3, 4, 5])
def test_long_beam_decode_config_full(ls):
    c = wl.make_named_decode("long_beam", device=DEV)
    check_decode(c, ls, "long_beam")


@pytest.mark.parametrize("r,w,lp,ls,cap,nq,nkv,d", [
    (2, 3, 0, 2, 3, 4, 2, 64),       # suffix only
    (2, 5, 7, 0, 2, 4, 2, 64),       # prefix only, ragged prefix tile
    (1, 1, 65, 1, 1, 8, 8, 128),     # one beam, MHA
    (3, 70, 130, 3, 4, 14, 2, 64),   # W*G not a multiple of 128
    (2, 9, 64, 2, 2, 16, 1, 128),    # group 16
    (1, 33, 1, 1, 1, 3, 1, 64),      # prefix of one token
    (2, 100, 70, 3, 4, 8, 8, 64),    # group 1: up to 128 beams per workgroup (suffix rows in two slots)
    (1, 130, 64, 2, 2, 4, 4, 128),   # group 1, a full and a ragged workgroup, one prompt tile
    (2, 512, 100, 16, 16, 16, 8, 64),   # the caps: 512 beams, 16 suffix positions
    (1, 512, 33, 16, 16, 4, 4, 128),    # the caps with group 1 (128 beams per workgroup)
])
def test_decode_edge_shapes(r, w, lp, ls, cap, nq, nkv, d):
    c = wl.make_decode_case(r, w, lp, cap, nq, nkv, d, seed=r * 1000 + w + lp)
    check_decode(c, ls, f"edge r{r} w{w} lp{lp} ls{ls}", scale=0.11)


def test_decode_equals_causal_prefill_last_row():
    """Decode over [prefix; suffix_b] vs the GPU's own causal prefill of that
    sequence with q_b at the last position (two different kernels)."""
    c = wl.make_decode_case(1, 4, 90, 3, 4, 2, 64, seed=5)
    ls = 3
    q, pk, pv, sk, sv = dev(c)
    out, lse = bga().shared_prefix_decode(q, pk, pv, sk, sv, ls)
    for b in range(c.w):
        n = c.lp + ls
        kk = torch.cat([pk[0], sk[0, b, :ls]]).contiguous()
        vv = torch.cat([pv[0], sv[0, b, :ls]]).contiguous()
        qq = torch.zeros((n, c.nq, c.d), dtype=torch.bfloat16, device=DEV)
        qq[-1] = q[0, b]
        cu = torch.tensor([0, n], dtype=torch.int32, device=DEV)
        op, lp_ = bga().packed_gqa_prefill(qq, kk, vv, cu, n)
        assert (op[-1].float() - out[0, b].float()).abs().max() <= 1e-2
        assert (lp_[-1] - lse[0, b]).abs().max() <= 1e-4


def test_decode_determinism_and_beam_permutation():
    c = wl.make_decode_case(2, 37, 100, 2, 4, 2, 64, seed=8)
    q, pk, pv, sk, sv = dev(c)
    o1, l1 = bga().shared_prefix_decode(q, pk, pv, sk, sv, 2)
    o2, l2 = bga().shared_prefix_decode(q, pk, pv, sk, sv, 2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    perm = torch.randperm(c.w, generator=torch.Generator().manual_seed(1)).to(DEV)
    o3, l3 = bga().shared_prefix_decode(q[:, perm].contiguous(), pk, pv, sk[:, perm].contiguous(),
                                        sv[:, perm].contiguous(), 2)
    assert torch.equal(o3, o1[:, perm]) and torch.equal(l3, l1[:, perm])


# ---------------------------------------------------------------- reorder

def test_reorder_at_the_caps():
    """512 beams, 16 suffix positions (BGA_MAX_BEAMS, BGA_MAX_SUFFIX), with token history."""
    c = wl.make_decode_case(2, 512, 1, 16, 16, 8, 128, seed=512)
    parent = wl.make_parents(2, 512, 512, seed=513)
    tok = np.random.default_rng(514).integers(0, 151936, (2, 512, 16)).astype(np.int32)
    dk, dv, dt = bga().suffix_reorder(c.suffix_k.to(DEV), c.suffix_v.to(DEV), torch.from_numpy(parent).to(DEV), 16,
                                      src_tokens=torch.from_numpy(tok).to(DEV), num_tokens=16)
    rk, rv, rt = oracle.suffix_reorder(c.suffix_k, c.suffix_v, parent, 16, tok, 16)
    assert np.array_equal(wl.bf16_bits(dk.cpu()), rk) and np.array_equal(wl.bf16_bits(dv.cpu()), rv)
    assert np.array_equal(dt.cpu().numpy(), rt)


@pytest.mark.parametrize("name,ls", [("short_decode", 4), ("long_beam", 5), ("long_beam", 1)])
def test_reorder_config_bit_exact(name, ls):
    cfg = wl.CONFIGS[name]
    c = wl.make_named_decode(name, device=DEV)
    parent = wl.make_parents(cfg["r"], cfg["w"], cfg["w"], seed=cfg["seed"] + 10 * ls)
    tok = torch.from_numpy(np.random.default_rng(ls).integers(0, 151936, (cfg["r"], cfg["w"], 8)).astype(np.int32))
    say(f"[reorder] {name} Ls={ls}")
    pdev = torch.from_numpy(parent).to(DEV)
    dk = torch.full_like(c.suffix_k, 3.0)
    dv = torch.full_like(c.suffix_v, 3.0)
    dk, dv, dt = bga().suffix_reorder(c.suffix_k, c.suffix_v, pdev, ls, dst_k=dk, dst_v=dv,
                                      src_tokens=tok.to(DEV), num_tokens=ls)
    rk, rv, rt = oracle.suffix_reorder(c.suffix_k.cpu(), c.suffix_v.cpu(), parent, ls, tok.numpy(), ls)
    gk = dk.cpu().view(torch.int16).numpy().view(np.uint16)
    gv = dv.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gk[:, :, :ls], rk[:, :, :ls]) and np.array_equal(gv[:, :, :ls], rv[:, :, :ls])
    # positions >= suffix_len untouched
    assert torch.all(dk[:, :, ls:] == 3.0) and torch.all(dv[:, :, ls:] == 3.0)
    assert np.array_equal(dt.cpu().numpy()[:, :, :ls], rt[:, :, :ls])


def test_reorder_identity_and_bad_parent():
    c = wl.make_decode_case(2, 6, 4, 3, 4, 2, 64, seed=2)
    sk, sv = c.suffix_k.to(DEV), c.suffix_v.to(DEV)
    ident = torch.arange(6, dtype=torch.int32, device=DEV).repeat(2, 1)
    dk, dv = bga().suffix_reorder(sk, sv, ident, 3)
    assert torch.equal(dk, sk) and torch.equal(dv, sv)
    bad = ident.clone()
    bad[1, 2] = 99
    dk, dv = bga().suffix_reorder(sk, sv, bad, 3)
    assert torch.all(dk[1, 2] == 0) and torch.equal(dk[0], sk[0]) and torch.equal(dk[1, 3], sk[1, 3])


# ---------------------------------------------------------------- prompts of their own lengths, packed

def packed_prompts(lps, w, ls_cap, nq, nkv, d, seed):
    c = wl.make_decode_case(len(lps), w, 1, ls_cap, nq, nkv, d, seed, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed + 1)
    tp = int(sum(lps))
    pk = wl.bf16_normal((tp, nkv, d), gen, DEV)
    pv = wl.bf16_normal((tp, nkv, d), gen, DEV)
    return c, pk, pv, wl.cu_seqlens_from_lengths(lps)


@pytest.mark.parametrize("lps,w,ls,cap,nq,nkv,d", [
    ((7, 0, 130, 64, 1), 5, 2, 3, 4, 2, 64),                  # an empty prompt, ragged and exact tiles
    ((480, 455, 512, 300, 479, 1, 64, 200), 400, 3, 5, 16, 8, 128),   # long prompts of their own lengths, W 400
    ((128, 96, 160, 33) * 8, 100, 4, 4, 16, 8, 64),           # 32 short-prompt requests, W 100
    ((65, 0, 17), 130, 1, 2, 4, 4, 128),                      # group 1, two slots of beams per workgroup
    ((5, 9), 9, 0, 2, 16, 1, 128),                            # no suffix: prompts only
])
def test_packed_prompt_decode(lps, w, ls, cap, nq, nkv, d):
    c, pk, pv, cu = packed_prompts(lps, w, cap, nq, nkv, d, seed=len(lps) * 100 + w)
    say(f"[decode packed] R={len(lps)} W={w} prompts {lps[:8]} Ls={ls}/{cap} nq={nq} nkv={nkv} d={d}")
    out, lse = bga().shared_prefix_decode_packed(c.q, pk, pv, torch.from_numpy(cu).to(DEV), c.suffix_k, c.suffix_v, ls)
    torch.cuda.synchronize()
    ro, rl = oracle.shared_prefix_decode_packed(c.q.cpu(), pk.cpu(), pv.cpu(), cu, c.suffix_k.cpu(), c.suffix_v.cpu(),
                                                ls)
    e = check_bf16(out, ro, "packed prompts out")
    l_ = check_lse(lse, rl, "packed prompts lse")
    say(f"    max |out err| {e:.2e}  max |lse err| {l_:.2e}")


def test_packed_prompts_of_equal_length_equal_the_strided_layout():
    """With every prompt of the same length the packed call is the strided call, bit for bit: the prefill's
    packed K/V of the prompts serves as the shared prefix unchanged."""
    c = wl.make_decode_case(4, 37, 90, 3, 8, 2, 64, seed=11, device=DEV)
    cu = torch.arange(0, 5 * 90, 90, dtype=torch.int32, device=DEV)
    o1, l1 = bga().shared_prefix_decode(c.q, c.prefix_k, c.prefix_v, c.suffix_k, c.suffix_v, 2)
    o2, l2 = bga().shared_prefix_decode_packed(c.q, c.prefix_k.view(-1, 2, 64), c.prefix_v.view(-1, 2, 64), cu,
                                               c.suffix_k, c.suffix_v, 2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- last valid token of each sequence

@pytest.mark.parametrize("lengths,row_shape,dtype", [
    ([3, 0, 1, 7, 0, 2], (16, 128), torch.bfloat16),
    (wl.lengths_uniform(15, 64, 480, 1), (16, 128), torch.bfloat16),
    ([1] * 33, (1000,), torch.float32),
    ([5, 300, 0, 11], (8192,), torch.float32),      # 32 KB rows: several workgroups per row
    ([0, 0], (8,), torch.float16),
])
def test_last_token_gather(lengths, row_shape, dtype):
    cu = wl.cu_seqlens_from_lengths(lengths)
    t = int(cu[-1])
    g = torch.Generator(device=DEV)
    g.manual_seed(t)
    x = torch.randn((t,) + row_shape, generator=g, device=DEV).to(dtype)
    say(f"[gather] B={len(lengths)} T={t} row {row_shape} {dtype}")
    y = bga().last_token_gather(x, torch.from_numpy(cu).to(DEV))
    ref = oracle.last_token_gather(x.cpu().view(torch.int16 if x.element_size() == 2 else torch.int32).numpy(), cu)
    got = y.cpu().view(torch.int16 if x.element_size() == 2 else torch.int32).numpy()
    assert np.array_equal(got, ref)
