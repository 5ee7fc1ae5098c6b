"""Baselines for the article's relative claims, timed beside the HIP kernels.

MEASUREMENT INFRASTRUCTURE ONLY: only bench.py and the tests use this package;
the product path (libbga and its binding) never does.

  * Explicit Torch attention for packed prefill (article section 3.1: the
    Triton Packed GQA kernel was measured against an explicit Torch packed
    attention, +12 % / +39 % whole-request throughput for medium / long
    prompts, and the explicit form also served as its numerical reference):
      - padded: every sequence padded to the longest, GQA K/V expanded to the
        query heads, scores materialised over [B, Nq, L_max, L_max] with a
        causal-and-valid mask (the B x L_max^2 form section 3.1 contrasts with
        sum L_i^2);
      - packed: the scores of the whole packed buffer [Nq, T, T] with the
        block-diagonal causal mask the sequence boundary defines.
  * The per-beam full K/V layout for beam decode (article section 3.2: every
    beam keeping its own [L_p + L_s] K/V, the W (L_p + L_s) state the
    shared-prefix layout replaces; the article reports decode attention time
    down about 60 % with the shared prefix): the concatenation
    [prompt; suffix of b] materialised per beam, then attention per beam in
    Torch (batched matrix products, fp32 softmax).

All matrix products take bf16 inputs with contiguous right operands; softmax
runs in fp32; outputs are bf16 like the kernels'.
"""
from __future__ import annotations

import torch


def _softmax_rows(s: torch.Tensor, mask: torch.Tensor) -> torch.Tensor:
    s = s.float().masked_fill(~mask, float("-inf"))
    return torch.softmax(s, dim=-1)


def padded_prefill(q, k, v, lengths, scale):
    """q [T, Nq, D], k/v [T, Nkv, D] packed (bf16); lengths: the B sequence lengths (host list).
    Returns the packed output [T, Nq, D] bf16."""
    T, nq, d = q.shape
    nkv = k.shape[1]
    g = nq // nkv
    B, L = len(lengths), max(lengths)
    dev = q.device
    starts = torch.tensor([0] + list(torch.tensor(lengths).cumsum(0)[:-1].tolist()), device=dev)
    pos = torch.arange(L, device=dev)
    valid = pos[None, :] < torch.tensor(lengths, device=dev)[:, None]                 # [B, L]
    idx = (starts[:, None] + pos[None, :]).clamp(max=T - 1)                           # [B, L]
    qp = q[idx].masked_fill(~valid[:, :, None, None], 0).permute(0, 2, 1, 3).contiguous()          # [B, Nq, L, D]
    kp = k[idx].repeat_interleave(g, dim=2).masked_fill(~valid[:, :, None, None], 0)
    vp = v[idx].repeat_interleave(g, dim=2).masked_fill(~valid[:, :, None, None], 0)
    kt = kp.permute(0, 2, 3, 1).contiguous()                                          # [B, Nq, D, L]
    vp = vp.permute(0, 2, 1, 3).contiguous()                                          # [B, Nq, L, D]
    s = torch.matmul(qp, kt) * scale                                                  # [B, Nq, L, L]
    mask = (pos[:, None] >= pos[None, :])[None, None] & valid[:, None, None, :]
    p = _softmax_rows(s, mask).to(torch.bfloat16)
    o = torch.matmul(p, vp).permute(0, 2, 1, 3)                                       # [B, L, Nq, D]
    return o[valid].contiguous()


def packed_prefill(q, k, v, cu_seqlens, scale):
    """The explicit block-diagonal causal form over the whole packed buffer ([Nq, T, T] scores).
    cu_seqlens [B+1] int32 on the device. Returns [T, Nq, D] bf16."""
    T, nq, d = q.shape
    g = nq // k.shape[1]
    dev = q.device
    seq = torch.bucketize(torch.arange(T, device=dev), cu_seqlens[1:].long(), right=True)   # sequence of each token
    tok = torch.arange(T, device=dev)
    mask = (seq[:, None] == seq[None, :]) & (tok[:, None] >= tok[None, :])
    qh = q.permute(1, 0, 2).contiguous()                                              # [Nq, T, D]
    kt = k.repeat_interleave(g, dim=1).permute(1, 2, 0).contiguous()                  # [Nq, D, T]
    vh = v.repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()                  # [Nq, T, D]
    s = torch.matmul(qh, kt) * scale
    p = _softmax_rows(s, mask[None]).to(torch.bfloat16)
    return torch.matmul(p, vh).permute(1, 0, 2).contiguous()


def per_beam_kv(prefix_k, prefix_v, suffix_k, suffix_v, suffix_len):
    """The per-beam full K/V state: for every (request, beam) its own [prompt; suffix] copy, stored as
    K^T [R, W, Nkv, D, L] and V [R, W, Nkv, L, D] (L = L_p + L_s), contiguous for the batched products."""
    R, W = suffix_k.shape[:2]
    lp = prefix_k.shape[1]
    kk = torch.cat([prefix_k[:, None].expand(R, W, lp, *prefix_k.shape[2:]), suffix_k[:, :, :suffix_len]], dim=2)
    vv = torch.cat([prefix_v[:, None].expand(R, W, lp, *prefix_v.shape[2:]), suffix_v[:, :, :suffix_len]], dim=2)
    return kk.permute(0, 1, 3, 4, 2).contiguous(), vv.permute(0, 1, 3, 2, 4).contiguous()


def per_beam_kv_packed(prefix_k, prefix_v, suffix_k, suffix_v, suffix_len):
    """The same per-beam copies as rows [R * W * L, Nkv, D] (beam after beam), the layout the library's packed
    decode reads when every beam is a request of its own."""
    R, W = suffix_k.shape[:2]
    lp = prefix_k.shape[1]
    kk = torch.cat([prefix_k[:, None].expand(R, W, lp, *prefix_k.shape[2:]), suffix_k[:, :, :suffix_len]], dim=2)
    vv = torch.cat([prefix_v[:, None].expand(R, W, lp, *prefix_v.shape[2:]), suffix_v[:, :, :suffix_len]], dim=2)
    return kk.reshape(-1, *kk.shape[3:]).contiguous(), vv.reshape(-1, *vv.shape[3:]).contiguous()


def per_beam_decode(q, kt_full, v_full, scale):
    """q [R, W, Nq, D]; K^T [R, W, Nkv, D, L]; V [R, W, Nkv, L, D]. Every beam attends over its own copy.
    Returns [R, W, Nq, D] bf16."""
    R, W, nq, d = q.shape
    nkv = kt_full.shape[2]
    g = nq // nkv
    qg = q.reshape(R, W, nkv, g, d)
    s = torch.matmul(qg, kt_full) * scale                                             # [R, W, Nkv, G, L]
    p = torch.softmax(s.float(), dim=-1).to(torch.bfloat16)
    return torch.matmul(p, v_full).reshape(R, W, nq, d)
