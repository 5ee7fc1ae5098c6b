"""Algorithmic work counts used for the roofline figures.

FLOPs follow the article's counting rule for logical matrix work (section 4.5,
"Mixed-precision effective MFU"): only the logical matrix products count, one
FMA is two FLOPs, and padding, blocking redundancy, softmax and selection are
excluded. For causal attention over a sequence of length L the number of
query-key pairs is the triangular count L(L+1)/2 (the chunked-prefill passage of
the inference-operations chapter), and each pair costs D MACs for Q.K^T and D
MACs for P.V, i.e. 4*D FLOPs per pair and query head.

Bytes are the algorithmic HBM traffic: every input read once, every output
written once. For shared-prefix decode the prompt K/V is counted once per
request, since reading it once per request instead of once per beam is what the
shared-prefix layout buys (article section 3.2, state L_p + W*L_s instead of
W*(L_p + L_s)).
"""
from __future__ import annotations


def causal_pairs(lengths) -> int:
    """Query-key pairs of block-diagonal causal attention: sum of L(L+1)/2."""
    return sum(int(n) * (int(n) + 1) // 2 for n in lengths)


def prefill_flops(lengths, nq: int, d: int) -> int:
    return 4 * d * nq * causal_pairs(lengths)


def prefill_bytes(lengths, nq: int, nkv: int, d: int, with_lse: bool = True) -> int:
    """Algorithmic HBM bytes of one packed prefill: Q, K, V read once, O (and LSE) written once."""
    t = int(sum(lengths))
    return t * (2 * nq + 2 * nkv) * d * 2 + (t * nq * 4 if with_lse else 0)


def decode_flops(r: int, w: int, nq: int, lp: int, ls: int, d: int) -> int:
    return 4 * r * w * nq * (lp + ls) * d


def decode_bytes(r: int, w: int, nq: int, nkv: int, lp: int, ls: int, d: int, with_lse: bool = True) -> int:
    bf16 = 2
    prefix = 2 * lp * nkv * d * bf16            # K and V, once per request
    suffix = 2 * w * ls * nkv * d * bf16        # K and V, per beam
    q_and_o = 2 * w * nq * d * bf16             # Q read, O written
    lse = 4 * w * nq if with_lse else 0
    return r * (prefix + suffix + q_and_o + lse)


def reorder_bytes(r: int, w: int, ls: int, nkv: int, d: int, n_tokens: int = 0) -> int:
    kv = 2 * 2 * r * w * ls * nkv * d * 2       # (K, V) x (read, write) x bf16
    parents = 4 * r * w
    tokens = 2 * 4 * r * w * n_tokens
    return kv + parents + tokens


def topk_bytes(r: int, w_in: int, vocab: int, k_global: int) -> int:
    return 2 * r * w_in * vocab + 4 * r * w_in + 12 * r * k_global


def state_elems_shared_prefix(lp: int, w: int, ls: int, nkv: int, d: int) -> int:
    """K (or V) elements held per request with one prompt copy plus per-beam suffixes."""
    return (lp + w * ls) * nkv * d


def state_elems_per_beam(lp: int, w: int, ls: int, nkv: int, d: int) -> int:
    """K (or V) elements held per request when every beam keeps a full copy."""
    return w * (lp + ls) * nkv * d


def effective_mfu(qps: float, f_bf16: float, p_bf16: float, f_fp8: float = 0.0, p_fp8: float = 1.0) -> float:
    """The article's mixed-precision effective MFU: QPS * (F_bf16/P_bf16 + F_fp8/P_fp8)."""
    return qps * (f_bf16 / p_bf16 + f_fp8 / p_fp8)


def swiglu_quant_bytes(t: int, inter: int) -> int:
    """Gate and up read once (bf16), E4M3 codes and the per-token fp32 scale written once."""
    return t * 2 * inter * 2 + t * inter + 4 * t


def gather_bytes(num_seqs: int, row_bytes: int) -> int:
    """One row read and one written per sequence, plus the offsets."""
    return 2 * num_seqs * row_bytes + 4 * (num_seqs + 1)


def beam_advance_bytes(r: int, w: int, w_in: int, step: int) -> int:
    """2W candidates read (token, parent, score); W new beams written (parent, score, step + 1 tokens) after
    reading their source tokens; the finished pool writes are data dependent and not counted."""
    return r * (2 * w * 12 + w * (8 + 4 * (step + 1)) + w * 4 * step)


def suffix_append_bytes(r: int, w: int, nkv: int, d: int) -> int:
    return 2 * 2 * r * w * nkv * d * 2
