"""Seeded synthetic inputs and algorithmic work counts for the attention hot path.

This package holds no part of the attention, selection or reorder arithmetic.
It only draws inputs (lengths, bf16 tensors, parent indices) from fixed seeds,
and counts logical matrix FLOPs and algorithmic bytes for the roofline figures.
Both the HIP path and the oracle consume the inputs it produces.
"""
from .generators import (  # noqa: F401
    CONFIGS,
    PrefillCase,
    DecodeCase,
    bf16_normal,
    lengths_lognormal,
    lengths_uniform,
    make_prefill_case,
    make_named_prefill,
    make_named_decode,
    prefill_lengths,
    bf16_bits,
    make_decode_case,
    make_logits,
    make_parents,
    cu_seqlens_from_lengths,
)
from .counts import (  # noqa: F401
    causal_pairs,
    prefill_flops,
    prefill_bytes,
    decode_flops,
    decode_bytes,
    reorder_bytes,
    topk_bytes,
    state_elems_shared_prefix,
    state_elems_per_beam,
    effective_mfu,
    swiglu_quant_bytes,
    gather_bytes,
    beam_advance_bytes,
    suffix_append_bytes,
)
