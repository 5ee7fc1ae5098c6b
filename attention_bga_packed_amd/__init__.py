"""attention_bga_packed_amd — the attention hot path of a bounded-generation
SLM engine (packed causal GQA prefill, shared-prefix beam decode, parent-index
reorder, two-stage beam top-K) as HIP kernels for MI355X (gfx950) behind the C
ABI in include/bga.h.

Importing the package loads libbga.so and raises if it is missing; there is no
fallback path.
"""
from ._binding import (  # noqa: F401
    BgaError,
    DEBUG_LIB_PATH,
    EXPORTS,
    LIB_PATH,
    RELEASE_LIB_PATH,
    beam_topk,
    beam_topk_noalloc,
    beam_topk_workspace_size,
    last_token_gather,
    lib,
    load_library,
    packed_gqa_prefill,
    shared_prefix_decode,
    shared_prefix_decode_packed,
    suffix_reorder,
    swiglu_quant_e4m3,
)
