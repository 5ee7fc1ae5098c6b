// C-ABI entry points of libbga: host-side argument validation, then one or two
// kernel launches on the caller's stream. Nothing is enqueued when validation
// fails. See include/bga.h for the contract of every call.
#include <math.h>
#include <stdint.h>

#include "bga.h"
#include "internal.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;
thread_local uint32_t g_last_violations = 0;

bga_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return BGA_OK;
    g_last_hip_error = (int32_t)e;
    return BGA_ERR_HIP;
}

#ifdef BGA_DEBUG
// Outcome of a debug build's device-side check: a HIP error, a violation, or go.
bga_status check_status(hipError_t e, uint32_t violations)
{
    if (e != hipSuccess) return hip_status(e);
    if (violations) {
        g_last_violations = violations;
        return BGA_ERR_PRECONDITION;
    }
    return BGA_OK;
}
#endif

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool heads_ok(int32_t nq, int32_t nkv)
{
    return nq > 0 && nkv > 0 && nq % nkv == 0 && nq / nkv <= BGA_MAX_GROUP;
}

// [a, a + na) and [b, b + nb) overlap (bytes)
bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

bga_status bga_packed_gqa_prefill(const bga_bf16 *q, const bga_bf16 *k, const bga_bf16 *v,
                                  const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                  int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, float softmax_scale, bga_bf16 *out, float *lse,
                                  hipStream_t stream)
{
    if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0) return BGA_ERR_SHAPE;
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return BGA_ERR_SHAPE;
    if (!heads_ok(num_q_heads, num_kv_heads)) return BGA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return BGA_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || max_seqlen > BGA_MAX_SEQLEN) return BGA_ERR_UNSUPPORTED;
    if ((int64_t)total_tokens * num_q_heads > 0x7fffffff) return BGA_ERR_UNSUPPORTED;   // output row index
    if (((int64_t)num_seqs * num_kv_heads + 7) / 8 * 8 * (((int64_t)max_seqlen * (num_q_heads / num_kv_heads) + 127) / 128) >
        0x7fffffff / 256)
        return BGA_ERR_UNSUPPORTED;   // workgroups of the 1-D grid
    if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return BGA_ERR_SHAPE;
    if (total_tokens > 0 && (num_seqs == 0 || max_seqlen == 0)) return BGA_ERR_SHAPE;   // rows nobody would write
    if (!cu_seqlens) return BGA_ERR_NULL;
    if (total_tokens == 0) return BGA_OK;
    if (!q || !k || !v || !out) return BGA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(cu_seqlens, 4) ||
        (lse && !aligned(lse, 4)))
        return BGA_ERR_ALIGN;
    const size_t qbytes = (size_t)total_tokens * num_q_heads * head_dim * 2;
    const size_t kvbytes = (size_t)total_tokens * num_kv_heads * head_dim * 2;
    if (overlap(out, qbytes, q, qbytes) || overlap(out, qbytes, k, kvbytes) || overlap(out, qbytes, v, kvbytes))
        return BGA_ERR_ALIAS;
#ifdef BGA_DEBUG
    {
        uint32_t bad = 0;
        const bga_status st =
            check_status(bga::debug_check_prefill(cu_seqlens, num_seqs, total_tokens, max_seqlen, stream, &bad), bad);
        if (st != BGA_OK) return st;
    }
#endif
    return hip_status(bga::launch_packed_prefill(q, k, v, cu_seqlens, num_seqs, total_tokens, max_seqlen,
                                                 num_q_heads, num_kv_heads, head_dim, softmax_scale, out, lse,
                                                 stream));
}

// Host checks shared by both decode entry points (prompt-specific checks are the caller's).
static bga_status decode_check(const bga_bf16 *q, const bga_bf16 *suffix_k, const bga_bf16 *suffix_v,
                               int32_t num_requests, int32_t beam_width, int32_t suffix_len, int32_t suffix_cap,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                               const bga_bf16 *out, const float *lse)
{
    if (num_requests < 0 || beam_width < 0 || suffix_len < 0 || suffix_cap < 0) return BGA_ERR_SHAPE;
    if (suffix_len > suffix_cap) return BGA_ERR_SHAPE;
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return BGA_ERR_SHAPE;
    if (!heads_ok(num_q_heads, num_kv_heads)) return BGA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return BGA_ERR_UNSUPPORTED;
    if (beam_width > BGA_MAX_BEAMS || suffix_cap > BGA_MAX_SUFFIX) return BGA_ERR_UNSUPPORTED;
    if ((int64_t)num_requests * num_kv_heads > 0x7fffffff) return BGA_ERR_UNSUPPORTED;
    if ((int64_t)num_requests * beam_width * num_q_heads > 0x7fffffff) return BGA_ERR_UNSUPPORTED;   // output row index
    if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return BGA_ERR_SHAPE;
    if (num_requests == 0 || beam_width == 0) return BGA_OK;
    if (!q || !out) return BGA_ERR_NULL;
    if (suffix_len > 0 && (!suffix_k || !suffix_v)) return BGA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(suffix_k, 16) || !aligned(suffix_v, 16) ||
        (lse && !aligned(lse, 4)))
        return BGA_ERR_ALIGN;
    const size_t obytes = (size_t)num_requests * beam_width * num_q_heads * head_dim * 2;
    const size_t sbytes = (size_t)num_requests * beam_width * suffix_cap * num_kv_heads * head_dim * 2;
    if (overlap(out, obytes, q, obytes) || overlap(out, obytes, suffix_k, sbytes) ||
        overlap(out, obytes, suffix_v, sbytes))
        return BGA_ERR_ALIAS;
    return BGA_OK;
}

bga_status bga_shared_prefix_decode(const bga_bf16 *q, const bga_bf16 *prefix_k, const bga_bf16 *prefix_v,
                                    const bga_bf16 *suffix_k, const bga_bf16 *suffix_v, int32_t num_requests,
                                    int32_t beam_width, int32_t prefix_len, int32_t suffix_len,
                                    int32_t suffix_cap, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, float softmax_scale, bga_bf16 *out, float *lse,
                                    hipStream_t stream)
{
    if (prefix_len < 0) return BGA_ERR_SHAPE;
    if (prefix_len + (int64_t)suffix_len < 1) return BGA_ERR_SHAPE;
    bga_status st = decode_check(q, suffix_k, suffix_v, num_requests, beam_width, suffix_len, suffix_cap, num_q_heads,
                                 num_kv_heads, head_dim, softmax_scale, out, lse);
    if (st == BGA_OK && prefix_len > BGA_MAX_SEQLEN) st = BGA_ERR_UNSUPPORTED;
    if (st != BGA_OK || num_requests == 0 || beam_width == 0) return st;
    if (prefix_len > 0 && (!prefix_k || !prefix_v)) return BGA_ERR_NULL;
    if (!aligned(prefix_k, 16) || !aligned(prefix_v, 16)) return BGA_ERR_ALIGN;
    const size_t obytes = (size_t)num_requests * beam_width * num_q_heads * head_dim * 2;
    const size_t pbytes = (size_t)num_requests * prefix_len * num_kv_heads * head_dim * 2;
    if (overlap(out, obytes, prefix_k, pbytes) || overlap(out, obytes, prefix_v, pbytes)) return BGA_ERR_ALIAS;
    return hip_status(bga::launch_shared_prefix_decode(q, prefix_k, prefix_v, nullptr, suffix_k, suffix_v,
                                                       num_requests, beam_width, prefix_len, suffix_len, suffix_cap,
                                                       num_q_heads, num_kv_heads, head_dim, softmax_scale, out, lse,
                                                       stream));
}

bga_status bga_shared_prefix_decode_packed(const bga_bf16 *q, const bga_bf16 *prefix_k, const bga_bf16 *prefix_v,
                                           const int32_t *prefix_cu, int32_t total_prefix_tokens,
                                           const bga_bf16 *suffix_k, const bga_bf16 *suffix_v,
                                           int32_t num_requests, int32_t beam_width, int32_t suffix_len,
                                           int32_t suffix_cap, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, float softmax_scale, bga_bf16 *out, float *lse,
                                           hipStream_t stream)
{
    if (total_prefix_tokens < 0) return BGA_ERR_SHAPE;
    if (total_prefix_tokens == 0 && suffix_len == 0 && num_requests > 0) return BGA_ERR_SHAPE;   // no key anywhere
    bga_status st = decode_check(q, suffix_k, suffix_v, num_requests, beam_width, suffix_len, suffix_cap, num_q_heads,
                                 num_kv_heads, head_dim, softmax_scale, out, lse);
    if (st != BGA_OK || num_requests == 0 || beam_width == 0) return st;
    if (!prefix_cu) return BGA_ERR_NULL;
    if (total_prefix_tokens > 0 && (!prefix_k || !prefix_v)) return BGA_ERR_NULL;
    if (!aligned(prefix_k, 16) || !aligned(prefix_v, 16) || !aligned(prefix_cu, 4)) return BGA_ERR_ALIGN;
    const size_t obytes = (size_t)num_requests * beam_width * num_q_heads * head_dim * 2;
    const size_t pbytes = (size_t)total_prefix_tokens * num_kv_heads * head_dim * 2;
    if (overlap(out, obytes, prefix_k, pbytes) || overlap(out, obytes, prefix_v, pbytes)) return BGA_ERR_ALIAS;
#ifdef BGA_DEBUG
    {
        uint32_t bad = 0;
        st = check_status(bga::debug_check_prompts(prefix_cu, num_requests, total_prefix_tokens, BGA_MAX_SEQLEN,
                                                   suffix_len == 0, stream, &bad),
                          bad);
        if (st != BGA_OK) return st;
    }
#endif
    return hip_status(bga::launch_shared_prefix_decode(q, prefix_k, prefix_v, prefix_cu, suffix_k, suffix_v,
                                                       num_requests, beam_width, 0, suffix_len, suffix_cap,
                                                       num_q_heads, num_kv_heads, head_dim, softmax_scale, out, lse,
                                                       stream));
}

bga_status bga_last_token_gather(const void *src, const int32_t *cu_seqlens, int32_t num_seqs,
                                 int32_t total_tokens, int64_t row_bytes, void *dst, hipStream_t stream)
{
    if (num_seqs < 0 || total_tokens < 0 || row_bytes <= 0 || row_bytes % 16) return BGA_ERR_SHAPE;
    if (num_seqs > 0x7fffffff / 2 || row_bytes / 16 > ((int64_t)1 << 40)) return BGA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return BGA_OK;
    if (!cu_seqlens || !dst || (total_tokens > 0 && !src)) return BGA_ERR_NULL;
    if (!aligned(dst, 16) || (src && !aligned(src, 16)) || !aligned(cu_seqlens, 4)) return BGA_ERR_ALIGN;
    if (total_tokens > 0 && overlap(dst, (size_t)num_seqs * row_bytes, src, (size_t)total_tokens * row_bytes))
        return BGA_ERR_ALIAS;
#ifdef BGA_DEBUG
    {
        uint32_t bad = 0;
        const bga_status st =
            check_status(bga::debug_check_prompts(cu_seqlens, num_seqs, total_tokens, 0x7fffffff, false, stream, &bad),
                         bad);
        if (st != BGA_OK) return st;
    }
#endif
    return hip_status(bga::launch_last_token_gather(total_tokens > 0 ? src : dst, cu_seqlens, num_seqs,
                                                    total_tokens > 0 ? total_tokens : 1, row_bytes, dst, stream));
}

bga_status bga_suffix_reorder(const bga_bf16 *src_k, const bga_bf16 *src_v, bga_bf16 *dst_k, bga_bf16 *dst_v,
                              const int32_t *parent, const int32_t *src_tokens, int32_t *dst_tokens,
                              int32_t num_requests, int32_t beam_width, int32_t suffix_len, int32_t suffix_cap,
                              int32_t num_kv_heads, int32_t head_dim, int32_t num_tokens, int32_t tok_cap,
                              hipStream_t stream)
{
    if (num_requests < 0 || beam_width < 0 || suffix_len < 0 || suffix_cap < 0 || suffix_len > suffix_cap)
        return BGA_ERR_SHAPE;
    if (num_kv_heads <= 0) return BGA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return BGA_ERR_UNSUPPORTED;
    if (beam_width > BGA_MAX_BEAMS || suffix_cap > BGA_MAX_SUFFIX) return BGA_ERR_UNSUPPORTED;
    if ((int64_t)num_requests * beam_width > 0x7fffffff) return BGA_ERR_UNSUPPORTED;   // one workgroup per beam
    if ((src_tokens == nullptr) != (dst_tokens == nullptr)) return BGA_ERR_NULL;
    if (src_tokens && (num_tokens < 0 || tok_cap < 0 || num_tokens > tok_cap)) return BGA_ERR_SHAPE;
    if (num_requests == 0 || beam_width == 0) return BGA_OK;
    if (!parent || !src_k || !src_v || !dst_k || !dst_v) return BGA_ERR_NULL;
    if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 16) || !aligned(dst_v, 16) ||
        !aligned(parent, 4) || (src_tokens && (!aligned(src_tokens, 4) || !aligned(dst_tokens, 4))))
        return BGA_ERR_ALIGN;
    const size_t kv = (size_t)num_requests * beam_width * suffix_cap * num_kv_heads * head_dim * 2;
    if (overlap(dst_k, kv, src_k, kv) || overlap(dst_k, kv, src_v, kv) || overlap(dst_v, kv, src_k, kv) ||
        overlap(dst_v, kv, src_v, kv) || overlap(dst_k, kv, dst_v, kv))
        return BGA_ERR_ALIAS;
    if (src_tokens) {
        const size_t tb = (size_t)num_requests * beam_width * tok_cap * 4;
        if (overlap(dst_tokens, tb, src_tokens, tb)) return BGA_ERR_ALIAS;
    }
#ifdef BGA_DEBUG
    {
        uint32_t bad = 0;
        const bga_status st =
            check_status(bga::debug_check_parents(parent, num_requests * beam_width, beam_width, stream, &bad), bad);
        if (st != BGA_OK) return st;
    }
#endif
    return hip_status(bga::launch_suffix_reorder(src_k, src_v, dst_k, dst_v, parent, src_tokens, dst_tokens,
                                                 num_requests, beam_width, suffix_len, suffix_cap, num_kv_heads,
                                                 head_dim, src_tokens ? num_tokens : 0, tok_cap, stream));
}

static bool topk_sizes_ok(int32_t R, int32_t W_in, int32_t V, int32_t k_local, int32_t k_global)
{
    if (R < 0 || W_in <= 0 || V <= 0 || k_local <= 0 || k_global <= 0) return false;
    if (W_in > BGA_MAX_BEAMS || V > BGA_MAX_VOCAB || k_local > V || k_local > BGA_MAX_K || k_global > BGA_MAX_K)
        return false;
    if ((int64_t)k_global > (int64_t)W_in * k_local) return false;
    if ((int64_t)R * W_in > 0x7fffffff) return false;   // one workgroup per beam row
    return true;
}

size_t bga_beam_topk_workspace_size(int32_t num_requests, int32_t num_src_beams, int32_t vocab, int32_t k_local,
                                    int32_t k_global)
{
    if (!topk_sizes_ok(num_requests, num_src_beams, vocab, k_local, k_global)) return 0;
    return bga::topk_workspace_layout(num_requests, num_src_beams, k_local).total;
}

// Host checks shared by both top-K entry points; *need = workspace bytes.
static bga_status topk_check(const bga_bf16 *logits, const float *cum_scores, int32_t num_requests,
                             int32_t num_src_beams, int32_t vocab, int32_t k_local, int32_t k_global,
                             int32_t *out_tokens, int32_t *out_parents, float *out_scores, int32_t *local_tokens,
                             float *local_scores, float *row_lse, size_t *need)
{
    *need = 0;
    if (num_requests < 0 || num_src_beams <= 0 || vocab <= 0 || k_local <= 0 || k_global <= 0)
        return BGA_ERR_SHAPE;
    if ((int64_t)k_global > (int64_t)num_src_beams * k_local || k_local > vocab) return BGA_ERR_SHAPE;
    if (!topk_sizes_ok(num_requests, num_src_beams, vocab, k_local, k_global)) return BGA_ERR_UNSUPPORTED;
    if (num_requests == 0) return BGA_OK;
    if (!logits || !out_tokens || !out_parents || !out_scores) return BGA_ERR_NULL;
    if (!aligned(logits, 16) || !aligned(out_tokens, 4) || !aligned(out_parents, 4) || !aligned(out_scores, 4) ||
        (cum_scores && !aligned(cum_scores, 4)) || (local_tokens && !aligned(local_tokens, 4)) ||
        (local_scores && !aligned(local_scores, 4)) || (row_lse && !aligned(row_lse, 4)))
        return BGA_ERR_ALIGN;
    *need = bga::topk_workspace_layout(num_requests, num_src_beams, k_local).total;
    return BGA_OK;
}

bga_status bga_beam_topk(const bga_bf16 *logits, const float *cum_scores, int32_t num_requests,
                         int32_t num_src_beams, int32_t vocab, int32_t k_local, int32_t k_global,
                         int32_t *out_tokens, int32_t *out_parents, float *out_scores, int32_t *local_tokens,
                         float *local_scores, float *row_lse, void *workspace, size_t workspace_bytes,
                         hipStream_t stream)
{
    size_t need = 0;
    bga_status st = topk_check(logits, cum_scores, num_requests, num_src_beams, vocab, k_local, k_global,
                               out_tokens, out_parents, out_scores, local_tokens, local_scores, row_lse, &need);
    if (st != BGA_OK || num_requests == 0) return st;
    if (!workspace || workspace_bytes < need) return BGA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return BGA_ERR_ALIGN;
    const size_t lbytes = (size_t)num_requests * num_src_beams * vocab * 2;
    if (overlap(workspace, need, logits, lbytes)) return BGA_ERR_ALIAS;
#ifdef BGA_DEBUG
    {
        uint32_t bad = 0;
        st = check_status(bga::debug_check_logits(logits, lbytes / 2, stream, &bad), bad);
        if (st != BGA_OK) return st;
    }
#endif
    return hip_status(bga::launch_beam_topk(logits, cum_scores, num_requests, num_src_beams, vocab, k_local,
                                            k_global, out_tokens, out_parents, out_scores, local_tokens,
                                            local_scores, row_lse, workspace, stream));
}

bga_status bga_beam_topk_noalloc(const bga_bf16 *logits, const float *cum_scores, int32_t num_requests,
                                 int32_t num_src_beams, int32_t vocab, int32_t k_local, int32_t k_global,
                                 int32_t *out_tokens, int32_t *out_parents, float *out_scores,
                                 int32_t *local_tokens, float *local_scores, float *row_lse, hipStream_t stream)
{
    size_t need = 0;
    bga_status st = topk_check(logits, cum_scores, num_requests, num_src_beams, vocab, k_local, k_global,
                               out_tokens, out_parents, out_scores, local_tokens, local_scores, row_lse, &need);
    if (st != BGA_OK || num_requests == 0) return st;
    if (need > BGA_TOPK_SCRATCH_BYTES) return BGA_ERR_WORKSPACE;
    void *workspace = nullptr;
    hipError_t e = bga::topk_scratch(&workspace);
    if (e != hipSuccess) return hip_status(e);
#ifdef BGA_DEBUG
    {
        uint32_t bad = 0;
        const size_t lbytes = (size_t)num_requests * num_src_beams * vocab * 2;
        st = check_status(bga::debug_check_logits(logits, lbytes / 2, stream, &bad), bad);
        if (st != BGA_OK) return st;
    }
#endif
    return hip_status(bga::launch_beam_topk(logits, cum_scores, num_requests, num_src_beams, vocab, k_local,
                                            k_global, out_tokens, out_parents, out_scores, local_tokens,
                                            local_scores, row_lse, workspace, stream));
}

bga_status bga_beam_advance(const int32_t *cand_tokens, const int32_t *cand_parents, const float *cand_scores,
                            int32_t num_requests, int32_t num_src_beams, int32_t beam_width, int32_t stop_token,
                            int32_t step, const int32_t *tokens_in, int32_t *tokens_out, int32_t tok_cap,
                            int32_t *parents_out, float *cum_out, float *pool_scores, int32_t *pool_lengths,
                            int32_t *pool_tokens, int32_t *pool_count, int32_t pool_cap, hipStream_t stream)
{
    if (num_requests < 0 || beam_width < 1 || num_src_beams < 1 || num_src_beams > beam_width || step < 0 ||
        step >= tok_cap || pool_cap < 1)
        return BGA_ERR_SHAPE;
    if (beam_width > BGA_MAX_BEAMS) return BGA_ERR_UNSUPPORTED;
    if ((int64_t)num_requests * pool_cap * tok_cap > 0x7fffffff) return BGA_ERR_UNSUPPORTED;
    if (num_requests == 0) return BGA_OK;
    if (!cand_tokens || !cand_parents || !cand_scores || !tokens_in || !tokens_out || !parents_out || !cum_out ||
        !pool_scores || !pool_lengths || !pool_tokens || !pool_count)
        return BGA_ERR_NULL;
    const void *ptrs[] = {cand_tokens, cand_parents, cand_scores, tokens_in, tokens_out, parents_out, cum_out,
                          pool_scores, pool_lengths, pool_tokens, pool_count};
    for (const void *p : ptrs)
        if (!aligned(p, 4)) return BGA_ERR_ALIGN;
    const size_t tin = (size_t)num_requests * num_src_beams * tok_cap * 4;
    const size_t tout = (size_t)num_requests * beam_width * tok_cap * 4;
    if (overlap(tokens_out, tout, tokens_in, tin)) return BGA_ERR_ALIAS;
    return hip_status(bga::launch_beam_advance(cand_tokens, cand_parents, cand_scores, num_requests, num_src_beams,
                                               beam_width, stop_token, step, tokens_in, tokens_out, tok_cap,
                                               parents_out, cum_out, pool_scores, pool_lengths, pool_tokens,
                                               pool_count, pool_cap, stream));
}

bga_status bga_suffix_append(const bga_bf16 *new_k, const bga_bf16 *new_v, bga_bf16 *suffix_k, bga_bf16 *suffix_v,
                             int32_t num_requests, int32_t beam_width, int32_t pos, int32_t suffix_cap,
                             int32_t num_kv_heads, int32_t head_dim, hipStream_t stream)
{
    if (num_requests < 0 || beam_width < 0 || pos < 0 || pos >= suffix_cap || num_kv_heads <= 0) return BGA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return BGA_ERR_UNSUPPORTED;
    if (beam_width > BGA_MAX_BEAMS || suffix_cap > BGA_MAX_SUFFIX) return BGA_ERR_UNSUPPORTED;
    if ((int64_t)num_requests * beam_width > 0x7fffffff) return BGA_ERR_UNSUPPORTED;
    if (num_requests == 0 || beam_width == 0) return BGA_OK;
    if (!new_k || !new_v || !suffix_k || !suffix_v) return BGA_ERR_NULL;
    if (!aligned(new_k, 16) || !aligned(new_v, 16) || !aligned(suffix_k, 16) || !aligned(suffix_v, 16))
        return BGA_ERR_ALIGN;
    const size_t nb = (size_t)num_requests * beam_width * num_kv_heads * head_dim * 2;
    const size_t sb = nb * suffix_cap;
    if (overlap(suffix_k, sb, new_k, nb) || overlap(suffix_k, sb, new_v, nb) || overlap(suffix_v, sb, new_k, nb) ||
        overlap(suffix_v, sb, new_v, nb) || overlap(suffix_k, sb, suffix_v, sb))
        return BGA_ERR_ALIAS;
    return hip_status(bga::launch_suffix_append(new_k, new_v, suffix_k, suffix_v, num_requests, beam_width, pos,
                                                suffix_cap, num_kv_heads, head_dim, stream));
}

bga_status bga_beam_finalize(const float *pool_scores, const int32_t *pool_lengths, const int32_t *pool_tokens,
                             const int32_t *pool_count, int32_t pool_cap, const float *cum, const int32_t *tokens,
                             int32_t num_requests, int32_t beam_width, int32_t length, int32_t tok_cap,
                             float *final_scores, int32_t *final_lengths, int32_t *final_tokens,
                             int32_t *final_count, hipStream_t stream)
{
    if (num_requests < 0 || beam_width < 1 || pool_cap < 1 || length < 1 || length > tok_cap) return BGA_ERR_SHAPE;
    if ((int64_t)pool_cap + beam_width > bga::beam_final_max()) return BGA_ERR_UNSUPPORTED;
    if ((int64_t)num_requests * (pool_cap + beam_width) * tok_cap > 0x7fffffff) return BGA_ERR_UNSUPPORTED;
    if (num_requests == 0) return BGA_OK;
    if (!pool_scores || !pool_lengths || !pool_tokens || !pool_count || !cum || !tokens || !final_scores ||
        !final_lengths || !final_tokens || !final_count)
        return BGA_ERR_NULL;
    const void *ptrs[] = {pool_scores, pool_lengths, pool_tokens, pool_count, cum, tokens,
                          final_scores, final_lengths, final_tokens, final_count};
    for (const void *p : ptrs)
        if (!aligned(p, 4)) return BGA_ERR_ALIGN;
    return hip_status(bga::launch_beam_finalize(pool_scores, pool_lengths, pool_tokens, pool_count, pool_cap, cum,
                                                tokens, num_requests, beam_width, length, tok_cap, final_scores,
                                                final_lengths, final_tokens, final_count, stream));
}

bga_status bga_swiglu_quant_e4m3(const bga_bf16 *gate_up, int32_t num_tokens, int32_t inter_size, uint8_t *codes,
                                 float *scale, hipStream_t stream)
{
    if (num_tokens < 0 || inter_size < 8 || inter_size % 8) return BGA_ERR_SHAPE;
    if (inter_size > bga::swiglu_quant_max_inter()) return BGA_ERR_UNSUPPORTED;
    if (num_tokens == 0) return BGA_OK;
    if (!gate_up || !codes || !scale) return BGA_ERR_NULL;
    if (!aligned(gate_up, 16) || !aligned(codes, 8) || !aligned(scale, 4)) return BGA_ERR_ALIGN;
    const size_t in = (size_t)num_tokens * inter_size * 4, cb = (size_t)num_tokens * inter_size;
    if (overlap(codes, cb, gate_up, in) || overlap(scale, (size_t)num_tokens * 4, gate_up, in) ||
        overlap(scale, (size_t)num_tokens * 4, codes, cb))
        return BGA_ERR_ALIAS;
    return hip_status(bga::launch_swiglu_quant(gate_up, num_tokens, inter_size, codes, scale, stream));
}

const char *bga_status_string(bga_status s)
{
    switch (s) {
    case BGA_OK: return "BGA_OK";
    case BGA_ERR_NULL: return "BGA_ERR_NULL: a required pointer is NULL";
    case BGA_ERR_SHAPE: return "BGA_ERR_SHAPE: inconsistent or negative sizes";
    case BGA_ERR_UNSUPPORTED: return "BGA_ERR_UNSUPPORTED: head_dim, group size or a cap is not supported";
    case BGA_ERR_ALIGN: return "BGA_ERR_ALIGN: a pointer is not aligned as required";
    case BGA_ERR_WORKSPACE: return "BGA_ERR_WORKSPACE: workspace missing or too small";
    case BGA_ERR_ALIAS: return "BGA_ERR_ALIAS: an output overlaps an input";
    case BGA_ERR_HIP: return "BGA_ERR_HIP: a HIP launch failed";
    case BGA_ERR_PRECONDITION: return "BGA_ERR_PRECONDITION: a device-side precondition does not hold (debug build)";
    }
    return "unknown bga_status";
}

int32_t bga_last_hip_error(void) { return g_last_hip_error; }

int32_t bga_version(void) { return 200; }

int32_t bga_debug_build(void)
{
#ifdef BGA_DEBUG
    return 1;
#else
    return 0;
#endif
}

uint32_t bga_last_violations(void) { return g_last_violations; }

}  // extern "C"
