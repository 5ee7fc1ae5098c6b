/*
 * libbga — the attention hot path of a bounded-generation SLM inference engine,
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the Meituan engineering article
 * "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化":
 *   - packed variable-length causal GQA prefill       (section 3.1)
 *   - shared-prefix beam-search decode attention      (section 3.2)
 *   - parent-index suffix K/V and token reorder        (sections 3.2, 3.3)
 *   - two-stage beam candidate selection              (section 3.3)
 *
 * Conventions for every entry point
 *   - All tensors are row-major and contiguous, head_dim fastest.
 *   - bf16 tensors are passed as raw 16-bit patterns (bga_bf16).
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise. The
 *     caller owns all memory; the library allocates nothing, keeps no state
 *     between calls, never synchronizes, and only enqueues work on `stream`.
 *   - Outputs are fully overwritten within their declared extents; nothing
 *     outside them is written.
 *   - Problems that can be checked on the host (null pointers, sizes, caps,
 *     alignment, workspace size, overlapping buffers) return a nonzero status
 *     BEFORE any device call: nothing is enqueued. BGA_ERR_HIP reports a failed
 *     launch; bga_last_hip_error() then returns the hipError_t.
 *   - Preconditions on device data (valid cu_seqlens, parent indices in range,
 *     finite logits) are documented per call. The release library does not
 *     check them. The debug library (libbga_debug.so, built with BGA_DEBUG)
 *     checks them on the device before each operation: it waits for the check
 *     on `stream` (the only calls that synchronize) and, when one fails,
 *     returns BGA_ERR_PRECONDITION without launching the operation, with the
 *     failed checks in bga_last_violations().
 *   - Calls on different streams may run concurrently; the library is reentrant.
 */
#ifndef BGA_H
#define BGA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t bga_bf16; /* raw bfloat16 bits */

typedef enum {
    BGA_OK = 0,
    BGA_ERR_NULL = 1,        /* a required pointer is NULL */
    BGA_ERR_SHAPE = 2,       /* inconsistent or negative sizes */
    BGA_ERR_UNSUPPORTED = 3, /* head_dim, group size, or a cap not supported */
    BGA_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
    BGA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    BGA_ERR_ALIAS = 6,       /* output overlaps an input that must stay intact */
    BGA_ERR_HIP = 7,         /* a HIP launch failed; see bga_last_hip_error() */
    BGA_ERR_PRECONDITION = 8 /* debug build only: a device-side precondition does not hold;
                                see bga_last_violations(); nothing was computed */
} bga_status;

/* Bits of bga_last_violations(): the device-side preconditions a debug build checks. */
#define BGA_VIOLATION_CU_SEQLENS 1u  /* cu_seqlens[0] != 0, decreasing, or cu_seqlens[B] != total_tokens */
#define BGA_VIOLATION_MAX_SEQLEN 2u  /* a sequence is longer than max_seqlen */
#define BGA_VIOLATION_PARENT 4u      /* a parent index outside [0, W) */
#define BGA_VIOLATION_LOGITS 8u      /* a logit is inf or NaN */
#define BGA_VIOLATION_NO_KEYS 16u    /* a request's beams would attend to no key (empty prompt, no suffix) */

/* Caps (the article bounds its workloads to <= 400 beams, <= 5 generated
 * tokens and prompts averaging under 500 tokens, section 1.2). Each cap is
 * exercised on the GPU by the parity tests. */
#define BGA_MAX_GROUP 16        /* num_q_heads / num_kv_heads */
#define BGA_MAX_SEQLEN 8192     /* longest packed sequence; longest prompt */
#define BGA_MAX_BEAMS 512       /* beam_width / num_src_beams */
#define BGA_MAX_SUFFIX 16       /* suffix_cap */
#define BGA_MAX_K 1024          /* k_local and k_global */
#define BGA_MAX_VOCAB 163840    /* vocabulary size */

/*
 * Packed variable-length causal GQA prefill (article section 3.1: the packed
 * Q/K/V/O layout, the block-diagonal causal mask implied by the sequence
 * boundary, and the blocked K/V scan with an fp32 online-softmax state).
 *
 *   q        [T, num_q_heads,  head_dim]  bf16
 *   k, v     [T, num_kv_heads, head_dim]  bf16
 *   cu_seqlens [num_seqs + 1] int32: cu[0] = 0, non-decreasing, cu[num_seqs] =
 *            total_tokens = T. Sequence i owns rows cu[i] .. cu[i+1]-1. Zero-length
 *            sequences are allowed.
 *   max_seqlen >= every cu[i+1]-cu[i] (precondition; rows of a longer sequence
 *            beyond max_seqlen are not written), <= BGA_MAX_SEQLEN, and >= 1
 *            when total_tokens > 0 (else BGA_ERR_SHAPE).
 *   Query head h reads K/V head h / (num_q_heads / num_kv_heads).
 *   A query at position t of its sequence attends to positions 0..t of the
 *   same sequence; scores are softmax_scale * <q, k>.
 *   out      [T, num_q_heads, head_dim] bf16 (round to nearest even)
 *   lse      [T, num_q_heads] fp32, natural-log log-sum-exp of the scaled
 *            scores, or NULL.
 * Supported: head_dim in {64, 128}; num_q_heads % num_kv_heads == 0 with group
 * <= BGA_MAX_GROUP; num_seqs <= 65535; total_tokens * num_q_heads < 2^31. q, k,
 * v, out 16-byte aligned; lse and cu_seqlens 4-byte aligned.
 */
bga_status bga_packed_gqa_prefill(const bga_bf16 *q, const bga_bf16 *k, const bga_bf16 *v,
                                  const int32_t *cu_seqlens, int32_t num_seqs, int32_t total_tokens,
                                  int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, float softmax_scale, bga_bf16 *out, float *lse,
                                  hipStream_t stream);

/*
 * Shared-prefix beam decode attention (article section 3.2: one prompt K/V per
 * request, a short suffix K/V per beam, and
 *   O_b = Attention(Q_b, [prefix_K; suffix_K[b]], [prefix_V; suffix_V[b]])
 * evaluated in one fp32 online-softmax state without building the
 * concatenation).
 *
 *   q          [R, W, num_q_heads, head_dim] bf16 (one query token per beam)
 *   prefix_k/v [R, prefix_len, num_kv_heads, head_dim] bf16
 *   suffix_k/v [R, W, suffix_cap, num_kv_heads, head_dim] bf16; positions
 *              0 .. suffix_len-1 are read (suffix_len counts the current token).
 *   No mask: every prefix and suffix key precedes the query.
 *   out        [R, W, num_q_heads, head_dim] bf16
 *   lse        [R, W, num_q_heads] fp32 natural-log log-sum-exp, or NULL
 * Requires prefix_len + suffix_len >= 1, 0 <= suffix_len <= suffix_cap <=
 * BGA_MAX_SUFFIX, W <= BGA_MAX_BEAMS, head_dim in {64, 128}, group <=
 * BGA_MAX_GROUP, R * W * num_q_heads < 2^31; suffix pointers may be NULL only
 * when suffix_len == 0.
 * q, prefix, suffix and out 16-byte aligned; lse 4-byte aligned.
 */
bga_status bga_shared_prefix_decode(const bga_bf16 *q, const bga_bf16 *prefix_k, const bga_bf16 *prefix_v,
                                    const bga_bf16 *suffix_k, const bga_bf16 *suffix_v, int32_t num_requests,
                                    int32_t beam_width, int32_t prefix_len, int32_t suffix_len,
                                    int32_t suffix_cap, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, float softmax_scale, bga_bf16 *out, float *lse,
                                    hipStream_t stream);

/*
 * Shared-prefix beam decode with prompts of their own lengths, kept packed
 * (article section 3.2 equation, with the prompt K/V in the packed layout the
 * packed prefill of section 3.1 produces: the prefill's K/V output serves as
 * the shared prefix with no copy).
 *
 *   prefix_k/v   [total_prefix_tokens, num_kv_heads, head_dim] bf16: request r's
 *                prompt is rows prefix_cu[r] .. prefix_cu[r+1]-1
 *   prefix_cu    [num_requests + 1] int32, device: prefix_cu[0] = 0,
 *                non-decreasing, prefix_cu[R] = total_prefix_tokens, every prompt
 *                <= BGA_MAX_SEQLEN tokens, and >= 1 token when suffix_len == 0
 *                (preconditions, checked by the debug library)
 *   every other argument, the layouts and the results as in
 *   bga_shared_prefix_decode (which is this call with equal prompt lengths).
 * A request whose prompt is empty attends to its beams' suffixes only.
 */
bga_status bga_shared_prefix_decode_packed(const bga_bf16 *q, const bga_bf16 *prefix_k, const bga_bf16 *prefix_v,
                                           const int32_t *prefix_cu, int32_t total_prefix_tokens,
                                           const bga_bf16 *suffix_k, const bga_bf16 *suffix_v,
                                           int32_t num_requests, int32_t beam_width, int32_t suffix_len,
                                           int32_t suffix_cap, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, float softmax_scale, bga_bf16 *out, float *lse,
                                           hipStream_t stream);

/*
 * The last valid token of every packed sequence (article section 3.1: after
 * packed attention the same sequence boundary selects each sequence's
 * last-position hidden state, the input of the per-sample score head).
 *
 *   src        [total_tokens, row_bytes] (any element type: rows are copied
 *              bit for bit), e.g. hidden states [T, H] or attention output
 *              [T, Nq, D]
 *   cu_seqlens [num_seqs + 1] int32, device, as in bga_packed_gqa_prefill
 *   dst        [num_seqs, row_bytes]: row i = src row cu[i+1]-1; a
 *              zero-length sequence gets a row of zeros
 * row_bytes must be a positive multiple of 16; src and dst 16-byte aligned and
 * not overlapping. Source rows are clamped to [0, total_tokens) on the device.
 */
bga_status bga_last_token_gather(const void *src, const int32_t *cu_seqlens, int32_t num_seqs,
                                 int32_t total_tokens, int64_t row_bytes, void *dst, hipStream_t stream);

/*
 * Parent-index reorder (article sections 3.2 and 3.3: after candidate
 * selection only the retained beams' short suffix K/V, token history and
 * scores move; the prompt K/V never does).
 *
 *   src_k/src_v, dst_k/dst_v [R, W, suffix_cap, num_kv_heads, head_dim] bf16
 *   parent     [R, W] int32; new beam b of request r copies beam parent[r, b]
 *              (precondition 0 <= parent < W; an out-of-range parent yields
 *              zeros for that beam).
 *   Positions 0 .. suffix_len-1 are copied; positions >= suffix_len of dst are
 *   left untouched.
 *   src_tokens/dst_tokens [R, W, tok_cap] int32, optional (both NULL or both
 *   set): the first num_tokens entries of each beam are copied the same way.
 * Out of place: dst buffers must not overlap src buffers (BGA_ERR_ALIAS).
 * K/V pointers 16-byte aligned.
 */
bga_status bga_suffix_reorder(const bga_bf16 *src_k, const bga_bf16 *src_v, bga_bf16 *dst_k, bga_bf16 *dst_v,
                              const int32_t *parent, const int32_t *src_tokens, int32_t *dst_tokens,
                              int32_t num_requests, int32_t beam_width, int32_t suffix_len, int32_t suffix_cap,
                              int32_t num_kv_heads, int32_t head_dim, int32_t num_tokens, int32_t tok_cap,
                              hipStream_t stream);

/*
 * Fixed-depth beam search state update (article section 2.3, the loop
 * "prompt prefill -> first-step initialisation -> (N_gen - 1) x [decode ->
 * per-beam selection -> cumulative merge -> parent update -> token and suffix
 * K/V reorder] -> final candidates and scores"; section 3.3: 2W global
 * candidates are kept so that hypotheses that produced the stop token finish
 * while W beams continue). One step of the loop is
 *     bga_suffix_append (the current token's K/V) -> bga_shared_prefix_decode
 *     (or _packed) -> [the model: logits] -> bga_beam_topk with k_local =
 *     k_global = 2W -> bga_beam_advance -> bga_suffix_reorder by the new parents;
 * the first step (step = 0) selects from the prompt's last-token logits with
 * num_src_beams = 1 and no cumulative scores, and bga_beam_finalize ranks the
 * result after the last step.
 */

/*
 * The 2W rule on the global candidates of one step, per request. Of the 2W
 * candidates (bga_beam_topk output with k_global = 2W, best first), every one
 * whose token is stop_token becomes a finished hypothesis: appended to the
 * request's pool with its score, length step + 1 and tokens (its source beam's
 * step tokens, then stop_token). The first W others become the new beams in
 * candidate order: parents_out, cum_out (their scores) and tokens_out (the
 * source beam's step tokens, then the new token). Each source beam's candidates
 * hold distinct tokens, so at most num_src_beams <= W of them are stop tokens
 * and the W beams always fill.
 *
 *   cand_tokens, cand_parents [R, 2W] int32; cand_scores [R, 2W] fp32
 *   tokens_in  [R, num_src_beams, tok_cap] int32 (positions < step are read)
 *   tokens_out [R, W, tok_cap] (positions <= step are written); must not
 *              overlap tokens_in
 *   parents_out [R, W] int32; cum_out [R, W] fp32
 *   pool_scores [R, pool_cap] fp32, pool_lengths [R, pool_cap] int32,
 *   pool_tokens [R, pool_cap, tok_cap] int32, pool_count [R] int32: the
 *              finished pool. At step 0 the pool is taken as empty (pool_count
 *              need not be initialised); later steps append after pool_count.
 *              Hypotheses beyond pool_cap are dropped (W x N_gen always
 *              suffices).
 * Requires 1 <= W <= BGA_MAX_BEAMS, 1 <= num_src_beams <= W, 0 <= step and
 * step < tok_cap, pool_cap >= 1; all pointers 4-byte aligned.
 */
bga_status bga_beam_advance(const int32_t *cand_tokens, const int32_t *cand_parents, const float *cand_scores,
                            int32_t num_requests, int32_t num_src_beams, int32_t beam_width, int32_t stop_token,
                            int32_t step, const int32_t *tokens_in, int32_t *tokens_out, int32_t tok_cap,
                            int32_t *parents_out, float *cum_out, float *pool_scores, int32_t *pool_lengths,
                            int32_t *pool_tokens, int32_t *pool_count, int32_t pool_cap, hipStream_t stream);

/*
 * The current token's K/V of every beam into suffix position `pos` (the K/V
 * projection of the token each beam selected at the previous step).
 *   new_k, new_v [R, W, num_kv_heads, head_dim] bf16
 *   suffix_k, suffix_v [R, W, suffix_cap, num_kv_heads, head_dim] bf16, written
 *   at position pos only. Requires 0 <= pos < suffix_cap <= BGA_MAX_SUFFIX;
 *   16-byte aligned; new and suffix buffers must not overlap.
 */
bga_status bga_suffix_append(const bga_bf16 *new_k, const bga_bf16 *new_v, bga_bf16 *suffix_k, bga_bf16 *suffix_v,
                             int32_t num_requests, int32_t beam_width, int32_t pos, int32_t suffix_cap,
                             int32_t num_kv_heads, int32_t head_dim, hipStream_t stream);

/*
 * Final candidates and scores: per request, the finished pool and the last W
 * beams (cum [R, W], tokens [R, W, tok_cap] of length `length`) ranked together
 * by score, best first (equal scores: finished before beams, earlier before
 * later, lower beam first; no length normalisation).
 *   final_scores [R, pool_cap + W] fp32, final_lengths [R, pool_cap + W] int32,
 *   final_tokens [R, pool_cap + W, tok_cap] int32, final_count [R] int32
 *   (= pool_count + W; entries past it are not written).
 * Requires pool_cap + W <= 8192, 1 <= length <= tok_cap.
 */
bga_status bga_beam_finalize(const float *pool_scores, const int32_t *pool_lengths, const int32_t *pool_tokens,
                             const int32_t *pool_count, int32_t pool_cap, const float *cum, const int32_t *tokens,
                             int32_t num_requests, int32_t beam_width, int32_t length, int32_t tok_cap,
                             float *final_scores, int32_t *final_lengths, int32_t *final_tokens,
                             int32_t *final_count, hipStream_t stream);

/* Bytes of device workspace bga_beam_topk needs for these sizes (0 on bad sizes). */
size_t bga_beam_topk_workspace_size(int32_t num_requests, int32_t num_src_beams, int32_t vocab,
                                    int32_t k_local, int32_t k_global);

/*
 * Two-stage beam candidate selection (article section 3.3):
 *  stage 1, per source beam row (r, b): the k_local token ids with the largest
 *    bf16 logits (equal logits: lower id first; -0 equals +0), ranked;
 *    lse = fp32 log-sum-exp of the row over the full vocabulary (float
 *    logits); lp = x - lse and score = cum[r, b] + lp, each one fp32 operation.
 *  stage 2, per request: the W_in * k_local candidates flattened as
 *    f = b * k_local + j; the k_global best scores (equal scores: lower f
 *    first), sorted best first; parent = f / k_local; token = the stage-1 id at
 *    (parent, f % k_local); out score = that candidate's score (the new
 *    cumulative score).
 *
 *   logits     [R, W_in, vocab] bf16, finite (precondition)
 *   cum_scores [R, W_in] fp32, or NULL for all zero (first step)
 *   out_tokens, out_parents [R, k_global] int32; out_scores [R, k_global] fp32
 *   local_tokens [R, W_in, k_local] int32 and local_scores fp32: optional
 *   row_lse    [R, W_in] fp32: optional
 *   workspace  device memory of >= bga_beam_topk_workspace_size(...) bytes,
 *              16-byte aligned; its contents on entry do not matter.
 * Requires 1 <= k_local <= min(vocab, BGA_MAX_K), 1 <= k_global <=
 * min(W_in * k_local, BGA_MAX_K), W_in <= BGA_MAX_BEAMS, vocab <= BGA_MAX_VOCAB.
 * logits 16-byte aligned; vocab % 8 == 0 is the fast path.
 */
bga_status bga_beam_topk(const bga_bf16 *logits, const float *cum_scores, int32_t num_requests,
                         int32_t num_src_beams, int32_t vocab, int32_t k_local, int32_t k_global,
                         int32_t *out_tokens, int32_t *out_parents, float *out_scores, int32_t *local_tokens,
                         float *local_scores, float *row_lse, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Size of the library's own per-device top-K workspace used by
 * bga_beam_topk_noalloc. */
#define BGA_TOPK_SCRATCH_BYTES ((size_t)24 << 20)

/*
 * bga_beam_topk for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc): the same
 * operation, arguments and results, with the stage-1 lists kept in a workspace
 * the library owns instead of a caller-provided one. No allocation of any kind
 * happens in this call; the caller still passes every input and output.
 *
 * The workspace is one array of BGA_TOPK_SCRATCH_BYTES per device, resident
 * from the library's first use on that device until the process ends. Sizes
 * whose bga_beam_topk_workspace_size() exceeds it return BGA_ERR_WORKSPACE
 * (8 x 400 source beams with k_local = 800 need 20.5 MB and fit). Every call on
 * one device shares that array: calls that overlap on one device (different
 * streams, or host threads) race and must be serialised by the caller; calls
 * on different devices do not interact.
 */
bga_status bga_beam_topk_noalloc(const bga_bf16 *logits, const float *cum_scores, int32_t num_requests,
                                 int32_t num_src_beams, int32_t vocab, int32_t k_local, int32_t k_global,
                                 int32_t *out_tokens, int32_t *out_parents, float *out_scores,
                                 int32_t *local_tokens, float *local_scores, float *row_lse, hipStream_t stream);

/*
 * Fused SwiGLU requantisation to FP8 E4M3 with a per-token dynamic scale
 * (article section 3.4: after the FP8 Gate/Up projection, one pass per token
 * computes SiLU(gate) * up in fp32, the amax reduction, the scale and the E4M3
 * requantisation the FP8 Down projection reads, without writing a bf16 SwiGLU
 * intermediate).
 *
 *   gate_up [T, 2 * inter_size] bf16: per token, gate in columns
 *           0 .. inter_size-1, up in inter_size .. 2*inter_size-1
 *   codes   [T, inter_size] uint8, OCP FP8 E4M3 (e4m3fn) codes of
 *           h * 448 / amax, h = gate / (1 + e^-gate) * up, amax = max(max |h|,
 *           1e-12), round to nearest even
 *   scale   [T] fp32: amax / 448, so that h ~= code * scale
 * Requires inter_size % 8 == 0 and 8 <= inter_size <= 16384; gate_up 16-byte
 * aligned, codes 8-byte aligned, scale 4-byte aligned; gate_up finite
 * (precondition).
 */
bga_status bga_swiglu_quant_e4m3(const bga_bf16 *gate_up, int32_t num_tokens, int32_t inter_size, uint8_t *codes,
                                 float *scale, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *bga_status_string(bga_status s);

/* hipError_t of the most recent BGA_ERR_HIP on the calling thread (0 if none). */
int32_t bga_last_hip_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t bga_version(void);

/* 1 in the debug library (device-side precondition checks), 0 in the release library. */
int32_t bga_debug_build(void);

/* BGA_VIOLATION_* bits of the most recent BGA_ERR_PRECONDITION on the calling thread (0 if none). */
uint32_t bga_last_violations(void);

#ifdef __cplusplus
}
#endif

#endif /* BGA_H */
