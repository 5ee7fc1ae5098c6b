// Host-side launchers of libbga's kernels. Arguments are validated by the
// C-ABI layer (bga_abi.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace bga {

// Every launcher returns hipSuccess or the launch error.

hipError_t launch_packed_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *cu,
                                 int num_seqs, int total_tokens, int max_seqlen, int nq, int nkv, int d, float scale,
                                 uint16_t *out, float *lse, hipStream_t stream);

// prefix_cu == nullptr: prompts of Lp tokens at [R, Lp, Nkv, D]; else request r's
// prompt is rows prefix_cu[r] .. prefix_cu[r+1]-1 of a packed [T_p, Nkv, D].
hipError_t launch_shared_prefix_decode(const uint16_t *q, const uint16_t *pk, const uint16_t *pv,
                                       const int32_t *prefix_cu, const uint16_t *sk, const uint16_t *sv, int R,
                                       int W, int Lp, int Ls, int Ls_cap, int nq, int nkv, int d, float scale,
                                       uint16_t *out, float *lse, hipStream_t stream);

hipError_t launch_last_token_gather(const void *src, const int32_t *cu, int num_seqs, int T, int64_t row_bytes,
                                    void *dst, hipStream_t stream);

hipError_t launch_suffix_reorder(const uint16_t *src_k, const uint16_t *src_v, uint16_t *dst_k, uint16_t *dst_v,
                                 const int32_t *parent, const int32_t *src_tok, int32_t *dst_tok, int R, int W,
                                 int Ls, int Ls_cap, int nkv, int d, int ntok, int tok_cap, hipStream_t stream);

// Workspace layout of the beam top-K (offsets in bytes, 256-byte aligned parts).
struct TopkWorkspace {
    size_t local_tok;    // int32 [R, W_in, k_local]
    size_t local_score;  // float [R, W_in, k_local]
    size_t total;
};
TopkWorkspace topk_workspace_layout(int R, int W_in, int k_local);

// Device address of the current device's BGA_TOPK_SCRATCH_BYTES of library-owned
// top-K workspace (looked up once per device, then cached).
hipError_t topk_scratch(void **ptr);

hipError_t launch_beam_topk(const uint16_t *logits, const float *cum, int R, int W_in, int V, int k_local,
                            int k_global, int32_t *out_tok, int32_t *out_par, float *out_score,
                            int32_t *local_tok, float *local_score, float *row_lse, void *workspace,
                            hipStream_t stream);

// Beam-search state update (beam.hip).
hipError_t launch_beam_advance(const int32_t *cand_tok, const int32_t *cand_par, const float *cand_score, int R,
                               int W_in, int W, int stop, int step, const int32_t *tok_in, int32_t *tok_out,
                               int tok_cap, int32_t *parents_out, float *cum_out, float *pool_score,
                               int32_t *pool_len, int32_t *pool_tok, int32_t *pool_count, int pool_cap,
                               hipStream_t stream);
hipError_t launch_suffix_append(const uint16_t *new_k, const uint16_t *new_v, uint16_t *sk, uint16_t *sv, int R, int W,
                                int pos, int cap, int nkv, int d, hipStream_t stream);
int beam_final_max();
hipError_t launch_beam_finalize(const float *pool_score, const int32_t *pool_len, const int32_t *pool_tok,
                                const int32_t *pool_count, int pool_cap, const float *cum, const int32_t *tok, int R,
                                int W, int len, int tok_cap, float *final_score, int32_t *final_len,
                                int32_t *final_tok, int32_t *final_count, hipStream_t stream);

// Fused SwiGLU requantisation (swiglu_fp8.hip); I % 8 == 0, I <= swiglu_quant_max_inter().
int swiglu_quant_max_inter();
hipError_t launch_swiglu_quant(const uint16_t *gate_up, int T, int I, uint8_t *codes, float *scale,
                               hipStream_t stream);

#ifdef BGA_DEBUG
// Debug build: device-side precondition checks (debug_checks.hip). Each runs a
// check kernel on `stream`, waits for it and returns the BGA_VIOLATION_* bits
// found in *violations.
hipError_t debug_check_prefill(const int32_t *cu, int B, int T, int max_seqlen, hipStream_t stream,
                               uint32_t *violations);
// cu_seqlens-style offsets of packed prompts; also flags a request with no key
// at all (an empty prompt when suffix_len == 0)
hipError_t debug_check_prompts(const int32_t *cu, int R, int T, int max_len, bool need_nonempty, hipStream_t stream,
                               uint32_t *violations);
hipError_t debug_check_parents(const int32_t *parent, int n, int W, hipStream_t stream, uint32_t *violations);
hipError_t debug_check_logits(const uint16_t *x, size_t n, hipStream_t stream, uint32_t *violations);
#endif

// Raise a kernel's dynamic-LDS limit to `bytes`, once per device: `done`
// (one per kernel) keeps a bit per device that has been set up.
inline hipError_t dynamic_lds_once(const void *kern, int bytes, std::atomic<uint64_t> &done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

}  // namespace bga
