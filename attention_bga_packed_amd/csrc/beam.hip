// State update of the fixed-depth beam search for gfx950: the stop-token rule
// on the global candidates, the current token's K/V append, and the final
// ranking.
//
// Article section 2.3 (the loop: prompt prefill -> first-step initialisation
// -> (N_gen - 1) x [decode -> per-beam selection -> cumulative merge -> parent
// update -> token and suffix K/V reorder] -> final candidates and scores) and
// section 3.3 (2W global candidates, so that hypotheses that produced the stop
// token finish while W beams continue; only the retained state moves).
//
//   advance:  one workgroup per request over its 2W candidates (best first).
//             Two block-wide exclusive counts give each candidate its place:
//             a stop-token candidate goes to the request's finished pool (its
//             source beam's tokens plus the stop token), any other takes the
//             next beam slot while fewer than W are taken. Each source beam's
//             stage-1 list holds distinct tokens, so at most W_in <= W of the
//             2W are stop tokens and the W slots always fill. The new beams'
//             token lists are written here (the source beam's tokens plus the
//             new one); their suffix K/V move with the reorder kernel.
//   append:   the current token's K/V of every beam into suffix position pos.
//   finalize: one workgroup per request ranks its finished hypotheses and its
//             last W beams together by score (ties: finished before beams,
//             earlier first), each entry's place being the count of entries
//             ahead of it, and writes them best first.
#include "device_common.hpp"
#include "internal.hpp"

namespace bga {

constexpr int BEAM_THREADS = 1024;

// Block-wide exclusive prefix count of `flag` over threads in id order; *total
// receives the block's count. Uses sh[0 .. 16].
__device__ __forceinline__ uint32_t block_exclusive_count(bool flag, uint32_t *sh, uint32_t *total)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
    const unsigned long long m = __ballot(flag);
    const uint32_t in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (lane == 0) sh[w] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int i = 0; i < nw; ++i) {
        const uint32_t c = sh[i];
        before += i < w ? c : 0u;
        all += c;
    }
    __syncthreads();   // sh may be reused by the caller
    *total = all;
    return before + in_wave;
}

__global__ __launch_bounds__(BEAM_THREADS) void beam_advance_kernel(
    const int32_t *__restrict__ cand_tok, const int32_t *__restrict__ cand_par, const float *__restrict__ cand_score,
    int K2, int W_in, int W, int stop, int step, const int32_t *__restrict__ tok_in, int32_t *__restrict__ tok_out,
    int tok_cap, int32_t *__restrict__ parents_out, float *__restrict__ cum_out, float *__restrict__ pool_score,
    int32_t *__restrict__ pool_len, int32_t *__restrict__ pool_tok, int32_t *__restrict__ pool_count, int pool_cap)
{
    __shared__ uint32_t sh[17];
    const int r = blockIdx.x, tid = threadIdx.x;
    const bool have = tid < K2;
    const int32_t tok = have ? cand_tok[(size_t)r * K2 + tid] : 0;
    const int32_t par = have ? min(max(cand_par[(size_t)r * K2 + tid], 0), W_in - 1) : 0;
    const float score = have ? cand_score[(size_t)r * K2 + tid] : 0.f;
    const bool is_stop = have && tok == stop;
    // the pool starts empty at the first step; a count read back is kept inside the pool
    const int count0 = step == 0 ? 0 : min(max(pool_count[r], 0), pool_cap);
    uint32_t n_stop = 0, n_keep = 0;
    const uint32_t stop_at = block_exclusive_count(is_stop, sh, &n_stop);
    const uint32_t keep_at = block_exclusive_count(have && !is_stop, sh, &n_keep);
    const int32_t *src = tok_in + ((size_t)r * W_in + par) * tok_cap;
    if (have && !is_stop && keep_at < (uint32_t)W) {
        const size_t b = (size_t)r * W + keep_at;
        parents_out[b] = par;
        cum_out[b] = score;
        int32_t *dst = tok_out + b * tok_cap;
        for (int i = 0; i < step; ++i) dst[i] = src[i];
        dst[step] = tok;
    }
    if (is_stop) {
        const int slot = count0 + (int)stop_at;
        if (slot < pool_cap) {
            const size_t p = (size_t)r * pool_cap + slot;
            pool_score[p] = score;
            pool_len[p] = step + 1;
            int32_t *dst = pool_tok + p * tok_cap;
            for (int i = 0; i < step; ++i) dst[i] = src[i];
            dst[step] = tok;
        }
    }
    __syncthreads();   // every thread has read pool_count[r]
    if (tid == 0) pool_count[r] = min(count0 + (int)n_stop, pool_cap);
}

__global__ __launch_bounds__(256) void suffix_append_kernel(const u32x4 *__restrict__ new_k,
                                                            const u32x4 *__restrict__ new_v, u32x4 *__restrict__ sk,
                                                            u32x4 *__restrict__ sv, int row16, int pos, int cap)
{
    const size_t rb = blockIdx.x;   // r * W + b
    const u32x4 *ak = new_k + rb * row16, *av = new_v + rb * row16;
    u32x4 *dk = sk + (rb * cap + pos) * row16, *dv = sv + (rb * cap + pos) * row16;
    for (int i = threadIdx.x; i < row16; i += 256) {
        const u32x4 a = ak[i], b = av[i];
        dk[i] = a;
        dv[i] = b;
    }
}

constexpr int FINAL_MAX = 8192;   // finished hypotheses + beams ranked per request

__global__ __launch_bounds__(BEAM_THREADS) void beam_finalize_kernel(
    const float *__restrict__ pool_score, const int32_t *__restrict__ pool_len, const int32_t *__restrict__ pool_tok,
    const int32_t *__restrict__ pool_count, int pool_cap, const float *__restrict__ cum, const int32_t *__restrict__ tok,
    int W, int len, int tok_cap, float *__restrict__ final_score, int32_t *__restrict__ final_len,
    int32_t *__restrict__ final_tok, int32_t *__restrict__ final_count)
{
    __shared__ float sc[FINAL_MAX];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int np = min(max(pool_count[r], 0), pool_cap);
    const int n = np + W;
    for (int i = tid; i < n; i += BEAM_THREADS)
        sc[i] = i < np ? pool_score[(size_t)r * pool_cap + i] : cum[(size_t)r * W + (i - np)];
    __syncthreads();
    const int fcap = pool_cap + W;
    for (int i = tid; i < n; i += BEAM_THREADS) {
        const float s = sc[i];
        int place = 0;
        for (int j = 0; j < n; ++j) {
            const float t = sc[j];
            place += (t > s || (t == s && j < i)) ? 1 : 0;
        }
        const size_t o = (size_t)r * fcap + place;
        final_score[o] = s;
        const int32_t *src;
        int l;
        if (i < np) {
            src = pool_tok + ((size_t)r * pool_cap + i) * tok_cap;
            l = pool_len[(size_t)r * pool_cap + i];
        } else {
            src = tok + ((size_t)r * W + (i - np)) * tok_cap;
            l = len;
        }
        l = min(max(l, 0), tok_cap);
        final_len[o] = l;
        int32_t *dst = final_tok + o * tok_cap;
        for (int k = 0; k < l; ++k) dst[k] = src[k];
    }
    if (tid == 0) final_count[r] = n;
}

hipError_t launch_beam_advance(const int32_t *cand_tok, const int32_t *cand_par, const float *cand_score, int R,
                               int W_in, int W, int stop, int step, const int32_t *tok_in, int32_t *tok_out,
                               int tok_cap, int32_t *parents_out, float *cum_out, float *pool_score,
                               int32_t *pool_len, int32_t *pool_tok, int32_t *pool_count, int pool_cap,
                               hipStream_t stream)
{
    hipLaunchKernelGGL(beam_advance_kernel, dim3(R), dim3(BEAM_THREADS), 0, stream, cand_tok, cand_par, cand_score,
                       2 * W, W_in, W, stop, step, tok_in, tok_out, tok_cap, parents_out, cum_out, pool_score,
                       pool_len, pool_tok, pool_count, pool_cap);
    return hipGetLastError();
}

hipError_t launch_suffix_append(const uint16_t *new_k, const uint16_t *new_v, uint16_t *sk, uint16_t *sv, int R, int W,
                                int pos, int cap, int nkv, int d, hipStream_t stream)
{
    const int row16 = nkv * d / 8;
    hipLaunchKernelGGL(suffix_append_kernel, dim3(R * W), dim3(256), 0, stream, (const u32x4 *)new_k,
                       (const u32x4 *)new_v, (u32x4 *)sk, (u32x4 *)sv, row16, pos, cap);
    return hipGetLastError();
}

int beam_final_max() { return FINAL_MAX; }

hipError_t launch_beam_finalize(const float *pool_score, const int32_t *pool_len, const int32_t *pool_tok,
                                const int32_t *pool_count, int pool_cap, const float *cum, const int32_t *tok, int R,
                                int W, int len, int tok_cap, float *final_score, int32_t *final_len,
                                int32_t *final_tok, int32_t *final_count, hipStream_t stream)
{
    hipLaunchKernelGGL(beam_finalize_kernel, dim3(R), dim3(BEAM_THREADS), 0, stream, pool_score, pool_len, pool_tok,
                       pool_count, pool_cap, cum, tok, W, len, tok_cap, final_score, final_len, final_tok,
                       final_count);
    return hipGetLastError();
}

}  // namespace bga
