// Two-stage beam candidate selection for gfx950.
//
// Article section 3.3 ("Beam 候选计算与状态更新"):
//   bf16 logits [W, V] -> per beam the 2W best token ids (chosen on the bf16
//   logits: log-softmax is strictly increasing within a row, so ranking by
//   logit ranks by log-probability) -> fp32 log-probabilities of those ids from
//   the full-vocabulary fp32 log-softmax -> plus each beam's cumulative score ->
//   flatten W x 2W -> global selection; the flat index gives the parent beam
//   and the slot within it. Cutting each beam at 2W loses nothing: a token
//   ranked below 2W in its own beam has 2W better candidates ahead of it.
//
// Keys. A bf16 logit maps to a 16-bit key that orders like the value (-0 is
// +0); key 0 is the NaN pattern 0xffff and marks "no element". An fp32 score
// maps to a 32-bit key the same way.
//
// Stage 1 (one 256-thread workgroup per beam row, several per CU):
//   pass 1 streams the row from HBM once. Each wave keeps its running maximum
//   key M_w, an fp64 sum of exp(x - M_w) per lane (fp32 exponentials, rescaled
//   when M_w grows) and an exact histogram of the 256 keys [M_w - 255, M_w]
//   (shifted when M_w grows; keys below the window can never re-enter it).
//   The waves' windows merge exactly into the histogram of [M - 255, M], M the
//   row maximum, from which the cut key kappa (the k-th largest) and the number
//   of keys above it follow directly. If the window holds fewer than k keys a
//   generic two-digit radix select over the row is used instead.
//   pass 2 re-reads the row (from cache) and gathers every key >= kappa; a
//   bitonic sort by (key desc, id asc) then puts the k winners first, which
//   also breaks ties at kappa by lower id. If too many keys equal kappa to fit,
//   ties are ranked by id with a block scan in id order instead.
// Stage 2 (one workgroup per request): each beam's list is sorted, so only its
// first min(k_local, k_global) entries can matter and the entries above any
// threshold form a prefix. A lower bound comes from the first J entries of
// every beam, prefix lengths from binary searches, the exact cut from a radix
// select over 32-bit score keys, ties by lower flat index, and a final bitonic
// sort by (score desc, flat index asc).
#include "device_common.hpp"
#include "internal.hpp"

namespace bga {

constexpr int TK1_THREADS = 256;   // stage 1: one workgroup per beam row
constexpr int TK1_WAVES = TK1_THREADS / 64;
constexpr int TK1_UNROLL = 4;      // 16-byte chunks in flight per thread
constexpr int TK_WIN = 256;        // keys per histogram window
constexpr int TK_LIST = 2048;      // gathered candidates (>= k + ties)
constexpr int TK2_THREADS = 1024;  // stage 2: one workgroup per request, one beam per thread

__device__ __forceinline__ uint32_t key16(uint32_t b)
{
    b = (b == 0x8000u) ? 0u : b;
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}

__device__ __forceinline__ float key16_value(uint32_t key)
{
    const uint32_t b = (key & 0x8000u) ? (key & 0x7fffu) : (~key & 0xffffu);
    return __uint_as_float(b << 16);
}

__device__ __forceinline__ uint32_t key32(float f)
{
    uint32_t b = __float_as_uint(f);
    b = (b == 0x80000000u) ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---- block-wide helpers ------------------------------------------------------

struct TkCommon {
    uint32_t hist[256];
    uint32_t wsum[16];
    uint32_t bcast[4];
};

// Given a 256-bin histogram (bins ordered by digit), find the bin holding the
// k-th largest element (1-based k): bcast[0] = bin, bcast[1] = elements in
// higher bins, bcast[2] = elements in that bin. Requires total >= k and
// blockDim.x >= 256.
__device__ __forceinline__ void select_bin(TkCommon &sh, const uint32_t *hist, uint32_t k)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint32_t c = 0, incl = 0;
    if (tid < 256) {
        c = hist[255 - tid];
        incl = wave_incl_scan_u32(c);
        if (lane == 63) sh.wsum[w] = incl;
    }
    __syncthreads();
    if (tid < 256) {
        uint32_t pre = 0;
        for (int i = 0; i < w; ++i) pre += sh.wsum[i];
        const uint32_t hi = pre + incl, lo = hi - c;
        if (lo < k && hi >= k) {
            sh.bcast[0] = 255 - tid;
            sh.bcast[1] = lo;
            sh.bcast[2] = c;
        }
    }
    __syncthreads();
}

// Exact radix select of the k-th largest key over the elements `each` visits
// (each(fn) calls fn(key) for every element of this thread). NPASS 8-bit
// digits, most significant first. Returns the key; *above = number of visited
// keys strictly greater, *equal = number equal to it.
template <int NPASS, typename Each>
__device__ __forceinline__ uint32_t radix_select(TkCommon &sh, Each each, uint32_t k, uint32_t *above,
                                                 uint32_t *equal)
{
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0, krem = k, abv = 0, eq = 0;
#pragma unroll 1
    for (int pass = 0; pass < NPASS; ++pass) {
        const int shift = 8 * (NPASS - 1 - pass);
        for (int i = tid; i < 256; i += blockDim.x) sh.hist[i] = 0;
        __syncthreads();
        each([&](uint32_t key) {
            if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        select_bin(sh, sh.hist, krem);
        const uint32_t bin = sh.bcast[0], ab = sh.bcast[1];
        eq = sh.bcast[2];
        __syncthreads();
        abv += ab;
        krem -= ab;
        prefix |= bin << shift;
        mask |= 255u << shift;
    }
    *above = abv;
    *equal = eq;
    return prefix;
}

// Exclusive prefix sum over the workgroup's threads; returns this thread's
// exclusive value, *total the sum.
__device__ __forceinline__ uint32_t block_excl_scan(TkCommon &sh, uint32_t x, uint32_t *total)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
    const uint32_t incl = wave_incl_scan_u32(x);
    if (lane == 63) sh.wsum[w] = incl;
    __syncthreads();
    uint32_t pre = 0, tot = 0;
    for (int i = 0; i < nw; ++i) {
        const uint32_t s = sh.wsum[i];
        pre += i < w ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return pre + incl - x;
}

// Bitonic sort of list[0..n) (n a power of two) into descending order.
__device__ __forceinline__ void bitonic_desc(unsigned long long *list, int n)
{
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < n; t += blockDim.x) {
                const int p = t ^ stride;
                if (p > t) {
                    const unsigned long long a = list[t], b = list[p];
                    const bool desc = (t & size) == 0;
                    if (desc ? (a < b) : (a > b)) {
                        list[t] = b;
                        list[p] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int pow2_at_least(int n)
{
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// ---- stage 1 ----------------------------------------------------------------

struct Tk1Shared {
    TkCommon c;
    uint32_t whist[TK1_WAVES][TK_WIN];   // per-wave window histograms
    uint32_t wmax[TK1_WAVES];
    double dsum[TK1_WAVES];
    unsigned long long list[TK_LIST];
    uint32_t count;
};

// Row chunk c (8 logits, ids 8c .. 8c+7) as four packed key pairs; missing
// logits get key 0.
template <bool VEC>
__device__ __forceinline__ u32x4 load_keys(const uint16_t *__restrict__ x, int c, int V, int nchunks)
{
    u32x4 raw = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    if (c < nchunks) {
        if (VEC) {
            raw = *(const u32x4 *)(x + (size_t)c * 8);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int id = c * 8 + j;
                const uint32_t b = id < V ? (uint32_t)x[id] : 0xffffu;
                raw[j / 2] = (j & 1) ? ((raw[j / 2] & 0xffffu) | (b << 16)) : ((raw[j / 2] & 0xffff0000u) | b);
            }
        }
    }
    u32x4 k;
#pragma unroll
    for (int e = 0; e < 4; ++e) k[e] = key16(raw[e] & 0xffffu) | (key16(raw[e] >> 16) << 16);
    return k;
}

template <bool VEC>
__global__ __launch_bounds__(TK1_THREADS) void topk_stage1_kernel(const uint16_t *__restrict__ logits,
                                                                  const float *__restrict__ cum, int V,
                                                                  int k_local, int32_t *__restrict__ ws_tok,
                                                                  float *__restrict__ ws_score,
                                                                  int32_t *__restrict__ local_tok,
                                                                  float *__restrict__ local_score,
                                                                  float *__restrict__ row_lse)
{
    __shared__ Tk1Shared sh;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const size_t row = blockIdx.x;
    const uint16_t *x = logits + row * (size_t)V;
    const int nchunks = (V + 7) / 8;
    const int nrows = (nchunks + TK1_THREADS - 1) / TK1_THREADS;   // chunk rows, id order
    const uint32_t k = (uint32_t)k_local;

    for (int i = lane; i < TK_WIN; i += 64) sh.whist[w][i] = 0;

    // ---- pass 1: running max, log-sum-exp and window histogram, per wave
    uint32_t mw = 0;          // wave running max key (0: nothing seen yet)
    float mwv = 0.f;          // its value
    double acc = 0.0;         // sum of exp(x - mwv) over this lane's logits
    uint32_t *hist = sh.whist[w];
    for (int i0 = 0; i0 < nrows; i0 += TK1_UNROLL) {
        u32x4 kk[TK1_UNROLL];
#pragma unroll
        for (int u = 0; u < TK1_UNROLL; ++u) kk[u] = load_keys<VEC>(x, (i0 + u) * TK1_THREADS + tid, V, nchunks);
        uint32_t lm = 0;
#pragma unroll
        for (int u = 0; u < TK1_UNROLL; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) lm = max(lm, max(kk[u][e] & 0xffffu, kk[u][e] >> 16));
        const uint32_t nm = wave_max_u32(lm);
        if (nm > mw) {  // wave-uniform
            const float nmv = key16_value(nm);
            if (mw != 0) acc *= exp((double)mwv - (double)nmv);
            // shift the window so that it ends at the new maximum
            const uint32_t d = nm - mw;
            uint32_t vals[TK_WIN / 64];
#pragma unroll
            for (int j = 0; j < TK_WIN / 64; ++j) {
                const uint32_t src = (uint32_t)(lane * (TK_WIN / 64) + j) + d;
                vals[j] = (mw != 0 && src < TK_WIN) ? hist[src] : 0u;
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < TK_WIN / 64; ++j) hist[lane * (TK_WIN / 64) + j] = vals[j];
            __builtin_amdgcn_wave_barrier();
            mw = nm;
            mwv = nmv;
        }
        const uint32_t base = mw > TK_WIN - 1 ? mw - (TK_WIN - 1) : 1u;
        const float mlog = mwv * kLog2e;
#pragma unroll
        for (int u = 0; u < TK1_UNROLL; ++u) {
            float cs = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t key = (kk[u][e] >> (16 * h)) & 0xffffu;
                    const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(key16_value(key), kLog2e, -mlog));
                    cs += key ? t : 0.f;
                    if (key >= base) atomicAdd(&hist[key - base], 1u);
                }
            acc += (double)cs;
        }
    }

    // ---- merge the waves: row max, log-sum-exp, window histogram of [M-255, M]
    if (lane == 0) sh.wmax[w] = mw;
    __syncthreads();
    uint32_t M = 0;
#pragma unroll
    for (int i = 0; i < TK1_WAVES; ++i) M = max(M, sh.wmax[i]);
    const float Mv = key16_value(M);
    acc = wave_sum_f64(acc);
    if (lane == 0) sh.dsum[w] = (mw != 0) ? acc * exp((double)mwv - (double)Mv) : 0.0;
    const uint32_t gbase = M > TK_WIN - 1 ? M - (TK_WIN - 1) : 1u;
    for (int b = tid; b < TK_WIN; b += TK1_THREADS) {
        uint32_t s = 0;
        const uint32_t key = gbase + b;
#pragma unroll
        for (int i = 0; i < TK1_WAVES; ++i) {
            const uint32_t mwi = sh.wmax[i];
            const uint32_t bi = mwi > TK_WIN - 1 ? mwi - (TK_WIN - 1) : 1u;
            if (mwi != 0 && key >= bi && key <= mwi) s += sh.whist[i][key - bi];
        }
        sh.c.hist[b] = s;
    }
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < TK1_WAVES; ++i) tot += sh.dsum[i];
    const float lse32 = (float)((double)Mv + log(tot));

    uint32_t in_win = 0;
    for (int b = 0; b < TK_WIN; ++b) in_win += sh.c.hist[b];   // uniform, LDS broadcast reads

    // ---- the cut key kappa, keys above it, keys equal to it
    uint32_t kappa, above, n_eq;
    if (in_win >= k) {
        select_bin(sh.c, sh.c.hist, k);
        kappa = gbase + sh.c.bcast[0];
        above = sh.c.bcast[1];
        n_eq = sh.c.bcast[2];
        __syncthreads();
    } else {
        // generic path: two 8-bit digits over the whole row
        kappa = radix_select<2>(sh.c, [&](auto fn) {
            for (int i = 0; i < nrows; ++i) {
                const u32x4 kk = load_keys<VEC>(x, i * TK1_THREADS + tid, V, nchunks);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (kk[e] & 0xffffu) fn(kk[e] & 0xffffu);
                    if (kk[e] >> 16) fn(kk[e] >> 16);
                }
            }
        }, k, &above, &n_eq);
    }
    const uint32_t need = k - above;   // keys equal to kappa that are kept (1 <= need <= n_eq)

    // ---- pass 2: gather the winners
    if (tid == 0) sh.count = 0;
    __syncthreads();
    int n;
    if (above + n_eq <= (uint32_t)TK_LIST) {
        // every key >= kappa; the sort puts ties in id order
        for (int i = 0; i < nrows; ++i) {
            const int c = i * TK1_THREADS + tid;
            const u32x4 kk = load_keys<VEC>(x, c, V, nchunks);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t key = (kk[e] >> (16 * h)) & 0xffffu;
                    if (key >= kappa && key != 0) {
                        const uint32_t slot = atomicAdd(&sh.count, 1u);
                        sh.list[slot] = ((unsigned long long)key << 32) | (0xffffffffu - (uint32_t)(c * 8 + e * 2 + h));
                    }
                }
        }
        n = (int)(above + n_eq);
    } else {
        // too many ties to hold: rank them by id, row of chunks by row of chunks
        uint32_t run = 0;
        for (int i = 0; i < nrows; ++i) {
            const int c = i * TK1_THREADS + tid;
            const u32x4 kk = load_keys<VEC>(x, c, V, nchunks);
            uint32_t nt = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) nt += ((kk[e] & 0xffffu) == kappa) + ((kk[e] >> 16) == kappa);
            uint32_t rowtot;
            uint32_t rank = run + block_excl_scan(sh.c, nt, &rowtot);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t key = (kk[e] >> (16 * h)) & 0xffffu;
                    bool take = key > kappa;
                    if (key == kappa) take = rank++ < need;
                    if (take) {
                        const uint32_t slot = atomicAdd(&sh.count, 1u);
                        sh.list[slot] = ((unsigned long long)key << 32) | (0xffffffffu - (uint32_t)(c * 8 + e * 2 + h));
                    }
                }
            run += rowtot;
        }
        n = (int)k;
    }
    __syncthreads();
    const int width = pow2_at_least(n);
    for (int i = n + tid; i < width; i += TK1_THREADS) sh.list[i] = 0ull;
    __syncthreads();
    bitonic_desc(sh.list, width);

    // ---- scores and outputs
    const float c0 = cum ? cum[row] : 0.f;
    for (int j = tid; j < k_local; j += TK1_THREADS) {
        const unsigned long long e = sh.list[j];
        const uint32_t key = (uint32_t)(e >> 32);
        const int32_t id = (int32_t)(0xffffffffu - (uint32_t)(e & 0xffffffffu));
        const float lp = key16_value(key) - lse32;
        const float s = c0 + lp;
        const size_t o = row * (size_t)k_local + j;
        ws_tok[o] = id;
        ws_score[o] = s;
        if (local_tok) local_tok[o] = id;
        if (local_score) local_score[o] = s;
    }
    if (tid == 0 && row_lse) row_lse[row] = lse32;
}

// ---- stage 2 ----------------------------------------------------------------

struct Tk2Shared {
    TkCommon c;
    unsigned long long list[1024];   // k_global <= 1024
    uint32_t count;
};

__global__ __launch_bounds__(TK2_THREADS) void topk_stage2_kernel(const int32_t *__restrict__ ws_tok,
                                                                  const float *__restrict__ ws_score, int W_in,
                                                                  int k_local, int k_global,
                                                                  int32_t *__restrict__ out_tok,
                                                                  int32_t *__restrict__ out_par,
                                                                  float *__restrict__ out_score)
{
    __shared__ Tk2Shared sh;
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const int kk = min(k_local, k_global);
    const float *sc = ws_score + (size_t)r * W_in * k_local;
    const uint32_t k = (uint32_t)k_global;
    const int b = tid;                       // one beam per thread (W_in <= 1024)
    const bool has_beam = b < W_in;
    const float *brow = sc + (size_t)(has_beam ? b : 0) * k_local;

    // number of entries j < kk of this beam with key >= t (its list is sorted)
    auto prefix_ge = [&](uint32_t t) -> int {
        int lo = 0, hi = kk;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (key32(brow[mid]) >= t) lo = mid + 1; else hi = mid;
        }
        return lo;
    };

    // -- lower bound tau: the k-th largest of the first J entries of every beam
    const int J = min(kk, (k_global + W_in - 1) / W_in + 1);
    uint32_t a_, e_;
    const uint32_t tau = radix_select<4>(sh.c, [&](auto fn) {
        if (has_beam)
            for (int j = 0; j < J; ++j) fn(key32(brow[j]));
    }, k, &a_, &e_);
    const int nb = has_beam ? prefix_ge(tau) : 0;

    // -- exact cut among the prefixes
    uint32_t above, n_eq;
    const uint32_t kappa = radix_select<4>(sh.c, [&](auto fn) {
        for (int j = 0; j < nb; ++j) fn(key32(brow[j]));
    }, k, &above, &n_eq);
    const uint32_t need = k - above;
    // entries [0, gt_end) are above kappa, [gt_end, eq_end) equal it
    const int gt_end = has_beam ? prefix_ge(kappa + 1u) : 0;   // finite scores: kappa < 0xffffffff
    int eq_end = gt_end;
    if (has_beam) {
        int lo = gt_end, hi = nb;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (key32(brow[mid]) >= kappa) lo = mid + 1; else hi = mid;
        }
        eq_end = lo;
    }
    uint32_t ties_total;
    const uint32_t tie_base = block_excl_scan(sh.c, (uint32_t)(eq_end - gt_end), &ties_total);
    int take_ties = 0;
    if (tie_base < need) take_ties = min(eq_end - gt_end, (int)(need - tie_base));

    const int width = pow2_at_least(k_global);
    for (int i = tid; i < width; i += TK2_THREADS) sh.list[i] = 0ull;
    if (tid == 0) sh.count = 0;
    __syncthreads();
    const int take = gt_end + take_ties;
    if (take > 0) {
        const uint32_t slot0 = atomicAdd(&sh.count, (uint32_t)take);
        for (int j = 0; j < take; ++j) {
            const uint32_t f = (uint32_t)(b * k_local + j);
            sh.list[slot0 + j] = ((unsigned long long)key32(brow[j]) << 32) | (0xffffffffu - f);
        }
    }
    __syncthreads();
    bitonic_desc(sh.list, width);

    for (int i = tid; i < k_global; i += TK2_THREADS) {
        const unsigned long long e = sh.list[i];
        const uint32_t f = 0xffffffffu - (uint32_t)(e & 0xffffffffu);
        const int parent = (int)(f / (uint32_t)k_local), j = (int)(f % (uint32_t)k_local);
        const size_t src = ((size_t)r * W_in + parent) * k_local + j;
        out_tok[(size_t)r * k_global + i] = ws_tok[src];
        out_par[(size_t)r * k_global + i] = parent;
        out_score[(size_t)r * k_global + i] = ws_score[src];
    }
}

TopkWorkspace topk_workspace_layout(int R, int W_in, int k_local)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t n = (size_t)R * W_in * k_local;
    TopkWorkspace l;
    l.local_tok = 0;
    l.local_score = up(n * sizeof(int32_t));
    l.total = l.local_score + up(n * sizeof(float));
    return l;
}

hipError_t launch_beam_topk(const uint16_t *logits, const float *cum, int R, int W_in, int V, int k_local,
                            int k_global, int32_t *out_tok, int32_t *out_par, float *out_score,
                            int32_t *local_tok, float *local_score, float *row_lse, void *workspace,
                            hipStream_t stream)
{
    const TopkWorkspace l = topk_workspace_layout(R, W_in, k_local);
    int32_t *ws_tok = (int32_t *)((char *)workspace + l.local_tok);
    float *ws_score = (float *)((char *)workspace + l.local_score);
    dim3 g1((unsigned)(R * W_in)), b1(TK1_THREADS);
    if (V % 8 == 0)
        hipLaunchKernelGGL(topk_stage1_kernel<true>, g1, b1, 0, stream, logits, cum, V, k_local, ws_tok, ws_score,
                           local_tok, local_score, row_lse);
    else
        hipLaunchKernelGGL(topk_stage1_kernel<false>, g1, b1, 0, stream, logits, cum, V, k_local, ws_tok,
                           ws_score, local_tok, local_score, row_lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_stage2_kernel, dim3(R), dim3(TK2_THREADS), 0, stream, ws_tok, ws_score, W_in, k_local,
                       k_global, out_tok, out_par, out_score);
    return hipGetLastError();
}

}  // namespace bga
