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
// Stage 1 (one 256-thread workgroup per beam row, several per CU) reads the
// row from HBM once:
//   threshold: the keys of a sample of 4096 logits (64 runs of 64, spread
//     evenly over the row) give a
//     cut t whose expected count in the row is about 2.5k (k = k_local); for
//     rows that fit the candidate list whole, t takes every element.
//   stream: every lane keeps a running offset m (its largest logit so far,
//     moved lazily) and an fp64 sum of fp32 exp(x - m); elements with key >= t
//     are appended to an LDS candidate list (a lane first checks its chunk
//     maximum against t, so the append path is rare).
//   selection: if the list holds at least k keys (and did not overflow), the
//     k-th largest key of the row is the k-th largest of the list, found by an
//     exact radix select; the entries at or above it are sorted by
//     (key desc, id asc), which also breaks ties by lower id. Otherwise (a
//     sample far from the row's distribution) the row is read again and the
//     cut found by a radix select over the whole row; if too many keys equal
//     the cut to sort, ties are ranked by id with a block scan in id order.
//   The lanes' (m, sum) pairs merge into the row's fp32 log-sum-exp.
// Stage 2 (one workgroup per request): each beam's list is sorted, so only its
// first min(k_local, k_global) entries can matter and the entries above any
// threshold form a prefix. A lower bound L on the cut comes from the first 8
// entries of every beam (two radix digits of their k-th largest, or all four
// when two let more entries in than the list holds); every entry >= L goes
// into an LDS list of up to 8192 (a beam whose 8th entry is >= L continues
// from memory, 256 entries per wave read); when more than 2048 are listed, a
// radix select over the listed keys gives the exact cut and keeps the k
// chosen entries (ties by lower flat index); the listed entries (at most 2048)
// are then sorted by (score desc, flat index asc) with one bitonic network and
// the first k are the output. When even the exact bound lets more than 8192
// entries in (many equal scores), the cut comes from radix selects over the
// beams' prefixes in memory instead.
#include <mutex>

#include "bga.h"
#include "device_common.hpp"
#include "internal.hpp"

namespace bga {

struct Parity0 { static constexpr int value = 0; };
struct Parity1 { static constexpr int value = 1; };

constexpr int TK1_THREADS = 256;   // stage 1: one workgroup per beam row
constexpr int TK1_WAVES = TK1_THREADS / 64;
constexpr int TK1_UNROLL = 4;      // 16-byte chunks in flight per thread
constexpr int TK_LIST = 4096;      // candidate list entries
constexpr int TK_SAMPLE = 512;     // sampled 8-logit chunks (4096 logits)
constexpr int TK_RING = 128;       // per wave: queued 16-byte chunks holding a candidate
constexpr int TK_RING_U64 = TK1_WAVES * 2 * TK_RING;       // the rings' share of the list, at its end
constexpr int TK_CAP = 2 * (TK_LIST - TK_RING_U64);        // candidates the stream can list (6144 words)
static_assert(TK_CAP % TK1_THREADS == 0 && TK_CAP >= 4096, "the stream's candidates and the rings share the list");
// a listed candidate is one word: (key - t) << 18 | (2^18 - 1 - id)
static_assert(BGA_MAX_VOCAB <= (1 << 18), "token ids fit 18 bits");
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

__device__ __forceinline__ float key32_value(uint64_t key64);

__device__ __forceinline__ uint32_t key32(float f)
{
    uint32_t b = __float_as_uint(f);
    b = (b == 0x80000000u) ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The score of a 32-bit key (every finite score but -0 maps back to itself;
// -0 was keyed as +0).
__device__ __forceinline__ float key32_value(uint64_t key64)
{
    const uint32_t key = (uint32_t)key64;
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
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

// Bitonic sort of list[0..1024) into descending order by 256 threads. Each
// thread holds the elements at positions tid + 256 i (i < 4): exchanges at
// distance 256 and 512 stay in the thread, distances below 64 are lane
// shuffles within the wave, and only distances 64 and 128 go through LDS.
__device__ __forceinline__ void bitonic1024_desc(unsigned long long *list)
{
    const int tid = threadIdx.x;
    unsigned long long v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = list[tid + 256 * i];
    auto cas = [](unsigned long long &a, unsigned long long &b, bool desc) {   // a at the lower position
        const bool swap = desc ? (a < b) : (a > b);
        const unsigned long long lo = swap ? b : a, hi = swap ? a : b;
        a = lo;
        b = hi;
    };
#pragma unroll 1
    for (int size = 2; size <= 1024; size <<= 1) {
#pragma unroll 1
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= 256) {
                const int d = stride / 256;   // 1 or 2
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!(i & d)) cas(v[i], v[i | d], ((tid + 256 * i) & size) == 0);
            } else if (stride >= 64) {
                __syncthreads();
#pragma unroll
                for (int i = 0; i < 4; ++i) list[tid + 256 * i] = v[i];
                __syncthreads();
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = tid + 256 * i;
                    const unsigned long long o = list[pos ^ stride];
                    const bool lower = (pos & stride) == 0, desc = (pos & size) == 0;
                    const bool take_max = lower == desc;
                    v[i] = take_max ? (v[i] > o ? v[i] : o) : (v[i] < o ? v[i] : o);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = tid + 256 * i;
                    const uint32_t lo = __shfl_xor((uint32_t)v[i], stride), hi = __shfl_xor((uint32_t)(v[i] >> 32), stride);
                    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
                    const bool lower = (pos & stride) == 0, desc = (pos & size) == 0;
                    const bool take_max = lower == desc;
                    v[i] = take_max ? (v[i] > o ? v[i] : o) : (v[i] < o ? v[i] : o);
                }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) list[tid + 256 * i] = v[i];
    __syncthreads();
}

// Value held by lane (lane ^ stride) of the wave, stride a power of two < 64:
// DPP quad permutes for 1 and 2, LDS-free swizzles for 4..16, a row swap for 32.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int stride)
{
    switch (stride) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (4 << 10));
    case 8: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (8 << 10));
    case 16: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (16 << 10));
    default: {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (threadIdx.x & 32) ? p[0] : p[1];
    }
    }
}

// Bitonic sort into descending order of 1024 32-bit values held 4 per thread
// by 256 threads (v[i] at position tid + 256 i). Distances 256 and 512 stay
// in the thread, distances below 64 are lane exchanges, 64 and 128 go through
// `scratch` (1024 words of LDS).
__device__ __forceinline__ void bitonic1024_desc_u32(uint32_t (&v)[4], uint32_t *scratch)
{
    const int tid = threadIdx.x;
#pragma unroll 1
    for (int size = 2; size <= 1024; size <<= 1) {
#pragma unroll 1
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= 256) {
                const int d = stride / 256;   // 1 or 2
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!(i & d)) {
                        const bool desc = ((tid + 256 * i) & size) == 0;
                        const uint32_t a = v[i], b = v[i | d];
                        v[i] = desc ? max(a, b) : min(a, b);
                        v[i | d] = desc ? min(a, b) : max(a, b);
                    }
            } else {
                uint32_t o[4];
                if (stride >= 64) {
                    __syncthreads();
#pragma unroll
                    for (int i = 0; i < 4; ++i) scratch[tid + 256 * i] = v[i];
                    __syncthreads();
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = scratch[(tid + 256 * i) ^ stride];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = lane_xor(v[i], stride);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int pos = tid + 256 * i;
                    const bool take_max = ((pos & stride) == 0) == ((pos & size) == 0);
                    v[i] = take_max ? max(v[i], o[i]) : min(v[i], o[i]);
                }
            }
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
    union {
        unsigned long long list[TK_LIST];     // candidates: key << 32 | ~id
        uint16_t sample[TK_SAMPLE * 8];       // sampled keys (before the stream)
    };
    uint32_t whist[TK1_THREADS / 64][256];    // per-wave digit histograms of the sample
    float lmax[TK1_THREADS / 64];
    double dsum[TK1_THREADS / 64];
    uint32_t wcnt[TK1_THREADS / 64];
    uint32_t ring_id[TK1_THREADS / 64][TK_RING];   // chunk index of each queued chunk
    uint32_t count;
    uint32_t wide;                            // a candidate lies 1024 or more keys above t
};

// The j-th largest nonzero key of sh.sample[0..n) (two 8-bit digits; each wave
// counts into its own histogram, since sample keys crowd into a few digits).
__device__ __forceinline__ uint32_t sample_select(Tk1Shared &sh, int n, uint32_t j)
{
    const int tid = threadIdx.x, w = tid >> 6;
    uint32_t prefix = 0, mask = 0, krem = j;
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = 8 * (1 - pass);
        for (int i = tid; i < (TK1_THREADS / 64) * 256; i += TK1_THREADS) (&sh.whist[0][0])[i] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += TK1_THREADS) {
            const uint32_t key = sh.sample[i];
            if (key && (key & mask) == prefix) atomicAdd(&sh.whist[w][(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 256) {
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < TK1_THREADS / 64; ++i) c += sh.whist[i][tid];
            sh.c.hist[tid] = c;
        }
        __syncthreads();
        select_bin(sh.c, sh.c.hist, krem);
        krem -= sh.c.bcast[1];
        prefix |= sh.c.bcast[0] << shift;
        mask |= 255u << shift;
        __syncthreads();
    }
    return prefix;
}

// The j-th largest (1 <= j <= 128) of the wave's 128 16-bit values (a and b of
// every lane), four bits per round: candidate d (1..15) extends the prefix by
// d, two ballots count the values at or above it, and since that count falls
// as d grows, the number of candidates whose count reaches j is the largest
// such d. The prefix stays the largest value with at least j values at or
// above it. Scalar work only after the compares; no LDS, no barrier.
__device__ __forceinline__ uint32_t wave_jth_largest16(uint32_t a, uint32_t b, uint32_t j)
{
    uint32_t prefix = 0;
#pragma unroll
    for (int round = 0; round < 4; ++round) {
        const int shift = 12 - 4 * round;
        uint32_t d = 0;
#pragma unroll
        for (int c = 1; c < 16; ++c) {
            const uint32_t cand = prefix | ((uint32_t)c << shift);
            const uint32_t n = (uint32_t)__popcll(__ballot(a >= cand)) + (uint32_t)__popcll(__ballot(b >= cand));
            d += n >= j ? 1u : 0u;
        }
        prefix |= d << shift;
    }
    return prefix;
}

// Raw bf16 bits of row chunk c (8 logits, ids 8c .. 8c+7) as four packed pairs;
// logits beyond the row read as -inf (0xff80). The load itself is clamped to
// the row and never skipped, so that a wave's loads are issued unconditionally
// (the compiler can then wait for exactly the loads it needs).
template <bool VEC>
__device__ __forceinline__ u32x4 load_raw(const uint16_t *__restrict__ x, int c, int V, int nchunks)
{
    u32x4 raw;
    if (VEC) {
        // every logit is read once: the non-temporal hint keeps the stream
        // from displacing what other workgroups still use in the caches
        raw = __builtin_nontemporal_load((const u32x4 *)(x + (size_t)min(c, nchunks - 1) * 8));
        if (c >= nchunks) raw = u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
    } else {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const int id = c * 8 + j;
            const uint32_t b0 = x[min(id, V - 1)], b1 = x[min(id + 1, V - 1)];
            raw[j / 2] = (id < V ? b0 : 0xff80u) | ((id + 1 < V ? b1 : 0xff80u) << 16);
        }
    }
    return raw;
}

// Keys of a chunk; logits beyond the row get key 0 (no element).
template <bool VEC>
__device__ __forceinline__ u32x4 load_keys(const uint16_t *__restrict__ x, int c, int V, int nchunks)
{
    const u32x4 raw = load_raw<VEC>(x, c, V, nchunks);
    u32x4 k;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int id = c * 8 + 2 * e;
        const uint32_t lo = id < V ? key16(raw[e] & 0xffffu) : 0u;
        const uint32_t hi = id + 1 < V ? key16(raw[e] >> 16) : 0u;
        k[e] = lo | (hi << 16);
    }
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
    const float c0 = cum ? cum[row] : 0.f;   // (needed at the end; loaded now)

    // ---- threshold key t from a strided sample (t = 1: every element)
    // Whole 8-chunk (128-byte) groups spread evenly over the row: the sample
    // costs its own size in traffic, not one cache line per chunk.
    const int ns = min(nchunks, TK_SAMPLE);
    const int ngrp = nchunks >> 3, sgrp = ns >> 3;
    const int nsamp = ns * 8;
    // expected count of row keys >= the j-th largest sample key: about j * V / nsamp = 1.5k
    // (plus a margin of 8 sample ranks)
    // (32-bit arithmetic: V <= BGA_MAX_VOCAB and k <= BGA_MAX_K keep every product below 2^31)
    const uint32_t j = min((uint32_t)nsamp, (3u * k * (uint32_t)nsamp + 2u * (uint32_t)V - 1u) / (2u * (uint32_t)V) + 8u);
    auto sample_chunk = [&](int i) {
        const uint32_t g = (uint32_t)(i >> 3);
        const int c = sgrp > 0 && (int)g < sgrp ? (int)((g * (uint32_t)ngrp) / (uint32_t)sgrp) * 8 + (i & 7)
                                                : (int)(((uint32_t)i * (uint32_t)nchunks) / (uint32_t)ns);
        return load_keys<VEC>(x, c, V, nchunks);
    };
    // the usual sample: 64 groups (sgrp = 64), a shift instead of a division;
    // raw bits (the index is clamped into the row)
    auto sample_raw64 = [&](int i) {
        const int c = min((int)(((uint32_t)(i >> 3) * (uint32_t)ngrp) >> 6) * 8 + (i & 7), nchunks - 1);
        if (VEC) return *(const u32x4 *)(x + (size_t)c * 8);
        return load_raw<VEC>(x, c, V, nchunks);   // ids past the row read as -inf, a key below every logit's
    };
    // Few sample ranks (the usual case): every wave takes the ceil(j/4)-th
    // largest of its lanes' two largest sample keys (16 per lane; three of a
    // wave's top keys rarely share a lane), and t is the mean of the four. The
    // sample loads go out first, then the stream's first chunks, which land
    // while the threshold is chosen.
    const bool quick = V > TK_LIST && j <= 64u && ns == 2 * TK1_THREADS;
    u32x4 bufa[TK1_UNROLL], bufb[TK1_UNROLL];
    auto first_batch = [&]() {
#pragma unroll
        for (int u = 0; u < TK1_UNROLL; ++u) bufa[u] = load_raw<VEC>(x, u * TK1_THREADS + tid, V, nchunks);
    };
    uint32_t tkey = 1u;
    if (quick) {
        u32x4 smp[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) smp[h] = sample_raw64(h * TK1_THREADS + tid);
        first_batch();
        uint32_t k1 = 0u, k2 = 0u;   // the lane's two largest sample keys
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t key = key16((smp[h][e >> 1] >> (16 * (e & 1))) & 0xffffu);
                k2 = max(k2, min(k1, key));
                k1 = max(k1, key);
            }
        const uint32_t tw = wave_jth_largest16(k1, k2, (j + TK1_WAVES - 1) / TK1_WAVES);
        if (lane == 0) sh.wcnt[w] = tw;
        __syncthreads();
        uint32_t sum = 0;
#pragma unroll
        for (int i = 0; i < TK1_WAVES; ++i) sum += sh.wcnt[i];
        tkey = sum / TK1_WAVES;
    } else {
        first_batch();
    }
    if (!quick && V > TK_LIST) {
        for (int i = tid; i < ns; i += TK1_THREADS) {
            const u32x4 kk = sample_chunk(i);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sh.sample[i * 8 + 2 * e] = (uint16_t)(kk[e] & 0xffffu);
                sh.sample[i * 8 + 2 * e + 1] = (uint16_t)(kk[e] >> 16);
            }
        }
        __syncthreads();
        tkey = sample_select(sh, nsamp, j);
    }
    // the stream counts its candidates' keys into 1024 bins above t
    uint32_t *const hist = &sh.whist[0][0];
    for (int i = tid; i < 1024; i += TK1_THREADS) hist[i] = 0u;
    if (tid == 0) {
        sh.count = 0u;
        sh.wide = 0u;
    }
    __syncthreads();   // the sample and the threshold's words are dead: the list reuses that memory
    const float tval = tkey > 1u ? key16_value(tkey) : -INFINITY;   // value form of the cut (prefilter)

    // ---- stream: per-lane lazy offset m and fp64 sum of exp(x - m); candidates >= t
    // A chunk whose maximum reaches t is pushed (data and index) onto the wave's
    // ring in LDS; whenever 64 are queued the wave takes one per lane, extracts
    // its keys >= t and appends them to the block's candidate list (one LDS
    // atomic per wave reserves the places). The row is read once: the
    // candidates come from data already in registers.
    float m = -INFINITY;
    double acc = 0.0;
    uint32_t rpos = 0;     // ring fill (wave-uniform)
    u32x4 *const ring = (u32x4 *)(sh.list + (TK_LIST - TK_RING_U64)) + w * TK_RING;
    uint32_t *const list32 = (uint32_t *)sh.list;
    uint32_t *const ring_id = sh.ring_id[w];
    auto drain = [&](uint32_t n) {   // the ring's first n <= 64 chunks (wave-uniform n)
        const bool have = (uint32_t)lane < n;
        const u32x4 d = have ? ring[lane] : u32x4{0u, 0u, 0u, 0u};
        const int c = have ? (int)ring_id[lane] : 0;
        uint32_t hm = 0;   // bit e*2+h: element 2e+h of the chunk is a candidate
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hm |= (bf16_lo(d[e]) >= tval ? 1u : 0u) << (2 * e);
            hm |= (bf16_hi(d[e]) >= tval ? 1u : 0u) << (2 * e + 1);
        }
        // finite logits: value order is key order (a candidate's key is >= t).
        // Only chunks inside the row
        // are queued (c < nchunks, so 1 <= V - 8c); its ids >= V are padding.
        hm = have ? hm & ((1u << min(8, V - c * 8)) - 1u) : 0u;
        const uint32_t cnt = (uint32_t)__popc(hm);
        const uint32_t incl = wave_incl_scan_u32(cnt);
        const uint32_t tot = (uint32_t)__shfl(incl, 63);
        uint32_t base = 0;
        if (lane == 0 && tot) base = atomicAdd(&sh.count, tot);   // past TK_CAP: counted, not stored
        uint32_t at = (uint32_t)__shfl((int)base, 0) + incl - cnt;
        while (hm) {
            const int b = __ffs(hm) - 1;
            hm &= hm - 1;
            const uint32_t word = d[b >> 1];
            const uint32_t key = key16((b & 1) ? (word >> 16) : (word & 0xffffu));
            const uint32_t id = (uint32_t)(c * 8 + b);
            const uint32_t dk = key - tkey;
            if (dk < 1024u) {
                atomicAdd(&hist[dk], 1u);
                if (at < (uint32_t)TK_CAP) list32[at] = (dk << 18) | (0x3ffffu - id);
            } else {
                sh.wide = 1u;
            }
            ++at;
        }
        // move the rest of the ring down (same wave: LDS keeps this order)
        const uint32_t rest = rpos - n;
        if ((uint32_t)lane < rest) {
            const u32x4 t = ring[n + lane];
            const uint32_t ti = ring_id[n + lane];
            ring[lane] = t;
            ring_id[lane] = ti;
        }
        rpos = rest;
    };
    // two buffers of chunks: one is reduced while the other is in flight
    auto load_batch = [&](u32x4 (&buf)[TK1_UNROLL], int i0) {
#pragma unroll
        for (int u = 0; u < TK1_UNROLL; ++u) buf[u] = load_raw<VEC>(x, (i0 + u) * TK1_THREADS + tid, V, nchunks);
    };
    auto consume = [&](const u32x4 (&raw)[TK1_UNROLL], int i0) {
        float cmax[TK1_UNROLL];
#pragma unroll
        for (int u = 0; u < TK1_UNROLL; ++u) {
            float c = -INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) c = fmaxf(c, fmaxf(bf16_lo(raw[u][e]), bf16_hi(raw[u][e])));
            cmax[u] = c;
        }
        float lm = cmax[0];
#pragma unroll
        for (int u = 1; u < TK1_UNROLL; ++u) lm = fmaxf(lm, cmax[u]);
        if (lm > m + 8.f) {   // lazy: exp(x - m) stays <= e^8 between moves
            if (m != -INFINITY) acc *= (double)__builtin_amdgcn_exp2f((m - lm) * kLog2e);
            m = lm;
        }
        if (m != -INFINITY) {
            const float mlog = m * kLog2e;
            float cs = 0.f;
#pragma unroll
            for (int u = 0; u < TK1_UNROLL; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cs += __builtin_amdgcn_exp2f(__builtin_fmaf(bf16_lo(raw[u][e]), kLog2e, -mlog));
                    cs += __builtin_amdgcn_exp2f(__builtin_fmaf(bf16_hi(raw[u][e]), kLog2e, -mlog));
                }
            acc += (double)cs;
        }
#pragma unroll
        for (int u = 0; u < TK1_UNROLL; ++u) {   // queue the row's chunks that hold keys >= t
            const bool hit = cmax[u] >= tval && (i0 + u) * TK1_THREADS + tid < nchunks;
            const unsigned long long mask = __ballot(hit);
            if (mask) {   // wave-uniform; the wave's own ring, no atomics
                const uint32_t pos = rpos + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                if (hit) {
                    ring[pos] = raw[u];
                    ring_id[pos] = (uint32_t)((i0 + u) * TK1_THREADS + tid);
                }
                rpos += (uint32_t)__popcll(mask);
                if (rpos >= 64u) drain(64u);
            }
        }
    };
    for (int i0 = 0; i0 < nrows; i0 += 2 * TK1_UNROLL) {
        load_batch(bufb, i0 + TK1_UNROLL);
        consume(bufa, i0);
        load_batch(bufa, i0 + 2 * TK1_UNROLL);
        consume(bufb, i0 + TK1_UNROLL);
    }
    while (rpos > 0u) drain(min(rpos, 64u));

    // ---- after the stream: the candidate count, the row's log-sum-exp and (the
    // usual case) the scan of the bin counts the stream kept, in two barriers
    {
        float Mw = m;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) Mw = fmaxf(Mw, __shfl_xor(Mw, o));
        if (lane == 0) sh.lmax[w] = Mw;
    }
    __syncthreads();
    const uint32_t found = sh.count;
    const bool noted_all = found <= (uint32_t)TK_CAP;
    const uint32_t count = min(found, (uint32_t)TK_CAP);
    // the same value in every thread: kept in a scalar register, so that the
    // loops below skip whole iterations past the listed entries
    const int ucnt = __builtin_amdgcn_readfirstlane((int)count);
    float M = sh.lmax[0];
#pragma unroll
    for (int i = 1; i < TK1_WAVES; ++i) M = fmaxf(M, sh.lmax[i]);
    {
        double part = (m != -INFINITY) ? acc * exp((double)m - (double)M) : 0.0;
        part = wave_sum_f64(part);
        if (lane == 0) sh.dsum[w] = part;
    }
    // Counting sort by key offset from t when every key >= t is listed, there
    // are at least k, and all lie within 1024 keys of t: the bins give each
    // key's place (keys above it) and ranks by id inside a bin finish the order.
    const bool fast = noted_all && count >= k && sh.wide == 0u;
    constexpr int kPerT = TK_CAP / TK1_THREADS;
    uint32_t ent[kPerT];
    uint32_t hc[4], loc = 0, incl = 0;
    if (fast) {
#pragma unroll
        for (int j = 0; j < kPerT; ++j) {
            const uint32_t idx = (uint32_t)(tid + j * TK1_THREADS);
            ent[j] = (j * TK1_THREADS < ucnt && idx < count) ? list32[idx] : 0u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hc[q] = hist[1023 - 4 * tid - q];   // thread t: bins 1023-4t down to 1020-4t
            loc += hc[q];
        }
        incl = wave_incl_scan_u32(loc);
        if (lane == 63) sh.c.wsum[w] = incl;
    }
    __syncthreads();   // (every listed entry is in registers: the list's memory is free)
    double dtot = 0.0;
#pragma unroll
    for (int i = 0; i < TK1_WAVES; ++i) dtot += sh.dsum[i];
    const float lse32 = (float)((double)M + log(dtot));

    auto emit = [&](int j, uint32_t key, int32_t id) {
        const float lp = key16_value(key) - lse32;
        const float s = c0 + lp;
        const size_t o = row * (size_t)k_local + j;
        ws_tok[o] = id;
        ws_score[o] = s;
        if (local_tok) local_tok[o] = id;
        if (local_score) local_score[o] = s;
    };

    if (fast) {
        uint32_t *start = list32;                   // entries above each bin (1024)
        uint32_t *bid = list32 + 1024;              // selected entries' low words, bin by bin (2048 + 8)
        uint32_t *out = list32 + 3088;              // the k chosen, in place order (<= 1024)
        uint16_t *sbin = (uint16_t *)(list32 + 4112);   // the bin of each filled slot (2048)
        uint32_t run = incl - loc;
        for (int i = 0; i < w; ++i) run += sh.c.wsum[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int b = 1023 - 4 * tid - q;
            start[b] = run;
            if (run < k && run + hc[q] >= k) {
                sh.c.bcast[0] = (uint32_t)b;
                sh.c.bcast[1] = run + hc[q];
            }
            run += hc[q];
        }
        __syncthreads();
        const uint32_t bk = sh.c.bcast[0];     // bin of the k-th largest key
        const uint32_t nsel = sh.c.bcast[1];   // entries in bins bk and above
        if (nsel <= 2048) {
            // bin dk holds slots [start[dk], start[dk - 1]) (start[-1] = count);
            // its counter, counted down, hands out the slots
#pragma unroll
            for (int j = 0; j < kPerT; ++j) {
                if (j * TK1_THREADS >= ucnt) continue;
                const uint32_t dk = ent[j] >> 18;
                if ((uint32_t)(tid + j * TK1_THREADS) < count && dk >= bk) {
                    const uint32_t slot = start[dk] + atomicSub(&hist[dk], 1u) - 1u;
                    bid[slot] = ent[j] & 0x3ffffu;
                    sbin[slot] = (uint16_t)dk;
                }
            }
            __syncthreads();
            // Every filled slot p (thread t: slots t + 256 q, q < 8) ranks its
            // entry inside its bin: the bin's entries with a lower id (a larger
            // low word), eight per pair of 16-byte reads from the aligned slots
            // around the bin, the eight slots' reads issued together. Slots
            // outside the bin are masked (reads past slot 2047 stay inside the
            // padding and are masked too).
            constexpr int NQ = 2048 / TK1_THREADS;
            uint32_t b0[NQ], b1[NQ], mine[NQ], rank[NQ], span = 0;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const uint32_t p = (uint32_t)(tid + q * TK1_THREADS);
                b0[q] = b1[q] = mine[q] = rank[q] = 0;
                if (p < nsel) {
                    const uint32_t dk = sbin[p];
                    b0[q] = start[dk];
                    b1[q] = dk > 0u ? start[dk - 1] : count;
                    mine[q] = bid[p];
                    span = max(span, b1[q] - (b0[q] & ~3u));
                }
            }
#pragma unroll 1
            for (uint32_t off = 0; off < span; off += 8) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const uint32_t a = (b0[q] & ~3u) + off;
                    if (a < b1[q]) {
                        const u32x4 q0 = *(const u32x4 *)(bid + a), q1 = *(const u32x4 *)(bid + a + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            rank[q] += (a + e >= b0[q] && a + e < b1[q] && q0[e] > mine[q]) ? 1u : 0u;
                            rank[q] += (a + 4 + e < b1[q] && q1[e] > mine[q]) ? 1u : 0u;
                        }
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const uint32_t p = (uint32_t)(tid + q * TK1_THREADS), at = b0[q] + rank[q];
                if (p < nsel && at < (uint32_t)k_local) out[at] = ((uint32_t)sbin[p] << 18) | mine[q];
            }
            __syncthreads();
            // the k entries in place order: consecutive threads store consecutive places
            for (int j = tid; j < k_local; j += TK1_THREADS) {
                const uint32_t e = out[j];
                emit(j, tkey + (e >> 18), (int32_t)(0x3ffffu - (e & 0x3ffffu)));
            }
            if (tid == 0 && row_lse) row_lse[row] = lse32;
            return;
        }
        __syncthreads();   // (every thread has read the bins: the general path reuses the memory)
    }

    // ---- the general path (the sample misled the threshold, or more than
    // 2048 entries tie at the cut): the cut key kappa, the keys above it and
    // the keys equal to it from a radix select over the whole row, read again
    uint32_t kappa, above, n_eq;
    int n;
    {
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
        const uint32_t need = k - above;   // keys equal to kappa that are kept (1 <= need <= n_eq)
        if (tid == 0) sh.count = 0;
        __syncthreads();
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
    }
    __syncthreads();
    if (n <= 1024) {
        // sort 32-bit words: (key - kappa) << 18 | (2^18 - 1 - id); 0 pads (ids < 2^18 - 1)
        uint32_t v[4];
        bool fits = true;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = tid + 256 * i;
            v[i] = 0u;
            if (pos < n) {
                const unsigned long long e = sh.list[pos];
                const uint32_t dk = (uint32_t)(e >> 32) - kappa;
                const uint32_t id = 0xffffffffu - (uint32_t)(e & 0xffffffffu);
                fits = fits && dk < (1u << 14);
                v[i] = (dk << 18) | (0x3ffffu - id);
            }
        }
        if (__syncthreads_and(fits)) {
            bitonic1024_desc_u32(v, (uint32_t *)sh.list);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int pos = tid + 256 * i;
                if (pos < k_local) emit(pos, kappa + (v[i] >> 18), (int32_t)(0x3ffffu - (v[i] & 0x3ffffu)));
            }
            if (tid == 0 && row_lse) row_lse[row] = lse32;
            return;
        }
    }
    const int width = pow2_at_least(n);
    for (int i = n + tid; i < width; i += TK1_THREADS) sh.list[i] = 0ull;
    __syncthreads();
    if (width == 1024)
        bitonic1024_desc(sh.list);
    else
        bitonic_desc(sh.list, width);

    // ---- scores and outputs
    for (int j = tid; j < k_local; j += TK1_THREADS) {
        const unsigned long long e = sh.list[j];
        emit(j, (uint32_t)(e >> 32), (int32_t)(0xffffffffu - (uint32_t)(e & 0xffffffffu)));
    }
    if (tid == 0 && row_lse) row_lse[row] = lse32;
}

// ---- stage 2 ----------------------------------------------------------------

constexpr int TK2_LIST = 8192;     // stage 2: candidates listed in LDS (one workgroup per request)
constexpr int TK2_PER = TK2_LIST / TK2_THREADS;
constexpr int TK2_SORT = 2 * TK2_THREADS;   // places of the final bitonic sort
static_assert(BGA_MAX_K <= TK2_SORT, "the sort holds every chosen entry");

// A listed stage-2 entry: key << 32 | (2^19 - 1 - flat index) << 13 | list slot
// (flat index = beam * k_local + slot < 2^19; list slot < 8192). Entries order
// by (score desc, flat index asc); the list slot names the entry's token,
// loaded when it is listed, so the output needs no second read of memory.
static_assert(BGA_MAX_BEAMS * BGA_MAX_K <= (1 << 19) && TK2_LIST <= (1 << 13), "stage-2 entry fields");

struct Tk2Shared {
    TkCommon c;
    unsigned long long list[TK2_LIST];             // candidates (entries as above)
    int32_t tok[TK2_LIST];                         // token of the entry listed at each slot
    uint32_t tie[TK2_LIST];                        // ~flat index of the entries whose key is the cut's
    uint32_t whist[TK2_THREADS / 64][256];         // per-wave digit histograms
    uint16_t inc[TK2_THREADS];                     // beams whose list continues above the bound
    uint32_t count, n_inc, n_tie;
};

// A lower bound on the k-th largest of the keys kv[0, C) of every thread
// (each thread's keys descending, 0 = no key; at least k keys in all): 8-bit
// digit passes [p0, p1) of a radix select of that key, one histogram per wave;
// a thread counts each run of equal digits with one atomic (its keys are
// sorted, so the keys that match the prefix and share a digit are adjacent).
// After passes [0, p) the bound is the k-th largest key with its low 32 - 8p
// bits cleared (keys >= it number at least k); the digits found so far stay in
// `st`, so later passes refine it.
struct DigitState {
    uint32_t prefix, mask, krem;
};
template <int C>
__device__ __forceinline__ uint32_t lower_bound_digits(Tk2Shared &sh, const uint32_t (&kv)[C], DigitState &st,
                                                       int p0, int p1)
{
    const int tid = threadIdx.x, w = tid >> 6;
    constexpr int NW = TK2_THREADS / 64;
    uint32_t prefix = st.prefix, mask = st.mask, krem = st.krem;
#pragma unroll 1
    for (int pass = p0; pass < p1; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < NW * 256; i += TK2_THREADS) (&sh.whist[0][0])[i] = 0;
        __syncthreads();
        uint32_t cur = 0, cnt = 0;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const uint32_t key = kv[j];
            if (key && (key & mask) == prefix) {
                const uint32_t d = (key >> shift) & 255u;
                if (cnt && d != cur) {
                    atomicAdd(&sh.whist[w][cur], cnt);
                    cnt = 0;
                }
                cur = d;
                ++cnt;
            }
        }
        if (cnt) atomicAdd(&sh.whist[w][cur], cnt);
        __syncthreads();
        if (tid < 256) {
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < NW; ++i) c += sh.whist[i][tid];
            sh.c.hist[tid] = c;
        }
        __syncthreads();
        select_bin(sh.c, sh.c.hist, krem);
        krem -= sh.c.bcast[1];
        prefix |= sh.c.bcast[0] << shift;
        mask |= 255u << shift;
        __syncthreads();
    }
    st = DigitState{prefix, mask, krem};
    return prefix;
}

__global__ __launch_bounds__(TK2_THREADS) void topk_stage2_kernel(const int32_t *__restrict__ ws_tok,
                                                                  const float *__restrict__ ws_score, int W_in,
                                                                  int k_local, int k_global,
                                                                  int32_t *__restrict__ out_tok,
                                                                  int32_t *__restrict__ out_par,
                                                                  float *__restrict__ out_score)
{
    __shared__ Tk2Shared sh;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = blockIdx.x;
    const int kk = min(k_local, k_global);
    const float *sc = ws_score + (size_t)r * W_in * k_local;
    const uint32_t k = (uint32_t)k_global;
    const int b = tid;                       // one beam per thread (W_in <= 1024)
    const bool has_beam = b < W_in;
    const float *brow = sc + (size_t)(has_beam ? b : 0) * k_local;
    const int32_t *tk = ws_tok + (size_t)r * W_in * k_local;
    auto entry = [&](uint32_t key, int beam, int j, uint32_t slot) {
        return ((unsigned long long)key << 32) | ((0x7ffffu - (uint32_t)(beam * k_local + j)) << 13) | slot;
    };

    // -- a lower bound L on the cut: the k-th largest of the first C entries of
    // every beam, or that key with its low 16 bits cleared (a subset of the
    // candidates holds k keys >= L, so the k-th largest of all of them is >= L)
    constexpr int C = 8;
    const int cb = min(kk, C);
    uint32_t kv[C];
#pragma unroll
    for (int j = 0; j < C; ++j) kv[j] = (has_beam && j < cb) ? key32(brow[j]) : 0u;   // 0: nothing (finite keys > 0)
    // -- every entry >= L goes into the list: the first C from registers; a
    // beam whose C-th entry is still >= L continues in memory (its list is
    // sorted, so its entries >= L form a prefix), read 64 at a time by a wave
    auto build_list = [&](uint32_t L) {
        if (tid == 0) {
            sh.count = 0;
            sh.n_inc = 0;
        }
        __syncthreads();
        uint32_t nreg = 0;
#pragma unroll
        for (int j = 0; j < C; ++j) nreg += kv[j] >= L ? 1u : 0u;
        if (nreg) {
            uint32_t at = atomicAdd(&sh.count, nreg);
#pragma unroll
            for (int j = 0; j < C; ++j)
                if (kv[j] >= L) {
                    if (at < (uint32_t)TK2_LIST) {
                        sh.list[at] = entry(kv[j], b, j, at);
                        sh.tok[at] = tk[(size_t)b * k_local + j];
                    }
                    ++at;
                }
        }
        if (has_beam && cb < kk && kv[cb - 1] >= L) sh.inc[atomicAdd(&sh.n_inc, 1u)] = (uint16_t)b;
        __syncthreads();
        const int n_inc = (int)sh.n_inc;
        for (int t = w; t < n_inc; t += TK2_THREADS / 64) {
            const int bb = sh.inc[t];
            const float *row = sc + (size_t)bb * k_local;
            // four runs of 64 per round trip (the loads of a round go out together)
            for (int j0 = C; j0 < kk; j0 += 256) {
                uint32_t key[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int j = j0 + 64 * u + lane;
                    key[u] = j < kk ? key32(row[j]) : 0u;
                }
                bool more = true;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int j = j0 + 64 * u + lane;
                    const bool take = more && key[u] >= L;
                    const unsigned long long mask = __ballot(take);
                    const uint32_t cnt = (uint32_t)__popcll(mask);
                    uint32_t base = 0;
                    if (lane == 0 && cnt) base = atomicAdd(&sh.count, cnt);
                    base = (uint32_t)__shfl((int)base, 0);
                    if (take) {
                        const uint32_t pos = base + __builtin_amdgcn_mbcnt_hi(
                                                        (uint32_t)(mask >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                        if (pos < (uint32_t)TK2_LIST) {
                            sh.list[pos] = entry(key[u], bb, j, pos);
                            sh.tok[pos] = tk[(size_t)bb * k_local + j];
                        }
                    }
                    more = more && cnt == 64u;   // a run not wholly >= L ends the beam's prefix
                }
                if (!more) break;
            }
        }
        __syncthreads();
        return sh.count;
    };
    // The bound first keeps the key's top 16 bits; if that lets more entries in
    // than the list holds (scores crowded near the cut, as after the first
    // step, when every beam descends from one), two more digits make it the
    // exact k-th largest of the first C entries and the list is built again.
    DigitState st{0u, 0u, k};
    const bool bounded = (long long)W_in * cb >= (long long)k;
    uint32_t n = build_list(bounded ? max(lower_bound_digits(sh, kv, st, 0, 2), 1u) : 1u);
    if (bounded && n > (uint32_t)TK2_LIST) n = build_list(max(lower_bound_digits(sh, kv, st, 2, 4), 1u));

    if (n > (uint32_t)TK2_LIST) {
        // Many entries at or above L (for example, many equal scores): the
        // exact cut kappa among the prefixes above a second bound, ties by
        // lower flat index, then the k chosen entries are sorted.
        auto prefix_ge = [&](uint32_t t) -> int {   // entries j < kk of this beam with key >= t
            int lo = 0, hi = kk;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (key32(brow[mid]) >= t) lo = mid + 1; else hi = mid;
            }
            return lo;
        };
        const int J = min(kk, (k_global + W_in - 1) / W_in + 1);
        uint32_t a_, e_;
        const uint32_t tau = radix_select<4>(sh.c, [&](auto fn) {
            if (has_beam)
                for (int j = 0; j < J; ++j) fn(key32(brow[j]));
        }, k, &a_, &e_);
        const int nb = has_beam ? prefix_ge(tau) : 0;
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
        if (tid == 0) sh.count = 0;
        __syncthreads();
        const int take = gt_end + take_ties;
        if (take > 0) {
            const uint32_t slot0 = atomicAdd(&sh.count, (uint32_t)take);
            for (int j = 0; j < take; ++j) {
                sh.list[slot0 + j] = entry(key32(brow[j]), b, j, slot0 + (uint32_t)j);
                sh.tok[slot0 + j] = tk[(size_t)b * k_local + j];
            }
        }
        __syncthreads();
    } else if (n > (uint32_t)TK2_SORT) {
        // Many more entries listed than chosen: the exact cut kappa among them
        // (a radix select over the listed keys, per-wave histograms), then only
        // the k chosen stay listed (keys above kappa, and of the keys equal to
        // it those with the lowest flat indices), so that the ordering below
        // sorts k entries, not n. (Up to 2048 listed entries are sorted as
        // they are.)
        unsigned long long e[TK2_PER];
#pragma unroll
        for (int q = 0; q < TK2_PER; ++q) {
            const uint32_t i = (uint32_t)(tid + q * TK2_THREADS);
            e[q] = i < n ? sh.list[i] : 0ull;   // 0: no entry (finite keys > 0)
        }
        uint32_t prefix = 0, mask = 0, krem = k, above = 0, n_eq = 0;
#pragma unroll 1
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            for (int i = tid; i < (TK2_THREADS / 64) * 256; i += TK2_THREADS) (&sh.whist[0][0])[i] = 0;
            __syncthreads();
#pragma unroll
            for (int q = 0; q < TK2_PER; ++q) {
                const uint32_t key = (uint32_t)(e[q] >> 32);
                if (key && (key & mask) == prefix) atomicAdd(&sh.whist[w][(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid < 256) {
                uint32_t c = 0;
#pragma unroll
                for (int i = 0; i < TK2_THREADS / 64; ++i) c += sh.whist[i][tid];
                sh.c.hist[tid] = c;
            }
            __syncthreads();
            select_bin(sh.c, sh.c.hist, krem);
            above += sh.c.bcast[1];
            krem -= sh.c.bcast[1];
            n_eq = sh.c.bcast[2];
            prefix |= sh.c.bcast[0] << shift;
            mask |= 255u << shift;
            __syncthreads();
        }
        const uint32_t kappa = prefix, need = k - above;   // 1 <= need <= n_eq
        // ties: when only some of the entries equal to kappa are chosen, an
        // entry's rank among them is the number with a lower flat index
        if (tid == 0) {
            sh.count = 0;
            sh.n_tie = 0;
        }
        __syncthreads();
        if (need < n_eq) {
#pragma unroll
            for (int q = 0; q < TK2_PER; ++q)
                if ((uint32_t)(e[q] >> 32) == kappa) sh.tie[atomicAdd(&sh.n_tie, 1u)] = (uint32_t)e[q];
            __syncthreads();
        }
        const uint32_t nt = sh.n_tie;
#pragma unroll
        for (int q = 0; q < TK2_PER; ++q) {
            const uint32_t key = (uint32_t)(e[q] >> 32);
            bool keep = key > kappa;
            if (key == kappa) {
                if (need >= n_eq) {
                    keep = true;
                } else {
                    uint32_t rank = 0;   // lower flat index <=> larger complemented index
                    for (uint32_t i = 0; i < nt; ++i) rank += sh.tie[i] > (uint32_t)e[q] ? 1u : 0u;
                    keep = rank < need;
                }
            }
            if (keep) sh.list[atomicAdd(&sh.count, 1u)] = e[q];
        }
        __syncthreads();
    }

    // -- order: the m <= 2048 listed entries (distinct: the flat index is part
    // of each; equal scores order by the complemented index, lower index first)
    // are sorted in descending order by a bitonic network over N = 1024 or 2048
    // places, N / 1024 per thread (places tid and tid + 1024), 0 padding the
    // list (below every entry). Distances below 64 are lane exchanges, 1024
    // stays inside the thread, the others go through the list in LDS; place
    // p < k of the sorted list is place p of the output.
    const int m = (int)min(sh.count, (uint32_t)TK2_SORT);   // >= k
    auto sort_and_store = [&](auto places) {
        constexpr int N = decltype(places)::value;
        constexpr int NPT = N / TK2_THREADS;
        unsigned long long v[NPT];
#pragma unroll
        for (int h = 0; h < NPT; ++h) {
            const int p = tid + h * TK2_THREADS;
            v[h] = p < m ? sh.list[p] : 0ull;
        }
        __syncthreads();   // every listed entry is in registers: the list serves the exchanges
#pragma unroll
        for (int k2 = 2; k2 <= N; k2 <<= 1)
#pragma unroll
            for (int j = k2 >> 1; j > 0; j >>= 1) {
                unsigned long long o[NPT];
                if (j == TK2_THREADS) {   // places tid and tid + 1024: the same thread
                    o[0] = v[NPT - 1];
                    o[NPT - 1] = v[0];
                } else if (j < 64) {
#pragma unroll
                    for (int h = 0; h < NPT; ++h) {
                        const uint32_t lo = lane_xor((uint32_t)v[h], j), hi = lane_xor((uint32_t)(v[h] >> 32), j);
                        o[h] = ((unsigned long long)hi << 32) | lo;
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < NPT; ++h) sh.list[tid + h * TK2_THREADS] = v[h];
                    __syncthreads();
#pragma unroll
                    for (int h = 0; h < NPT; ++h) o[h] = sh.list[(tid + h * TK2_THREADS) ^ j];
                    __syncthreads();
                }
#pragma unroll
                for (int h = 0; h < NPT; ++h) {
                    const int p = tid + h * TK2_THREADS;
                    // in a descending block of size k2 the lower place of a pair keeps the larger entry
                    const bool keep_max = ((p & j) == 0) == ((p & k2) == 0);
                    const bool larger = v[h] > o[h];
                    v[h] = keep_max == larger ? v[h] : o[h];
                }
            }
#pragma unroll
        for (int h = 0; h < NPT; ++h) {
            const int place = tid + h * TK2_THREADS;
            if (place < (int)k) {
                const unsigned long long e = v[h];
                const uint32_t low = (uint32_t)e;
                const uint32_t f = 0x7ffffu - (low >> 13);
                out_tok[(size_t)r * k_global + place] = sh.tok[low & 0x1fffu];
                out_par[(size_t)r * k_global + place] = (int)(f / (uint32_t)k_local);
                out_score[(size_t)r * k_global + place] = key32_value(e >> 32);
            }
        }
    };
    if (m <= TK2_THREADS)
        sort_and_store(std::integral_constant<int, TK2_THREADS>{});
    else
        sort_and_store(std::integral_constant<int, TK2_SORT>{});
}

// The library's own workspace for callers that cannot allocate device memory
// (bga_beam_topk_noalloc): one array per device, in the code object's
// zero-initialised data, held from the module's load until the process ends.
// Host code never uses the array's name as an address (on the host it is a
// stand-in, not device memory): topk_scratch() looks up each device's copy
// once, with that device current, and every later use goes through that
// pointer. Stage 1 writes every entry stage 2 reads, so nothing is cleared.
static __device__ __align__(256) unsigned char scratch[BGA_TOPK_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t topk_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
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
