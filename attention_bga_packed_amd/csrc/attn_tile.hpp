// Blocked K/V scan with an fp32 online-softmax state, shared by the packed
// prefill and the shared-prefix decode kernels.
//
// One wave owns 32 query rows. Scores are computed transposed, S^T = K * Q^T,
// on 32x32x16 bf16 MFMA so that each lane ends up holding one query row (lane
// & 31) and 16 of its keys per 32-key block: the row max and row sum are then
// in-lane reductions plus one exchange between lanes l and l^32
// (v_permlane32_swap). The output is accumulated transposed as well,
// O^T = V^T * P^T, with P^T taken straight from the score accumulators.
//
// A tile is 64 keys. K and V are copied global -> LDS with no register staging
// (global_load_lds_dwordx4: each wave instruction fills 1 KB of LDS, 16 bytes
// per lane, from any 16-byte-aligned global address per lane), both row-major.
// Since the LDS side of such a copy is contiguous, rows cannot be padded;
// instead the 16-byte chunks of every row are XOR-swizzled (the lane filling a
// slot fetches the chunk that belongs there) so that the reads below are free
// of bank conflicts for both 32- and 64-bank LDS organisations:
//   K: ds_read_b128 of one row chunk per lane (32 consecutive rows per wave);
//   V: ds_read_b64_tr_b16, which hands lane i of each 16-lane group the same
//      column of four rows, i.e. exactly the V^T operand layout the MFMA wants.
//
// K and V tiles are double-buffered, K one tile ahead of V. One step of the
// scan does, for tile t, in a single branch-free block: the MFMAs of the
// scores of tile t+1, the exponentials of tile t, and the MFMAs of P(t)*V(t);
// scheduling barriers interleave the MFMAs with the exponentials so that the
// matrix cores and the vector ALU work at the same time within one wave.
// The copies of K(t+2) and V(t+1) are in flight meanwhile.
//
// Softmax rescaling is lazy: a row's reference maximum only moves (and O and l
// are only rescaled) when a tile raises the row maximum by more than 2^8 in
// probability; until then probabilities up to 256 are accumulated, which fp32
// and bf16 represent as well as values up to 1. The result is the same softmax
// (the final division uses the same reference).
#pragma once

#include "device_common.hpp"

#define BGA_LDS __attribute__((address_space(3)))

namespace bga {

typedef short i16x4 __attribute__((ext_vector_type(4)));

// One global_load_lds_dwordx4: 64 lanes x 16 bytes from global addresses
// sbase + voff (a wave-uniform base and a per-lane byte offset) into 1 KB of
// LDS at byte address `lds_dst` (+16 * lane). Written as
// inline assembly so that the compiler does not treat the in-flight copy as
// aliasing every later LDS read (which would make it wait for the copy
// mid-tile); the callers wait for completion themselves (s_waitcnt vmcnt(0) +
// barrier) before any wave reads the slot.
__device__ __forceinline__ void lds_dma16(const void *sbase, uint32_t voff, uint32_t lds_dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
    const uint64_t a = (uint64_t)(size_t)sbase;
    // readfirstlane yields a signed int: widen through uint32_t (no sign extension)
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint64_t sa = lo | (hi << 32);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sa), "s"(m0)
                 : "memory", "m0");
}

__device__ __forceinline__ const BGA_LDS char *lds_ptr(const void *p) { return (const BGA_LDS char *)p; }
__device__ __forceinline__ uint32_t lds_addr(const BGA_LDS char *p) { return (uint32_t)(size_t)p; }

template <int D>
struct AttnTile {
    static constexpr int BN = 64;                 // keys per tile
    static constexpr int ROWB = D * 2;            // bytes per K or V row
    static constexpr int CHUNKS = D / 8;          // 16-byte chunks per row
    static constexpr int KBYTES = BN * ROWB;      // one K (or V) tile
    static constexpr size_t SMEM_BYTES = 4 * KBYTES;   // K slots 0,1 then V slots 0,1
    static constexpr int DMA = KBYTES / 1024;     // 1 KB copy instructions per K (or V) tile
    static constexpr int RPI = 1024 / ROWB;       // rows per copy instruction
    static constexpr int MAXI = DMA / 4;          // copies per wave per tile (>= 4 waves)

    // chunk swizzles (see the header comment)
    __device__ static __forceinline__ int swk(int row)
    {
        return D == 128 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
    }
    __device__ static __forceinline__ int swv(int row)
    {
        // rows are read in aligned groups of four; see the header comment
        const int r = row & 3;
        return D == 128 ? ((0xCA60 >> (4 * r)) & 15) : 2 * r;   // {0,6,10,12} / {0,2,4,6}
    }
    // byte offsets of the slots inside the dynamic LDS block
    static constexpr uint32_t kslot(int j) { return (uint32_t)(j * KBYTES); }
    static constexpr uint32_t vslot(int j) { return (uint32_t)((2 + j) * KBYTES); }
};

// This wave's share of the copies of one tile: copy j of the wave is
// instruction i = wave + j * nwaves of the tile; it moves tile row row(j)
// (0..63), chunk-swizzled, into bytes i * 1 KB of the slot. Each lane keeps
// its byte offset within the row (the swizzled chunk); the row offset goes
// into the wave-uniform base wherever possible. NW is the number of waves when
// known at compile time (0: run-time). When NW copies cover a multiple of 16
// rows, row(j) - row(0) is a multiple of 16, the swizzle of every copy equals
// that of copy 0, and one set of per-lane values serves all copies.
template <int D, int NW = 0>
struct DmaPlan {
    using T = AttnTile<D>;
    static constexpr bool kStrided = NW > 0 && (NW * T::RPI) % 16 == 0;
    static constexpr int kSlots = kStrided ? 1 : T::MAXI;
    int wave, nwaves, n;                 // wave-uniform: copies this wave issues per tile
    int row[kSlots];                     // tile row of copy j (kStrided: of copy 0)
    uint32_t kch[kSlots], vch[kSlots];   // byte offset of this lane's 16 bytes within the K / V row

    __device__ __forceinline__ void init(int wave_, int nwaves_)
    {
        const int lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(wave_);
        nwaves = NW > 0 ? NW : __builtin_amdgcn_readfirstlane(nwaves_);
        n = 0;
#pragma unroll
        for (int j = 0; j < T::MAXI; ++j) n += wave + j * nwaves < T::DMA;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            const int r = (wave + j * nwaves) * T::RPI + lane / T::CHUNKS, pc = lane % T::CHUNKS;
            row[j] = r;
            kch[j] = (uint32_t)((pc ^ T::swk(r)) * 16);
            vch[j] = (uint32_t)((pc ^ T::swv(r)) * 16);
        }
    }

    // Copy rows [kstart, kstart + 64) of one matrix into the slot at LDS byte
    // address `slot`. Rows >= kend are clamped to kend - 1 (valid memory; those
    // keys are masked or never used).
    __device__ __forceinline__ void issue(uint32_t slot, const uint16_t *__restrict__ base, uint32_t row_stride,
                                          int kstart, int kend, bool is_v) const
    {
        const char *b = (const char *)(base + (size_t)kstart * row_stride);
        const uint32_t rbytes = row_stride * 2;
        const bool full = kstart + T::BN <= kend;
        const int last = kend - 1 - kstart;   // last valid tile row
#pragma unroll
        for (int j = 0; j < T::MAXI; ++j)
            if (j < n) {
                const int s = kStrided ? 0 : j;
                const uint32_t ch = is_v ? vch[s] : kch[s];
                const uint32_t dst = slot + (uint32_t)((wave + j * nwaves) * 1024);
                if constexpr (kStrided) {
                    // copy j = copy 0 moved down by j * NW * RPI rows
                    const int dr = j * NW * T::RPI;
                    if (full) {
                        lds_dma16(b + (size_t)dr * rbytes, (uint32_t)row[0] * rbytes + ch, dst);
                    } else {
                        const int r = min(row[0] + dr, last);
                        lds_dma16(b, (uint32_t)r * rbytes + ch, dst);
                    }
                } else {
                    const int r = full ? row[j] : min(row[j], last);
                    lds_dma16(b, (uint32_t)r * rbytes + ch, dst);
                }
            }
    }
};

// value of x at lane l ^ 32 combined with x, via v_permlane32_swap
__device__ __forceinline__ float pair_max(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Online-softmax state of one wave (32 query rows) and its per-lane LDS read offsets.
template <int D>
struct WaveAttn {
    using T = AttnTile<D>;
    f32x16 o[D / 32];   // O^T: lane holds query (lane & 31), d = blk*32 + (r/4)*8 + (lane>>5)*4 + r%4
    float m;            // reference max of raw scores q.k (unscaled)
    float l;            // partial sum over the keys this lane holds
    const BGA_LDS char *kofs[D / 16];   // K read of step ks (row lane&31, first 32 rows), slot 0
    const BGA_LDS char *vofs[D / 32];   // V^T read of block b, keys 0..3 of the tile, slot 0

    static constexpr float kLazy = 8.f;   // log2 of the largest unnormalised probability kept

    // empty state: no keys seen
    __device__ __forceinline__ void reset()
    {
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
        m = -INFINITY;
        l = 0.f;
    }

    __device__ __forceinline__ void init(const BGA_LDS char *lds_base)
    {
        reset();
        const int lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
        // rows col and col + 32 share the K swizzle (it looks at the low four bits only)
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            kofs[ks] = lds_base + (col * T::ROWB + (((ks * 2 + half) ^ T::swk(col)) << 4));
        const int g = lane >> 4, sl = lane & 15;
        const int row1 = half * 4 + (sl >> 2);   // other reads: + multiples of 4 rows, same V swizzle
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
            const int colv = b * 32 + (g & 1) * 16 + (sl & 3) * 4;
            vofs[b] = lds_base + (row1 * T::ROWB + (((colv >> 3) ^ T::swv(row1)) << 4) + (colv & 7) * 2);
        }
    }

    // Mask, row max and (lazy) rescale for the scores s of one tile. Keys with
    // index (kstart + offset) > limit are masked when need_mask. Returns the
    // exponent offset m * c2 for the probabilities.
    __device__ __forceinline__ float prepare(f32x16 (&s)[2], float c2, bool need_mask, int kstart, int limit)
    {
        const int half = (threadIdx.x & 63) >> 5;
        if (need_mask) {
            // element (kb, r) holds key kstart + kb*32 + (r/4)*8 + half*4 + r%4; it is
            // masked when its offset kb*32 + (r/4)*8 + r%4 exceeds thr
            const int thr = limit - kstart - half * 4;
            const bool hi_masked = __all(thr < 32);   // the second 32 keys are masked for every row
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if ((r / 4) * 8 + (r % 4) > thr) s[0][r] = -INFINITY;
            if (hi_masked) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[1][r] = -INFINITY;
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 + (r / 4) * 8 + (r % 4) > thr) s[1][r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
        mx = pair_max(mx);
        const bool grow = (mx - m) * c2 > kLazy;   // first tile: m = -inf -> grow
        if (__any(grow)) {
            const float m_new = grow ? mx : m;
            const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c2);   // 1 when not growing
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
        }
        return m * c2;
    }

    // Scores of one tile from K slot KSLOT (byte offset from the LDS base).
    template <uint32_t KSLOT>
    __device__ __forceinline__ void scores(const bf16x8 *qop, f32x16 (&s)[2]) const
    {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 a = *(const BGA_LDS u32x4 *)(kofs[ks] + (KSLOT + kb * 32 * T::ROWB));
                s[kb] = mfma32x32x16(as_bf16x8(a), qop[ks], s[kb]);
            }
        // K reads run two MFMAs ahead, no further (bounded register pressure)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }

    // The fused step body (no branches): scores of the next tile into sn from
    // K slot KNEXT, probabilities of the current tile from sc (after prepare()),
    // and O += P * V from V slot VCUR.
    template <uint32_t KNEXT, uint32_t VCUR>
    __device__ __forceinline__ void fused(const bf16x8 *qop, const f32x16 (&sc)[2], f32x16 (&sn)[2], float c2,
                                          float mc)
    {
        scores<KNEXT>(qop, sn);
        uint32_t pk[2][8];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], c2, -mc));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r + 1], c2, -mc));
                pk[kb][r / 2] = pack_bf16x2(p0, p1);
                psum += p0 + p1;   // fp32 probabilities: the log-sum-exp keeps full precision
            }
        l += psum;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4 pv = {pk[kb][kk * 4 + 0], pk[kb][kk * 4 + 1], pk[kb][kk * 4 + 2], pk[kb][kk * 4 + 3]};
#pragma unroll
                for (int b = 0; b < D / 32; ++b) {
                    // V^T operand: two transposing reads of four keys each
                    const BGA_LDS char *a1 = vofs[b] + (VCUR + (kb * 32 + kk * 16) * T::ROWB);
                    const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BGA_LDS i16x4 *)a1);
                    const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BGA_LDS i16x4 *)(a1 + 8 * T::ROWB));
                    const u32x2 xu = __builtin_bit_cast(u32x2, x), yu = __builtin_bit_cast(u32x2, y);
                    const u32x4 va = {xu[0], xu[1], yu[0], yu[1]};
                    o[b] = mfma32x32x16(as_bf16x8(va), as_bf16x8(pv), o[b]);
                }
            }
        // Interleave: while the score MFMAs of the next tile run, the
        // exponentials of this tile issue behind them; then the P*V MFMAs, each
        // with its two transposing V reads and the remaining vector work.
        constexpr int NS = D / 8;                // score MFMAs (2 blocks x D/16 steps)
        constexpr int VS = D == 128 ? 6 : 11;    // vector instructions behind each of them
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // LDS reads run two MFMAs ahead
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            __builtin_amdgcn_sched_group_barrier(0x002, VS, 0);  // VALU
        }
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads (V^T operand)
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
        }
    }

    // Final normalisation and stores for this lane's query row.
    // orow: output row [D] of this query; lse_ptr: fp32 slot or nullptr.
    __device__ __forceinline__ void finish(uint16_t *orow, float *lse_ptr, bool row_valid, float scale)
    {
        const int lane = threadIdx.x & 63, half = lane >> 5;
        const float lt = pair_sum(l);
        const float inv = 1.f / lt;
        if (!row_valid) return;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = b * 32 + rg * 8 + half * 4;
                const u32x2 val = {pack_bf16x2(o[b][rg * 4 + 0] * inv, o[b][rg * 4 + 1] * inv),
                                   pack_bf16x2(o[b][rg * 4 + 2] * inv, o[b][rg * 4 + 3] * inv)};
                *(u32x2 *)(orow + d0) = val;
            }
        if (half == 0 && lse_ptr) *lse_ptr = m * scale + __logf(lt);
    }
};

// Q^T operand of one lane: query row `qrow` (D elements), k-slots (lane>>5)*8 + [0,8)
// of every 16-wide d step. Invalid rows get zeros.
template <int D>
__device__ __forceinline__ void load_q_operand(bf16x8 *qop, const uint16_t *qrow, bool valid)
{
    const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (valid) v = *(const u32x4 *)(qrow + ks * 16 + half * 8);
        qop[ks] = as_bf16x8(v);
    }
}

struct Parity0 { static constexpr int value = 0; };
struct Parity1 { static constexpr int value = 1; };

// Copies of the first tile's K and V into slots 0 (the scan's prologue; a
// caller may issue them early and pass first_issued = true to the scan).
template <int D, typename Plan>
__device__ __forceinline__ void attn_scan_first(const Plan &plan, uint32_t lds_base, const uint16_t *kbase,
                                                const uint16_t *vbase, uint32_t row_stride, int key0, int kend)
{
    using T = AttnTile<D>;
    plan.issue(lds_base + T::kslot(0), kbase, row_stride, key0, kend, false);
    plan.issue(lds_base + T::vslot(0), vbase, row_stride, key0, kend, true);
}

// The double-buffered scan over tiles [0, nkt) shared by both kernels.
// Tile kt holds keys [key0 + 64*kt, key0 + 64*kt + 64); K/V row `key` lives at
// kbase/vbase + key * row_stride; keys >= kend are clamped. need_mask(kt) says
// whether tile kt is masked (keys > mask_limit). Every wave of the workgroup
// must call this (it contains barriers); waves without work compute on
// whatever their inputs are and discard the result. The state st may already
// hold keys folded in by the caller.
template <int D, typename Plan, typename NeedMask>
__device__ __forceinline__ void attn_scan(WaveAttn<D> &st, const Plan &plan, uint32_t lds_base,   // LDS byte address
                                          const bf16x8 *qop, const uint16_t *kbase, const uint16_t *vbase,
                                          uint32_t row_stride, int key0, int kend, int nkt, float c2,
                                          NeedMask need_mask, int mask_limit, bool first_issued = false)
{
    using T = AttnTile<D>;
    if (nkt <= 0) return;
    if (!first_issued) attn_scan_first<D>(plan, lds_base, kbase, vbase, row_stride, key0, kend);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    __syncthreads();
    if (nkt > 1) plan.issue(lds_base + T::kslot(1), kbase, row_stride, key0 + T::BN, kend, false);
    f32x16 sa[2], sb[2];
    st.template scores<T::kslot(0)>(qop, sa);
    // the step for tile kt, whose K sits in slot P = kt & 1: consume sc, fill sn
    auto step = [&](int kt, auto parity, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
        constexpr int P = decltype(parity)::value;
        const int kstart = key0 + kt * T::BN;
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): K(kt+1) and V(kt) have landed (this wave's copies)
        __syncthreads();                      // ... every wave's; K(kt) and V(kt-1) are no longer read
        if (kt + 2 < nkt) plan.issue(lds_base + T::kslot(P), kbase, row_stride, kstart + 2 * T::BN, kend, false);
        if (kt + 1 < nkt) plan.issue(lds_base + T::vslot(1 - P), vbase, row_stride, kstart + T::BN, kend, true);
        const float mc = st.prepare(sc, c2, need_mask(kt), kstart, mask_limit);
        st.template fused<T::kslot(1 - P), T::vslot(P)>(qop, sc, sn, c2, mc);
    };
    for (int kt = 0; kt < nkt; kt += 2) {   // unrolled by two: slots and score buffers alternate
        step(kt, Parity0{}, sa, sb);
        if (kt + 1 < nkt) step(kt + 1, Parity1{}, sb, sa);
    }
}

}  // namespace bga
