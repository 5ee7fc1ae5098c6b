// Blocked K/V scan with an fp32 online-softmax state for the packed prefill
// kernel: the building blocks of one wave's work on one 64-key tile.
//
// Rows. A wave owns 32 query rows. In the packed GQA prefill the rows of one
// (sequence, kv head) are the pairs (token t, query head h of the group) in
// token-major order, n = t * G + h; every row of the group reads the same K/V,
// so the G heads never expand K/V and a 32-row block is full whatever G is.
//
// Scores are computed transposed, S^T = K * Q^T, on 32x32x16 bf16 MFMA, so each
// lane ends up holding one query row (lane & 31) and 16 of its keys per 32-key
// block: row max and row sum are in-lane reductions plus one exchange between
// lanes l and l ^ 32 (v_permlane32_swap). The output is accumulated transposed
// as well, O^T = V^T * P^T, with P^T packed straight from the score registers.
//
// K and V tiles are copied global -> LDS with global_load_lds_dwordx4 (no
// register staging; one wave instruction fills 1 KB of LDS, 16 bytes per
// lane, from a wave-uniform base plus a per-lane offset). The LDS side of such
// a copy is contiguous, so rows cannot be padded; the 16-byte chunks of every
// row are XOR-swizzled instead (the lane filling a slot fetches the chunk that
// belongs there), which keeps the reads below free of bank conflicts:
//   K: ds_read_b128 of one row chunk per lane (32 consecutive rows per wave);
//   V: ds_read_b64_tr_b16, which hands every lane one column of four rows,
//      i.e. exactly the V^T operand layout of the MFMA.
//
// Pipelining inside one wave, per tile t (K one tile ahead of V):
//   phase 1: score MFMAs of tile t+1, interleaved with the exponentials of
//            tile t (12 of its 16 value pairs);
//   phase 2: P(t)*V(t) MFMAs of the first 32 keys with the remaining four
//            exponential pairs, then those of the last 32 keys with the
//            (mask and) row maximum of tile t+1.
// Each group of one MFMA and its share of vector work is fenced with a
// scheduling barrier, so the vector ALU issues in the shadow of the matrix
// core instead of the two running one after the other.
//
// Softmax rescaling is lazy: a row's reference maximum only moves (and O and l
// are only rescaled) when a tile raises the row maximum by more than 2^8 in
// probability; until then probabilities up to 256 are accumulated, which fp32
// and bf16 represent as well as values up to 1. The result is the same softmax
// (numerator and denominator use the same reference).
//
// Two row sums are kept. The P*V product sees every probability rounded to
// bf16, so O is normalised by the sum of those same rounded values (ln, one
// v_dot2 per pair): the output is then an exact convex combination of the V
// rows with weights off by the rounding only, which keeps it within 1e-2 of
// the exact softmax for outputs up to 4 in magnitude (a numerator of rounded
// and a denominator of unrounded probabilities can miss by 0.0105 there). The
// log-sum-exp uses the sum of the fp32 probabilities (l).
#pragma once

#include <type_traits>

#include "device_common.hpp"

#define BGA_LDS __attribute__((address_space(3)))

namespace bga {
namespace core {

typedef short i16x4 __attribute__((ext_vector_type(4)));

// One global_load_lds_dwordx4: 64 lanes x 16 bytes from global address
// sbase + voff (wave-uniform 64-bit base, per-lane 32-bit byte offset) into
// 1 KB of LDS at byte address lds_dst (+16 * lane). Inline assembly, so that the
// compiler does not treat the in-flight copy as aliasing every later LDS read
// (it would wait for the copy mid-tile); the scan waits itself (vmcnt(0) +
// barrier) before any wave reads the slot.
__device__ __forceinline__ void dma16(uint64_t sbase, uint32_t voff, uint32_t lds_dst)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_dst)
                 : "memory", "m0");
}

// a wave-uniform 64-bit value kept in scalar registers
__device__ __forceinline__ uint64_t uni64(uint64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return (uint64_t)lo | ((uint64_t)hi << 32);
}

__device__ __forceinline__ void wait_copies_and_sync()
{
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's copies have landed
    __syncthreads();                      // ... and every other wave's
}

template <int D>
struct Geo {
    static constexpr int BN = 64;                 // keys per tile
    static constexpr int ROWB = D * 2;            // bytes per K or V row
    static constexpr int CHUNKS = D / 8;          // 16-byte chunks per row
    static constexpr int KBYTES = BN * ROWB;      // one K (or V) tile
    static constexpr int DMA = KBYTES / 1024;     // 1 KB copies per K (or V) tile
    static constexpr int RPI = 1024 / ROWB;       // rows per copy
    static constexpr int NS = D / 8;              // score MFMAs per tile (2 key blocks x D/16 steps)
    static constexpr int NB = D / 32;             // 32-wide d blocks of O
    static constexpr size_t SMEM = 4 * KBYTES;    // K slots 0, 1, then V slots 0, 1
    static constexpr uint32_t kslot(int j) { return (uint32_t)(j * KBYTES); }
    static constexpr uint32_t vslot(int j) { return (uint32_t)((2 + j) * KBYTES); }

    // chunk swizzles; both have period 16 in the row index
    __device__ static __forceinline__ int swk(int row)
    {
        return D == 128 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
    }
    __device__ static __forceinline__ int swv(int row)
    {
        // rows are read in aligned groups of four
        const int r = row & 3;
        return D == 128 ? ((0xCA60 >> (4 * r)) & 15) : 2 * r;   // {0,6,10,12} / {0,2,4,6}
    }
};

// This wave's share of the copies of one K or V tile. Copy j of wave w is
// instruction i = w + j * NW of the tile: tile rows i * RPI + [0, RPI) into LDS
// bytes i * 1 KB of the slot. NW * RPI is a multiple of 16 rows, so every copy
// of a wave sees the same swizzle and one per-lane offset serves them all.
template <int D, int NW>
struct Copier {
    using G = Geo<D>;
    static constexpr int N = G::DMA / NW;   // copies per wave per tile
    static_assert(G::DMA % NW == 0, "copies must split evenly over the waves");
    static_assert((NW * G::RPI) % 16 == 0, "copy stride must keep the swizzle");
    uint32_t koff, voff;   // per-lane byte offset of a full tile's copy (row within copy, swizzled chunk)
    uint32_t kch, vch;     // swizzled chunk byte offsets
    int lrow;              // lane's row within its copy
    int wave;              // wave-uniform
    uint32_t rbytes;       // global row stride in bytes (uniform)

    __device__ __forceinline__ void init(int wave_, uint32_t rbytes_)
    {
        const int lane = lane_id();
        wave = wave_;
        rbytes = rbytes_;
        lrow = lane / G::CHUNKS;
        const int pc = lane % G::CHUNKS, row0 = wave * G::RPI + lrow;
        kch = (uint32_t)((pc ^ G::swk(row0)) * 16);
        vch = (uint32_t)((pc ^ G::swv(row0)) * 16);
        koff = (uint32_t)lrow * rbytes + kch;
        voff = (uint32_t)lrow * rbytes + vch;
    }

    // Copy the 64 rows starting at global byte address `tile` into the slot at
    // LDS byte address `slot`. `last` is the last valid row of the tile when it
    // is partial (rows past it are clamped to it: valid memory, finite values,
    // masked or never used), or -1 when all 64 rows are valid.
    template <bool IS_V>
    __device__ __forceinline__ void issue(uint32_t slot, uint64_t tile, int last) const
    {
        const uint32_t ch = IS_V ? vch : kch;
        // opaque to the optimiser: the per-copy addresses are formed here, in
        // scalar registers, instead of being hoisted out of the scan as one
        // 64-bit constant per copy and slot (which overflows the scalar file)
        asm volatile("" : "+s"(tile), "+s"(slot));
        if (last < 0) {
            const uint32_t off = IS_V ? voff : koff;
#pragma unroll
            for (int j = 0; j < N; ++j) {
                const int i = wave + j * NW;
                dma16(tile + (uint32_t)(i * G::RPI) * rbytes, off, slot + (uint32_t)(i * 1024));
            }
        } else {
#pragma unroll
            for (int j = 0; j < N; ++j) {
                const int i = wave + j * NW;
                const int r = min(i * G::RPI + lrow, last);
                dma16(tile, (uint32_t)r * rbytes + ch, slot + (uint32_t)(i * 1024));
            }
        }
    }
};

// Per-lane LDS read offsets of the MFMA operands (slot 0; other slots and key
// blocks are immediate offsets).
template <int D>
struct Reads {
    using G = Geo<D>;
    uint32_t k[D / 16];   // K rows (lane & 31), chunk of step ks (this lane's d half)
    uint32_t v[D / 32];   // V^T block b, keys 0..3 (+ multiples of 4 rows)

    __device__ __forceinline__ void init(uint32_t lds_base)
    {
        const int lane = lane_id(), col = lane & 31, half = lane >> 5;
        // rows col and col + 32 share the K swizzle (period 16)
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            k[ks] = lds_base + (uint32_t)(col * G::ROWB + (((ks * 2 + half) ^ G::swk(col)) << 4));
        const int grp = lane >> 4, sl = lane & 15;
        const int row1 = half * 4 + (sl >> 2);
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
            const int colv = b * 32 + (grp & 1) * 16 + (sl & 3) * 4;
            v[b] = lds_base + (uint32_t)(row1 * G::ROWB + (((colv >> 3) ^ G::swv(row1)) << 4) + (colv & 7) * 2);
        }
    }
    __device__ __forceinline__ u32x4 kop(int ks, uint32_t off) const
    {
        return *(const BGA_LDS u32x4 *)(size_t)(k[ks] + off);
    }
    // V^T operand of d block b for keys kbase + [0, 16) of a slot (two transposing reads)
    __device__ __forceinline__ u32x4 vop(int b, uint32_t off) const
    {
        const BGA_LDS char *a = (const BGA_LDS char *)(size_t)(v[b] + off);
        const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BGA_LDS i16x4 *)a);
        const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((BGA_LDS i16x4 *)(a + 8 * G::ROWB));
        const u32x2 xu = __builtin_bit_cast(u32x2, x), yu = __builtin_bit_cast(u32x2, y);
        return u32x4{xu[0], xu[1], yu[0], yu[1]};
    }
};

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

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }
// pins the computation of x before this point (the optimiser would otherwise
// sink it to its first use, out of the interleaved block)
__device__ __forceinline__ void keep(float &x) { asm volatile("" : "+v"(x)); }

// Online-softmax state and the per-tile work of one wave.
template <int D>
struct Wave {
    using G = Geo<D>;
    static constexpr float kLazy = 8.f;   // log2 of the largest unnormalised probability kept
    static constexpr int KLA = D == 128 ? 2 : 2;   // K operand reads issued this many MFMAs ahead
    static constexpr int VLA = D == 128 ? 2 : 2;   // V^T operand reads issued this many MFMAs ahead
    // exponential pairs computed beside the score MFMAs (the rest ride on the
    // first half of the P*V MFMAs; all of the first 32 keys' pairs, 0..7, must
    // be among the former)
    static constexpr int E1 = D == 128 ? 12 : 12;
    static_assert(E1 >= 8 && E1 <= 16, "pairs of keys 0..31 feed the first P*V MFMAs");

    f32x16 o[D / 32];   // O^T: lane holds row (lane & 31), d = b*32 + (r/4)*8 + (lane>>5)*4 + r%4
    float m;            // reference maximum of the raw scores q.k (unscaled)
    float mc;           // m * c2
    float l;            // partial row sum of the fp32 probabilities of the keys this lane holds
    float ln;           // the same over the bf16-rounded probabilities (normalises O)
    uint32_t pk[2][8];  // bf16 P^T of the current tile: pk[kb][j] = keys of elements 2j, 2j+1
    float psum, psn;

    // empty state: no keys seen
    __device__ __forceinline__ void reset()
    {
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
        l = 0.f;
        ln = 0.f;
        m = -INFINITY;
        mc = -INFINITY;
    }

    // probabilities of value pair p (0..15) of tile scores s: block p / 8, elements 2(p%8), 2(p%8)+1
    __device__ __forceinline__ void exp_pair(const f32x16 (&s)[2], int p, float c2)
    {
        const int kb = p >> 3, r = (p & 7) * 2;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c2, -mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c2, -mc));
        const uint32_t packed = pack_bf16x2(p0, p1);
        pk[kb][r >> 1] = packed;
        // fp32 probabilities: the log-sum-exp keeps full precision
        psum = p == 0 ? p0 + p1 : psum + (p0 + p1);
        keep(psum);
        // the rounded probabilities the P*V product sees
        psn = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                              __builtin_bit_cast(bf16x2, 0x3f803f80u), p == 0 ? 0.f : psn, false);
        keep(psn);
    }

    // one P*V MFMA: d block b, keys kb*32 + kk*16 + [0, 16), V^T operand va
    __device__ __forceinline__ void pv(int kb, int kk, int b, const u32x4 &va)
    {
        const u32x4 pb = {pk[kb][kk * 4 + 0], pk[kb][kk * 4 + 1], pk[kb][kk * 4 + 2], pk[kb][kk * 4 + 3]};
        o[b] = mfma32x32x16(as_bf16x8(va), as_bf16x8(pb), o[b]);
    }

    // Mask keys whose offset within the tile exceeds lim (per lane; the tile's
    // first key has offset 0).
    __device__ __forceinline__ static void mask(f32x16 (&s)[2], int lim_tile)
    {
        const int half = lane_id() >> 5;
        const int lim = lim_tile - half * 4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kb * 32 + (r / 4) * 8 + (r % 4) > lim) s[kb][r] = -INFINITY;
    }

    // three-input max as one instruction (the optimiser would otherwise pair
    // the values up first: 24 instead of 17 per tile)
    __device__ __forceinline__ static float max3(float a, float b, float c)
    {
        float r;
        asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
        return r;
    }
    // two independent chains of v_max3 (one per 32-key block), then one max
    __device__ __forceinline__ static float rowmax(const f32x16 (&s)[2])
    {
        float m0 = max3(s[0][0], s[0][1], s[0][2]), m1 = max3(s[1][0], s[1][1], s[1][2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) {
            m0 = max3(m0, s[0][r], s[0][r + 1]);
            m1 = max3(m1, s[1][r], s[1][r + 1]);
        }
        return pair_max(max3(m0, s[0][15], fmaxf(m1, s[1][15])));
    }

    // lazy move of the reference maximum (mx: the row maximum of a new tile)
    __device__ __forceinline__ void update_max(float mx, float c2)
    {
        const bool grow = (mx - m) * c2 > kLazy;
        if (__builtin_expect(__any(grow), 0)) {
            const float m_new = grow ? mx : m;
            const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c2);   // 1 when not growing
            m = m_new;
            mc = m_new * c2;
            l *= alpha;
            ln *= alpha;
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
        }
    }

    // scores of one tile from the K slot at byte offset `ks_off`, no overlap
    __device__ __forceinline__ static void scores(const Reads<D> &rd, const bf16x8 *qop, uint32_t ks_off,
                                                  f32x16 (&s)[2])
    {
        const f32x16 z = {};
        u32x4 ka[3];
        ka[0] = rd.kop(0, ks_off);
        ka[1] = rd.kop(0, ks_off + 32 * G::ROWB);
#pragma unroll
        for (int i = 0; i < G::NS; ++i) {
            if (i + 2 < G::NS) {
                const int j = i + 2;
                ka[j % 3] = rd.kop(j >> 1, ks_off + (uint32_t)((j & 1) * 32 * G::ROWB));
            }
            const int ks = i >> 1, kb = i & 1;
            s[kb] = mfma32x32x16(as_bf16x8(ka[i % 3]), qop[ks], ks == 0 ? z : s[kb]);
            fence();
        }
    }

    // One pipelined step, straight-line code: exponentials and P*V of the
    // current tile (scores sc, V slot at vs_off) and the scores of the next
    // tile into sn (K slot at kn_off). Returns the row maximum of sn as
    // computed (unmasked); a caller that masks sn recomputes it.
    __device__ __forceinline__ float step(const Reads<D> &rd, const bf16x8 *qop, const f32x16 (&sc)[2],
                                          f32x16 (&sn)[2], uint32_t kn_off, uint32_t vs_off, float c2)
    {
        constexpr int NS = G::NS;
        const f32x16 z = {};
        // phase 1: NS score MFMAs (operands KLA ahead) with exponential pairs 0..E1-1
        auto kread = [&](int j) { return rd.kop(j >> 1, kn_off + (uint32_t)((j & 1) * 32 * G::ROWB)); };
        u32x4 ka[KLA + 1];
#pragma unroll
        for (int j = 0; j < KLA; ++j) ka[j] = kread(j);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i + KLA < NS) ka[(i + KLA) % (KLA + 1)] = kread(i + KLA);
            const int ks = i >> 1, kb = i & 1;
            sn[kb] = mfma32x32x16(as_bf16x8(ka[i % (KLA + 1)]), qop[ks], ks == 0 ? z : sn[kb]);
#pragma unroll
            for (int p = i * E1 / NS; p < (i + 1) * E1 / NS; ++p) exp_pair(sc, p, c2);
            fence();
        }
        // phase 2: the 4 * NB P*V MFMAs in order (key block kb, 16-key half kk,
        // d block b), operands VLA ahead; exponential pairs E1..15 ride on the
        // first half (keys 0..31), the next tile's row maximum on the second
        constexpr int NPV = 4 * G::NB;
        auto vread = [&](int mi) {
            const int kb = mi / (2 * G::NB), kk = (mi / G::NB) & 1, b = mi % G::NB;
            return rd.vop(b, vs_off + (uint32_t)((kb * 32 + kk * 16) * G::ROWB));
        };
        u32x4 va[VLA + 1];
#pragma unroll
        for (int j = 0; j < VLA; ++j) va[j] = vread(j);
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            if (i + VLA < NPV) va[(i + VLA) % (VLA + 1)] = vread(i + VLA);
            const int kb = i / (2 * G::NB), kk = (i / G::NB) & 1, b = i % G::NB;
            pv(kb, kk, b, va[i % (VLA + 1)]);
            if (i < NPV / 2) {
#pragma unroll
                for (int p = E1 + i * 2 * (16 - E1) / NPV; p < E1 + (i + 1) * 2 * (16 - E1) / NPV; ++p)
                    exp_pair(sc, p, c2);
                if (i == NPV / 2 - 1) {
                    l += psum;
                    ln += psn;
                }
            } else if (i == NPV / 2) {
                mx = rowmax(sn);
            }
            fence();
        }
        return mx;
    }

    // The last tile of a wave: exponentials and P*V only.
    __device__ __forceinline__ void last(const Reads<D> &rd, const f32x16 (&sc)[2], uint32_t vs_off, float c2)
    {
        constexpr int NPV = 4 * G::NB;
#pragma unroll
        for (int p = 0; p < 8; ++p) exp_pair(sc, p, c2);
        auto vread = [&](int mi) {
            const int kb = mi / (2 * G::NB), kk = (mi / G::NB) & 1, b = mi % G::NB;
            return rd.vop(b, vs_off + (uint32_t)((kb * 32 + kk * 16) * G::ROWB));
        };
        u32x4 va[3];
        va[0] = vread(0);
        va[1] = vread(1);
        fence();
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            if (i + 2 < NPV) va[(i + 2) % 3] = vread(i + 2);
            const int kb = i / (2 * G::NB), kk = (i / G::NB) & 1, b = i % G::NB;
            pv(kb, kk, b, va[i % 3]);
            if (i < NPV / 2) {
#pragma unroll
                for (int p = 8 + i * 16 / NPV; p < 8 + (i + 1) * 16 / NPV; ++p) exp_pair(sc, p, c2);
            }
            fence();
        }
        l += psum;
        ln += psn;
    }

    // Final normalisation and stores of the wave's 32 rows. This lane's row is
    // output row `orow_idx` of `out` ([*, D] bf16), stored if `store`; lse_ptr
    // is its fp32 slot (or nullptr). Lanes l and l ^ 32 hold the two halves of
    // the row, in 8-byte pieces 16 bytes apart, so storing straight from the
    // accumulators would write 16 bytes into each of 32 rows per instruction.
    // Instead the wave writes its bf16 rows into its own LDS region `stage`
    // (32 rows x D, 16-byte chunks XOR-swizzled by row) and reads them back
    // row-major: every global store instruction then writes 64 / (D / 8) whole
    // rows. The region must not be in use by any other wave (the caller
    // synchronises the workgroup before the first wave writes it).
    __device__ __forceinline__ void finish(uint16_t *out, uint32_t orow_idx, float *lse_ptr, bool store, float scale,
                                           uint32_t stage)
    {
        constexpr int CH = D / 8;       // 16-byte chunks per row
        constexpr int RPI = 64 / CH;    // rows per store instruction
        const int lane = lane_id(), col = lane & 31, half = lane >> 5;
        const float lt = pair_sum(l);
        const float inv = 1.f / pair_sum(ln);
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c = b * 4 + rg;   // chunk of d0 = c * 8 + half * 4
                const u32x2 val = {pack_bf16x2(o[b][rg * 4 + 0] * inv, o[b][rg * 4 + 1] * inv),
                                   pack_bf16x2(o[b][rg * 4 + 2] * inv, o[b][rg * 4 + 3] * inv)};
                const uint32_t a = stage + (uint32_t)(col * G::ROWB + ((c ^ (col & (CH - 1))) << 4) + half * 8);
                *(BGA_LDS u32x2 *)(size_t)a = val;
            }
        if (half == 0 && lse_ptr && store) *lse_ptr = m * scale + __logf(lt);
        const int c = lane % CH;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int r = i * RPI + lane / CH;
            const uint32_t ri = (uint32_t)__shfl((int)orow_idx, r);
            const bool ok = __shfl((int)store, r) != 0;
            const u32x4 val =
                *(const BGA_LDS u32x4 *)(size_t)(stage + (uint32_t)(r * G::ROWB + ((c ^ (r & (CH - 1))) << 4)));
            if (ok) __builtin_nontemporal_store(val, (u32x4 *)(out + (size_t)ri * D + c * 8));
        }
    }
};

// The first copies of a scan over keys [0, kend) (tiles [0, nkt), nkt >= 1):
// K and V of tiles 0 and 1 go into their slots at once, so that the scan's
// first tiles do not wait for a copy issued after the prologue.
template <int D, int NW>
__device__ __forceinline__ void first_copies(const Copier<D, NW> &cp, uint32_t lds_base, uint64_t kbase,
                                             uint64_t vbase, int kend, int nkt)
{
    using G = Geo<D>;
    const uint64_t tile_bytes = (uint64_t)G::BN * cp.rbytes;
    const int last0 = kend < G::BN ? kend - 1 : -1;
    cp.template issue<false>(lds_base + G::kslot(0), kbase, last0);
    cp.template issue<true>(lds_base + G::vslot(0), vbase, last0);
    if (nkt > 1) {
        const int last1 = kend < 2 * G::BN ? kend - 1 - G::BN : -1;
        cp.template issue<false>(lds_base + G::kslot(1), kbase + tile_bytes, last1);
        cp.template issue<true>(lds_base + G::vslot(1), vbase + tile_bytes, last1);
    }
}

// The blocked scan over keys [0, kend) of one K/V range, shared by the
// prefill and decode kernels. Tile kt holds keys 64 kt + [0, 64); K/V row `key`
// lives at byte address kbase / vbase + key * row stride. Every wave of the
// workgroup calls this (it holds the barriers) with the workgroup's tile count
// nkt; the wave computes tiles [0, nkt_w) only. Keys past `lim` (this lane's
// last allowed key) are masked in tiles kt >= kt_mask. The caller has issued
// first_copies (tiles 0 and 1) and waited for them (wait_copies_and_sync);
// the state st is empty when `fresh`, else it may already hold keys.
// extra(kt) runs in every tile step, after that step's barrier and copies.
struct NoExtra {
    __device__ __forceinline__ void operator()(int) const {}
};

template <int D, int NW, typename Extra = NoExtra>
__device__ __forceinline__ void scan(Wave<D> &st, const Reads<D> &rd, const Copier<D, NW> &cp, const bf16x8 *qop,
                                     uint32_t lds_base, uint64_t kbase, uint64_t vbase, int kend, int nkt, int nkt_w,
                                     int lim, int kt_mask, float c2, bool fresh, Extra extra = Extra())
{
    using G = Geo<D>;
    const uint64_t tile_bytes = (uint64_t)G::BN * cp.rbytes;
    auto last_row = [&](int kt) { return kt * G::BN + G::BN > kend ? kend - 1 - kt * G::BN : -1; };

    f32x16 sa[2], sb[2];
    if (nkt_w > 0) {
        Wave<D>::scores(rd, qop, G::kslot(0), sa);
        if (kt_mask == 0) Wave<D>::mask(sa, lim);
        const float mx = Wave<D>::rowmax(sa);
        if (fresh) {   // every row has a key in tile 0
            st.m = mx;
            st.mc = mx * c2;
        } else {
            st.update_max(mx, c2);
        }
    }
    // Tile kt: K(kt) and V(kt) sit in slot kt & 1. Every tile starts with a
    // barrier after which K(kt+2) and V(kt+1) are copied into the slots that
    // K(kt) and V(kt-1) held (V(1) came with the first copies).
    auto sync_and_copy = [&](int kt) {
        wait_copies_and_sync();   // K(kt+1), V(kt) landed; K(kt), V(kt-1) no longer read
        const uint32_t p = (uint32_t)(kt & 1);
        if (kt + 2 < nkt)
            cp.template issue<false>(lds_base + p * G::KBYTES, kbase + (uint64_t)(kt + 2) * tile_bytes,
                                     last_row(kt + 2));
        if (kt >= 1 && kt + 1 < nkt)
            cp.template issue<true>(lds_base + G::vslot(0) + (1 - p) * G::KBYTES,
                                    vbase + (uint64_t)(kt + 1) * tile_bytes, last_row(kt + 1));
        extra(kt);
    };
    // all but the wave's last tile: exponentials and P*V of tile kt, scores of kt+1
    auto step = [&](int kt, auto parity, f32x16(&sc)[2], f32x16(&sn)[2]) {
        constexpr int P = decltype(parity)::value;
        sync_and_copy(kt);
        float mx = st.step(rd, qop, sc, sn, G::kslot(1 - P), G::vslot(P), c2);
        if (kt + 1 >= kt_mask) {   // the next tile has keys past some row's limit
            Wave<D>::mask(sn, lim - (kt + 1) * G::BN);
            mx = Wave<D>::rowmax(sn);
        }
        st.update_max(mx, c2);
    };
    const int klast = nkt_w - 1;
    int kt = 0;
    for (; kt + 1 < klast; kt += 2) {
        step(kt, std::integral_constant<int, 0>{}, sa, sb);
        step(kt + 1, std::integral_constant<int, 1>{}, sb, sa);
    }
    if (kt < klast) {
        step(kt, std::integral_constant<int, 0>{}, sa, sb);
        ++kt;
    }
    // the wave's last tile
    if (kt == klast) {
        sync_and_copy(kt);
        if ((kt & 1) == 0)
            st.last(rd, sa, G::vslot(0), c2);
        else
            st.last(rd, sb, G::vslot(1), c2);
        ++kt;
    }
    // the workgroup's remaining tiles: copies and barriers only
    for (; kt < nkt; ++kt) sync_and_copy(kt);
}

// Q^T operand of one lane: query row `qrow` (D elements), k slots (lane>>5)*8 + [0,8)
// of every 16-wide d step.
template <int D>
__device__ __forceinline__ void load_q(bf16x8 *qop, const uint16_t *qrow)
{
    const int half = lane_id() >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qop[ks] = as_bf16x8(*(const u32x4 *)(qrow + ks * 16 + half * 8));
}

}  // namespace core
}  // namespace bga
