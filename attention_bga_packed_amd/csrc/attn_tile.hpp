// Blocked K/V scan with an fp32 online-softmax state, shared by the packed
// prefill and the shared-prefix decode kernels.
//
// One wave owns 32 query rows. Scores are computed transposed, S^T = K * Q^T,
// on 32x32x16 bf16 MFMA so that each lane ends up holding one query row (lane
// & 31) and 16 of its keys per 32-key block: the row max and row sum are then
// in-lane reductions plus one exchange with lane ^ 32. The output is
// accumulated transposed as well, O^T = V^T * P^T, with P^T taken straight from
// the score accumulators (no LDS round trip for P).
//
// A tile is 64 keys. K is staged in LDS row-major ([key][d], rows padded by 8
// elements); V is staged transposed ([d][key], rows padded by 4) so that the
// eight keys one lane feeds to an MFMA k-slot group are two 8-byte LDS reads.
// Both pads make the LDS reads bank-conflict free. Tiles are double-buffered:
// the global loads of tile t+1 are in flight while tile t is computed.
#pragma once

#include "device_common.hpp"

namespace bga {

template <int D>
struct AttnTile {
    static constexpr int BN = 64;            // keys per tile
    static constexpr int KS = D + 8;         // K row stride in LDS (elements)
    static constexpr int VS = BN + 4;        // V^T row stride in LDS (elements)
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr size_t SMEM_BYTES = 2 * STAGE * sizeof(uint16_t);
    static constexpr int KCH = BN * D / 8;          // 16-byte chunks of a K tile
    static constexpr int VTASK = (BN / 4) * (D / 8); // 4-key x 8-d transpose tasks
    // launches always use >= 256 threads per workgroup
    static constexpr int K_IT = (KCH + 255) / 256;
    static constexpr int V_IT = (VTASK + 255) / 256;

    u32x4 kreg[K_IT];
    u32x4 vreg[V_IT][4];

    // Global -> registers for keys [kstart, kstart + 64). Row `key` of K lives at
    // kbase + key * row_stride; keys >= kend are zero-filled (never read).
    __device__ __forceinline__ void load(const uint16_t *__restrict__ kbase, const uint16_t *__restrict__ vbase,
                                         size_t row_stride, int kstart, int kend, int tid, int nthr)
    {
#pragma unroll
        for (int i = 0; i < K_IT; ++i) {
            const int c = tid + i * nthr;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (c < KCH) {
                const int row = c / (D / 8), cc = (c % (D / 8)) * 8;
                const int key = kstart + row;
                if (key < kend) val = *(const u32x4 *)(kbase + (size_t)key * row_stride + cc);
            }
            kreg[i] = val;
        }
#pragma unroll
        for (int i = 0; i < V_IT; ++i) {
            const int c = tid + i * nthr;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x4 val = {0u, 0u, 0u, 0u};
                if (c < VTASK) {
                    const int dchunk = c % (D / 8), kg = c / (D / 8);
                    const int key = kstart + kg * 4 + j;
                    if (key < kend) val = *(const u32x4 *)(vbase + (size_t)key * row_stride + dchunk * 8);
                }
                vreg[i][j] = val;
            }
        }
    }

    // Registers -> one LDS stage (K row-major, V transposed).
    __device__ __forceinline__ void store(uint16_t *stage, int tid, int nthr) const
    {
        uint16_t *Ks = stage;
        uint16_t *Vt = stage + K_ELEMS;
#pragma unroll
        for (int i = 0; i < K_IT; ++i) {
            const int c = tid + i * nthr;
            if (c < KCH) {
                const int row = c / (D / 8), cc = (c % (D / 8)) * 8;
                *(u32x4 *)(Ks + row * KS + cc) = kreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < V_IT; ++i) {
            const int c = tid + i * nthr;
            if (c < VTASK) {
                const int dchunk = c % (D / 8), kg = c / (D / 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t a0 = vreg[i][0][e / 2], a1 = vreg[i][1][e / 2];
                    const uint32_t a2 = vreg[i][2][e / 2], a3 = vreg[i][3][e / 2];
                    uint32_t lo, hi;
                    if (e & 1) {
                        lo = (a0 >> 16) | (a1 & 0xffff0000u);
                        hi = (a2 >> 16) | (a3 & 0xffff0000u);
                    } else {
                        lo = (a0 & 0xffffu) | (a1 << 16);
                        hi = (a2 & 0xffffu) | (a3 << 16);
                    }
                    u32x2 pair = {lo, hi};
                    *(u32x2 *)(Vt + (dchunk * 8 + e) * VS + kg * 4) = pair;
                }
            }
        }
    }
};

// Online-softmax state of one wave (32 query rows).
template <int D>
struct WaveAttn {
    f32x16 o[D / 32];   // O^T: lane holds query (lane & 31), d = blk*32 + (r/4)*8 + (lane>>5)*4 + r%4
    float m;            // running max of raw scores q.k (unscaled)
    float l;            // partial sum over the keys this lane holds

    __device__ __forceinline__ void init()
    {
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
        m = -INFINITY;
        l = 0.f;
    }

    // One 64-key tile staged in LDS. c2 = softmax_scale * log2(e).
    // Keys with index (kstart + offset) > limit are masked when need_mask.
    __device__ __forceinline__ void tile(const uint16_t *Ks, const uint16_t *Vt, const bf16x8 *qop, float c2,
                                         bool need_mask, int kstart, int limit)
    {
        using T = AttnTile<D>;
        const int lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const u32x4 a = *(const u32x4 *)(Ks + (kb * 32 + col) * T::KS + ks * 16 + half * 8);
                s[kb] = mfma32x32x16(as_bf16x8(a), qop[ks], s[kb]);
            }
        }
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kstart + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
                    if (key > limit) s[kb][r] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c2);
        const float mc = m_new * c2;
        uint32_t pk[2][8];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c2, -mc));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c2, -mc));
                psum += p0 + p1;
                pk[kb][r / 2] = pack_bf16x2(p0, p1);
            }
        l = l * alpha + psum;
        m = m_new;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4 pv = {pk[kb][kk * 4 + 0], pk[kb][kk * 4 + 1], pk[kb][kk * 4 + 2], pk[kb][kk * 4 + 3]};
                const bf16x8 pop = as_bf16x8(pv);
#pragma unroll
                for (int b = 0; b < D / 32; ++b) {
                    const uint16_t *vrow = Vt + (b * 32 + col) * T::VS + kb * 32 + kk * 16 + half * 4;
                    const u32x2 v0 = *(const u32x2 *)(vrow);
                    const u32x2 v1 = *(const u32x2 *)(vrow + 8);
                    const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
                    o[b] = mfma32x32x16(as_bf16x8(va), pop, o[b]);
                }
            }
    }

    // Final normalisation and stores for this lane's query row.
    // orow: output row [D] of this query; lse_ptr: fp32 slot or nullptr.
    __device__ __forceinline__ void finish(uint16_t *orow, float *lse_ptr, bool row_valid, float scale)
    {
        const int lane = threadIdx.x & 63, half = lane >> 5;
        const float lt = l + xor32(l);
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

}  // namespace bga
