// Packed variable-length causal GQA prefill for gfx950.
//
// Article section 3.1 ("变长样本的 Packed Prefill"): sequences are packed back to
// back as Q [T, Nq, D], K/V [T, Nkv, D]; the sequence boundary (cu_seqlens)
// implies a block-diagonal causal mask; the kernel never expands GQA K/V heads
// and never materialises the score matrix; for each query block it derives the
// valid K/V range from the boundary and scans it blockwise with an fp32 online
// softmax.
//
// Work unit = (kv head g, sequence, query tile of BM = 32*TS tokens). The
// workgroup holds H*TS waves (H = up to 8 of the group's G query heads at
// d 128, up to 4 at d 64; larger groups are split over several workgroups):
// wave w serves one query head for the 32 tokens of sub-tile w / H, so every
// K/V tile staged in LDS is shared by H query heads and TS sub-tiles. Keys run
// from the start of the sequence to the end of the query tile; only tiles
// that reach past a wave's first query are masked.
//
// Grid = (Nkv * splits, B, max tiles per sequence). The tile index is reversed so the
// longest (last) query tiles of every sequence are dispatched first. With
// consecutive workgroups dealt round-robin over the 8 XCDs, putting the kv head
// in x keeps all tiles of one (sequence, kv head) on the same XCD (and L2)
// when Nkv is a multiple of 8.
#include "attn_tile.hpp"
#include "internal.hpp"

namespace bga {

// NW: waves per workgroup when fixed at compile time (0: any)
template <int D, int NW>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2))) void packed_prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ cu, int nq, int nkv, int group, int hsplit, int hpw, int ts_per_wg, float scale,
    uint16_t *__restrict__ out, float *__restrict__ lse)
{
    using T = AttnTile<D>;
    extern __shared__ __align__(16) uint16_t smem[];

    const int g = blockIdx.x / hsplit, split = blockIdx.x % hsplit, seq = blockIdx.y;
    const int bm = 32 * ts_per_wg;
    const int tile = gridDim.z - 1 - blockIdx.z;
    const int s0 = cu[seq], s1 = cu[seq + 1];
    const int q_lo = s0 + tile * bm;
    if (q_lo >= s1) return;  // uniform over the workgroup
    const int kend = min(q_lo + bm, s1);
    const int nkt = (kend - s0 + T::BN - 1) / T::BN;

    const int nthr = blockDim.x;
    const int w = threadIdx.x >> 6, col = threadIdx.x & 31;
    const int hig = split * hpw + (w % hpw);   // head within the group
    const int head = g * group + min(hig, group - 1);
    const int qw0 = q_lo + (w / hpw) * 32;
    const int qtok = qw0 + col;
    const bool wave_active = qw0 < s1 && hig < group;
    const bool row_valid = qtok < s1 && wave_active;

    bf16x8 qop[D / 16];
    load_q_operand<D>(qop, q + ((size_t)qtok * nq + head) * D, row_valid);

    const BGA_LDS char *lds = lds_ptr(smem);
    const uint32_t lds_base = lds_addr(lds);
    WaveAttn<D> st;
    st.init(lds);
    const float c2 = scale * kLog2e;
    const uint32_t row_stride = (uint32_t)(nkv * D);
    DmaPlan<D, NW> plan;
    plan.init(w, nthr >> 6);
    // tile kt needs masking when it reaches past this wave's first query; tiles
    // entirely after the wave's last query are fully masked (contribute zero)
    auto need_mask = [&](int kt) { return s0 + kt * AttnTile<D>::BN + AttnTile<D>::BN - 1 > qw0; };
    attn_scan<D>(st, plan, lds_base, qop, k + (size_t)g * D, v + (size_t)g * D, row_stride, s0, kend, nkt, c2,
                 need_mask, qtok);
    if (!wave_active) return;
    st.finish(out + ((size_t)qtok * nq + head) * D, lse ? lse + (size_t)qtok * nq + head : nullptr, row_valid,
              scale);
}

template <int D>
static hipError_t launch_prefill_d(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *cu,
                                   int num_seqs, int max_seqlen, int nq, int nkv, float scale, uint16_t *out,
                                   float *lse, hipStream_t stream)
{
    const int group = nq / nkv;
    // At d 64 a wave fits in 168 registers (3 waves per SIMD, 12 per CU): groups are
    // split into workgroups of <= 4 query heads so that several workgroups share a
    // CU and one's prologue and epilogue overlap another's tiles. At d 128 (2 waves
    // per SIMD) up to 8 heads share a workgroup.
    const int hsplit = D == 64 ? (group + 3) / 4 : (group + 7) / 8;
    const int hpw = (group + hsplit - 1) / hsplit;
    const int ts = hpw >= 4 ? 1 : (hpw == 1 ? 4 : 2); // >= 4 waves per workgroup
    const int bm = 32 * ts;
    const int tiles = (max_seqlen + bm - 1) / bm;
    const int nw = hpw * ts;
    const void *kern = nw == 4   ? (const void *)packed_prefill_kernel<D, 4>
                       : nw == 8 ? (const void *)packed_prefill_kernel<D, 8>
                                 : (const void *)packed_prefill_kernel<D, 0>;
    const size_t smem = AttnTile<D>::SMEM_BYTES;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    dim3 grid(nkv * hsplit, num_seqs, tiles), block(64 * nw);
    if (nw == 4)
        hipLaunchKernelGGL((packed_prefill_kernel<D, 4>), grid, block, smem, stream, q, k, v, cu, nq, nkv, group, hsplit,
                           hpw, ts, scale, out, lse);
    else if (nw == 8)
        hipLaunchKernelGGL((packed_prefill_kernel<D, 8>), grid, block, smem, stream, q, k, v, cu, nq, nkv, group, hsplit,
                           hpw, ts, scale, out, lse);
    else
        hipLaunchKernelGGL((packed_prefill_kernel<D, 0>), grid, block, smem, stream, q, k, v, cu, nq, nkv, group, hsplit,
                           hpw, ts, scale, out, lse);
    return hipGetLastError();
}

hipError_t launch_packed_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *cu,
                                 int num_seqs, int max_seqlen, int nq, int nkv, int d, float scale, uint16_t *out,
                                 float *lse, hipStream_t stream)
{
    if (d == 64) return launch_prefill_d<64>(q, k, v, cu, num_seqs, max_seqlen, nq, nkv, scale, out, lse, stream);
    return launch_prefill_d<128>(q, k, v, cu, num_seqs, max_seqlen, nq, nkv, scale, out, lse, stream);
}

}  // namespace bga
