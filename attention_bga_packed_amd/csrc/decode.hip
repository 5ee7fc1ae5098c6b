// Shared-prefix beam decode attention for gfx950.
//
// Article section 3.2 ("请求内共享前缀的 K/V 布局"): one prompt K/V per request
// [L_p, Nkv, D], a short suffix K/V per beam [W, L_s, Nkv, D], one query token
// per beam [W, Nq, D], and O_b = Attention(Q_b, [prefix_K; suffix_K[b]],
// [prefix_V; suffix_V[b]]) computed in a single fp32 online-softmax state
// without any concatenated tensor.
//
// The prefix segment is the dense part: for a (request, kv head) all W beams'
// G query heads form a [W*G, D] block that multiplies the same [L_p, D] prefix,
// so it runs on MFMA exactly like a prefill tile (no mask except the ragged end
// of the prefix). A workgroup takes 128 of those query rows (4 waves x 32) and
// streams the prefix through LDS once; the prefix is therefore read from HBM
// once per (request, kv head) and from L2 by the other row blocks. The suffix
// segment is a handful of per-beam keys: each lane pair (lanes l and l^32, one
// query row) forms the dot products with its own beam's suffix keys from the
// d-halves it already holds and folds them into the same (m, l, O) state.
//
// Grid = (R*Nkv, row blocks). Consecutive workgroups are dealt round-robin over
// the 8 XCDs, so with R*Nkv a multiple of 8 every row block of one
// (request, kv head) lands on the same XCD and shares its L2 copy of the prefix.
#include "attn_tile.hpp"
#include "internal.hpp"

namespace bga {

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void shared_prefix_decode_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ pk, const uint16_t *__restrict__ pv,
    const uint16_t *__restrict__ sk, const uint16_t *__restrict__ sv, int W, int Lp, int Ls, int Ls_cap, int nq,
    int nkv, int group, float scale, uint16_t *__restrict__ out, float *__restrict__ lse)
{
    using T = AttnTile<D>;
    extern __shared__ __align__(16) uint16_t smem[];

    const int rg = blockIdx.x;
    const int r = rg / nkv, g = rg % nkv;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int w = tid >> 6;
    const int rows = W * group;
    const bool wave_active = blockIdx.y * 128 + w * 32 < rows;

    // query row within (r, g): beam * G + head-in-group
    auto query_row = [&](bool &valid, int &beam) {
        const int n = blockIdx.y * 128 + w * 32 + (threadIdx.x & 31);
        valid = n < rows;
        beam = valid ? n / group : 0;
        const int head = g * group + (valid ? n % group : 0);
        return ((size_t)r * W + beam) * nq + head;
    };

    bf16x8 qop[D / 16];
    {
        bool valid;
        int beam;
        const size_t qi = query_row(valid, beam);
        load_q_operand<D>(qop, q + qi * D, valid);
    }

    const BGA_LDS char *lds = lds_ptr(smem);
    const uint32_t lds_base = lds_addr(lds);
    WaveAttn<D> st;
    st.init(lds);
    const float c2 = scale * kLog2e;

    // the row's indices (recomputed where needed: fewer registers live across the scan)
    const int half = (threadIdx.x & 63) >> 5;

    // ---- suffix segment: this beam's own keys, folded into the same state
    // (invalid query rows read beam 0's rows, which exist, and are dropped at the end)
    struct SuffixKey {
        u32x4 k[D / 16];      // K row: this lane's d-half of every 16-wide d step
        u32x2 v[D / 32][4];   // V row: the d values this lane accumulates
    };
    auto suffix = [&]() {   // after the prefix scan (its registers are free by then)
        bool valid;
        int beam;
        query_row(valid, beam);
        const size_t sbase = (((size_t)r * W + beam) * Ls_cap * nkv + g) * D;
        const uint32_t rs = (uint32_t)(nkv * D);
        for (int j = 0; j < Ls; ++j) {
            SuffixKey x;
            const uint16_t *kr = sk + sbase + (size_t)j * rs, *vr = sv + sbase + (size_t)j * rs;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) x.k[ks] = *(const u32x4 *)(kr + ks * 16 + half * 8);
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
#pragma unroll
                for (int rgi = 0; rgi < 4; ++rgi) x.v[b][rgi] = *(const u32x2 *)(vr + b * 32 + rgi * 8 + half * 4);
            float part = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const u32x4 qv = __builtin_bit_cast(u32x4, qop[ks]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    part = __builtin_fmaf(bf16_lo(qv[e]), bf16_lo(x.k[ks][e]), part);
                    part = __builtin_fmaf(bf16_hi(qv[e]), bf16_hi(x.k[ks][e]), part);
                }
            }
            const float s = pair_sum(part);
            const float m_new = fmaxf(st.m, s);
            const float alpha = __builtin_amdgcn_exp2f((st.m - m_new) * c2);   // 0 on the first key (m = -inf)
            const float p = __builtin_amdgcn_exp2f((s - m_new) * c2);
            st.l = st.l * alpha + (half == 0 ? p : 0.f);
            st.m = m_new;
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
#pragma unroll
                for (int rgi = 0; rgi < 4; ++rgi) {
                    const u32x2 vv = x.v[b][rgi];
                    st.o[b][rgi * 4 + 0] = __builtin_fmaf(st.o[b][rgi * 4 + 0], alpha, p * bf16_lo(vv[0]));
                    st.o[b][rgi * 4 + 1] = __builtin_fmaf(st.o[b][rgi * 4 + 1], alpha, p * bf16_hi(vv[0]));
                    st.o[b][rgi * 4 + 2] = __builtin_fmaf(st.o[b][rgi * 4 + 2], alpha, p * bf16_lo(vv[1]));
                    st.o[b][rgi * 4 + 3] = __builtin_fmaf(st.o[b][rgi * 4 + 3], alpha, p * bf16_hi(vv[1]));
                }
        }
    };

    // ---- prefix segment: MFMA tiles through LDS, shared by the 4 waves
    const uint32_t row_stride = (uint32_t)(nkv * D);
    DmaPlan<D, 4> plan;   // 4 waves per workgroup
    plan.init(w, nthr >> 6);
    const size_t pbase = (size_t)r * Lp * row_stride + (size_t)g * D;
    const int nkt = (Lp + AttnTile<D>::BN - 1) / AttnTile<D>::BN;
    attn_scan<D>(st, plan, lds_base, qop, pk + pbase, pv + pbase, row_stride, 0, Lp, nkt, c2,
                 [&](int kt) { return (kt + 1) * AttnTile<D>::BN > Lp; }, Lp - 1);
    if (!wave_active) return;
    suffix();
    bool row_valid;
    int beam;
    const size_t qrow_idx = query_row(row_valid, beam);
    st.finish(out + qrow_idx * D, lse ? lse + qrow_idx : nullptr, row_valid, scale);
}

template <int D>
static hipError_t launch_decode_d(const uint16_t *q, const uint16_t *pk, const uint16_t *pv, const uint16_t *sk,
                                  const uint16_t *sv, int R, int W, int Lp, int Ls, int Ls_cap, int nq, int nkv,
                                  float scale, uint16_t *out, float *lse, hipStream_t stream)
{
    const int group = nq / nkv;
    const int rows = W * group;
    const size_t smem = AttnTile<D>::SMEM_BYTES;
    hipError_t e = hipFuncSetAttribute((const void *)shared_prefix_decode_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    dim3 grid(R * nkv, (rows + 127) / 128), block(256);
    hipLaunchKernelGGL(shared_prefix_decode_kernel<D>, grid, block, smem, stream, q, pk, pv, sk, sv, W, Lp, Ls,
                       Ls_cap, nq, nkv, group, scale, out, lse);
    return hipGetLastError();
}

hipError_t launch_shared_prefix_decode(const uint16_t *q, const uint16_t *pk, const uint16_t *pv,
                                       const uint16_t *sk, const uint16_t *sv, int R, int W, int Lp, int Ls,
                                       int Ls_cap, int nq, int nkv, int d, float scale, uint16_t *out, float *lse,
                                       hipStream_t stream)
{
    if (d == 64)
        return launch_decode_d<64>(q, pk, pv, sk, sv, R, W, Lp, Ls, Ls_cap, nq, nkv, scale, out, lse, stream);
    return launch_decode_d<128>(q, pk, pv, sk, sv, R, W, Lp, Ls, Ls_cap, nq, nkv, scale, out, lse, stream);
}

}  // namespace bga
