// Parent-index reorder of the per-beam state for gfx950.
//
// Article sections 3.2 and 3.3: once the global candidates are chosen, new beam
// b continues the hypothesis of beam parent[b]; only the short suffix K/V and
// the generated-token history are gathered (the shared prompt K/V never moves,
// and eliminated candidates are never copied).
//
// For fixed (request, beam) the first L_s suffix positions of K (and of V) are
// one contiguous run of L_s*Nkv*D bf16, so a workgroup per destination beam
// copies two runs with 16-byte vector loads and stores, plus the token run.
#include "device_common.hpp"
#include "internal.hpp"

namespace bga {

__global__ __launch_bounds__(256) void suffix_reorder_kernel(
    const uint16_t *__restrict__ src_k, const uint16_t *__restrict__ src_v, uint16_t *__restrict__ dst_k,
    uint16_t *__restrict__ dst_v, const int32_t *__restrict__ parent, const int32_t *__restrict__ src_tok,
    int32_t *__restrict__ dst_tok, int W, int run16, size_t beam_stride, int ntok, int tok_cap)
{
    const int rb = blockIdx.x;            // r * W + b
    const int r = rb / W;
    const int p = parent[rb];
    const bool ok = p >= 0 && p < W;
    const size_t src_off = ((size_t)r * W + (ok ? p : 0)) * beam_stride;
    const size_t dst_off = (size_t)rb * beam_stride;
    const u32x4 *sk = (const u32x4 *)(src_k + src_off);
    const u32x4 *svv = (const u32x4 *)(src_v + src_off);
    u32x4 *dk = (u32x4 *)(dst_k + dst_off);
    u32x4 *dv = (u32x4 *)(dst_v + dst_off);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // up to 4 chunks of K and of V per thread in flight before any store
    constexpr int U = 4;
    for (int i0 = 0; i0 < run16; i0 += U * 256) {
        u32x4 a[U], b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * 256 + (int)threadIdx.x;
            a[u] = zero;
            b[u] = zero;
            if (ok && i < run16) {
                a[u] = sk[i];
                b[u] = svv[i];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * 256 + (int)threadIdx.x;
            if (i < run16) {   // non-temporal: the next step reads them once, in another kernel
                __builtin_nontemporal_store(a[u], dk + i);
                __builtin_nontemporal_store(b[u], dv + i);
            }
        }
    }
    if (src_tok) {
        const int32_t *st = src_tok + ((size_t)r * W + (ok ? p : 0)) * tok_cap;
        int32_t *dt = dst_tok + (size_t)rb * tok_cap;
        for (int i = threadIdx.x; i < ntok; i += blockDim.x) dt[i] = ok ? st[i] : 0;
    }
}

hipError_t launch_suffix_reorder(const uint16_t *src_k, const uint16_t *src_v, uint16_t *dst_k, uint16_t *dst_v,
                                 const int32_t *parent, const int32_t *src_tok, int32_t *dst_tok, int R, int W,
                                 int Ls, int Ls_cap, int nkv, int d, int ntok, int tok_cap, hipStream_t stream)
{
    const size_t beam_stride = (size_t)Ls_cap * nkv * d;   // elements
    const int run16 = (int)((size_t)Ls * nkv * d / 8);     // 16-byte chunks per beam
    dim3 grid(R * W), block(256);
    hipLaunchKernelGGL(suffix_reorder_kernel, grid, block, 0, stream, src_k, src_v, dst_k, dst_v, parent, src_tok,
                       dst_tok, W, run16, beam_stride, ntok, tok_cap);
    return hipGetLastError();
}

}  // namespace bga
