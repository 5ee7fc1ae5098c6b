// Fused SwiGLU requantisation to FP8 E4M3 for gfx950.
//
// Article section 3.4 (selective FP8 for the dense matrix paths): after the
// FP8 Gate/Up projection, one pass per token computes SiLU(gate) * up in fp32,
// the row's largest magnitude, the per-token dynamic scale and the E4M3 codes
// that the FP8 Down projection reads, without writing the bf16 SwiGLU
// intermediate anywhere.
//
// One workgroup (256 threads) per token row: every thread loads its 16-byte
// chunks of gate and up (8 bf16 each; consecutive lanes take consecutive chunks,
// so each wave reads 1 KB runs), keeps h = gate * up / (1 + e^-gate) in
// registers (I / 256 values per thread), the block finds the row's amax (wave
// max, then across the four waves through LDS), and the same registers are
// scaled by 448 / amax and converted two at a time with the hardware's OCP
// E4M3 conversion (round to nearest even), 8 codes per 8-byte store. The row
// is read from HBM once and the codes written once.
#include "device_common.hpp"
#include "internal.hpp"

namespace bga {

constexpr int SQ_THREADS = 256;
constexpr float kE4M3Max = 448.f;
constexpr float kAmaxFloor = 1e-12f;

template <int NCH>   // 16-byte chunks of gate (and of up) per thread
__global__ __launch_bounds__(SQ_THREADS) void swiglu_quant_kernel(const u32x4 *__restrict__ gu, int I,
                                                                  u32x2 *__restrict__ codes,
                                                                  float *__restrict__ scale)
{
    __shared__ float wmax[SQ_THREADS / 64];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nch = I / 8;                                   // chunks per half row
    const u32x4 *gate = gu + (size_t)t * 2 * nch;
    const u32x4 *up = gate + nch;
    u32x4 g[NCH], u[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int c = k * SQ_THREADS + tid;
        const bool ok = c < nch;
        // read once: non-temporal
        g[k] = ok ? __builtin_nontemporal_load(gate + c) : u32x4{0u, 0u, 0u, 0u};
        u[k] = ok ? __builtin_nontemporal_load(up + c) : u32x4{0u, 0u, 0u, 0u};
    }
    float h[NCH][8];
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float g0 = bf16_lo(g[k][e]), g1 = bf16_hi(g[k][e]);
            const float u0 = bf16_lo(u[k][e]), u1 = bf16_hi(u[k][e]);
            // SiLU(x) = x / (1 + e^-x), fp32
            const float s0 = g0 * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-g0 * kLog2e));
            const float s1 = g1 * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-g1 * kLog2e));
            h[k][2 * e] = s0 * u0;
            h[k][2 * e + 1] = s1 * u1;
            amax = fmaxf(amax, fmaxf(fabsf(h[k][2 * e]), fabsf(h[k][2 * e + 1])));
        }
    amax = wave_max(amax);
    if (lane == 0) wmax[w] = amax;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < SQ_THREADS / 64; ++i) amax = fmaxf(amax, wmax[i]);
    const float a = fmaxf(amax, kAmaxFloor);
    const float inv = kE4M3Max / a;                          // codes = E4M3(h * 448 / amax)
    if (tid == 0) scale[t] = a / kE4M3Max;
    u32x2 *out = codes + (size_t)t * nch;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int c = k * SQ_THREADS + tid;
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(h[k][0] * inv, h[k][1] * inv, 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(h[k][2] * inv, h[k][3] * inv, lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(h[k][4] * inv, h[k][5] * inv, 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(h[k][6] * inv, h[k][7] * inv, hi, true);
        if (c < nch) out[c] = u32x2{(uint32_t)lo, (uint32_t)hi};
    }
}

// up to 8 chunks of 8 values per thread
int swiglu_quant_max_inter() { return 8 * SQ_THREADS * 8; }

hipError_t launch_swiglu_quant(const uint16_t *gate_up, int T, int I, uint8_t *codes, float *scale,
                               hipStream_t stream)
{
    const int nch = I / 8;
    const int per = (nch + SQ_THREADS - 1) / SQ_THREADS;   // chunks per thread
    dim3 grid(T), block(SQ_THREADS);
    const u32x4 *src = (const u32x4 *)gate_up;
    u32x2 *dst = (u32x2 *)codes;
    if (per <= 1)
        hipLaunchKernelGGL(swiglu_quant_kernel<1>, grid, block, 0, stream, src, I, dst, scale);
    else if (per <= 2)
        hipLaunchKernelGGL(swiglu_quant_kernel<2>, grid, block, 0, stream, src, I, dst, scale);
    else if (per <= 4)
        hipLaunchKernelGGL(swiglu_quant_kernel<4>, grid, block, 0, stream, src, I, dst, scale);
    else
        hipLaunchKernelGGL(swiglu_quant_kernel<8>, grid, block, 0, stream, src, I, dst, scale);
    return hipGetLastError();
}

}  // namespace bga
