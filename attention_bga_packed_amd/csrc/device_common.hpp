// Device-side helpers shared by the HIP kernels of libbga (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// work-item and workgroup ids straight from the hardware registers (the
// blockIdx / threadIdx wrappers can end up as out-of-line library calls)
__device__ __forceinline__ int thread_id() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_workitem_id_x() & 63; }
__device__ __forceinline__ int group_id_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int group_id_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16x2 bits, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l & 31), B column (l & 31); k slots (l >> 5) * 8 + [0, 8).
// C/D: lane l holds column (l & 31), rows (r / 4) * 8 + (l >> 5) * 4 + (r % 4), r in [0, 16).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ double wave_sum_f64(double x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        uint32_t y = __shfl_xor(x, o);
        x = x > y ? x : y;
    }
    return x;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

}  // namespace bga
