// Device-side precondition checks of the debug build (compiled with BGA_DEBUG).
//
// The release entry points trust what only the device can see: a valid
// cu_seqlens, parent indices inside the beam range, finite logits. In a debug
// build every entry point first runs the matching check kernel here on the
// caller's stream, waits for it and reads the device violation word; when a
// check failed the entry point returns BGA_ERR_PRECONDITION and does not launch
// the operation's kernels. Every check kernel reads only inside the extents
// the host validated and always runs to its end.
#include "bga.h"
#include "device_common.hpp"
#include "internal.hpp"

#ifdef BGA_DEBUG

#include <mutex>

namespace bga {

// One violation word per device; bits are BGA_VIOLATION_*.
__device__ __align__(256) uint32_t g_violation_word;

namespace {

__device__ __forceinline__ void flag(bool bad, uint32_t bit)
{
    // one atomic per wave that saw a violation
    if (__any(bad) && lane_id() == 0) atomicOr(&g_violation_word, bit);
}

__global__ void clear_word_kernel(uint32_t *w) { *w = 0u; }

// cu[0] == 0, cu non-decreasing, cu[B] == T, every length <= max_seqlen (and
// >= 1 when need_nonempty)
__global__ __launch_bounds__(256) void check_cu_seqlens_kernel(const int32_t *__restrict__ cu, int B, int T,
                                                               int max_seqlen, bool need_nonempty)
{
    for (int i0 = blockIdx.x * 256; i0 <= B; i0 += gridDim.x * 256) {
        const int i = i0 + (int)threadIdx.x;
        bool bad_cu = false, bad_len = false, empty = false;
        if (i <= B) {
            const int c = cu[i];
            if (i == 0) bad_cu |= c != 0;
            if (i == B) bad_cu |= c != T;
            if (i < B) {
                const int n = cu[i + 1] - c;
                bad_cu |= n < 0;
                bad_len |= n > max_seqlen;
                empty = need_nonempty && n == 0;
            }
        }
        flag(bad_cu, BGA_VIOLATION_CU_SEQLENS);
        flag(bad_len, BGA_VIOLATION_MAX_SEQLEN);
        flag(empty, BGA_VIOLATION_NO_KEYS);
    }
}

__global__ __launch_bounds__(256) void check_parents_kernel(const int32_t *__restrict__ parent, int n, int W)
{
    for (int i0 = blockIdx.x * 256; i0 < n; i0 += gridDim.x * 256) {
        const int i = i0 + (int)threadIdx.x;
        bool bad = false;
        if (i < n) {
            const int p = parent[i];
            bad = p < 0 || p >= W;
        }
        flag(bad, BGA_VIOLATION_PARENT);
    }
}

// a bf16 value is not finite when its exponent bits are all ones
__global__ __launch_bounds__(256) void check_logits_kernel(const uint16_t *__restrict__ x, size_t n)
{
    const size_t stride = (size_t)gridDim.x * 256;
    bool bad = false;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) bad |= (x[i] & 0x7f80u) == 0x7f80u;
    flag(bad, BGA_VIOLATION_LOGITS);
}

std::mutex g_mu;
uint32_t *g_word_ptr[64];   // device address of g_violation_word per device id

hipError_t word_address(uint32_t **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_word_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_violation_word));
        if (e != hipSuccess) return e;
        g_word_ptr[dev] = (uint32_t *)p;
    }
    *out = g_word_ptr[dev];
    return hipSuccess;
}

// Clear the word, run `launch_check(word)` on the stream, wait, read the word.
template <typename F>
hipError_t run_check(hipStream_t stream, uint32_t *violations, F launch_check)
{
    uint32_t *w = nullptr;
    hipError_t e = word_address(&w);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, stream, w);
    launch_check();
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint32_t host = 0;
    if ((e = hipMemcpyAsync(&host, w, sizeof host, hipMemcpyDeviceToHost, stream)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
    *violations = host;
    return hipSuccess;
}

int grid_for(size_t n) { return (int)std::min<size_t>((n + 255) / 256 + 1, 4096); }

}  // namespace

hipError_t debug_check_prefill(const int32_t *cu, int B, int T, int max_seqlen, hipStream_t stream,
                               uint32_t *violations)
{
    return run_check(stream, violations, [&] {
        hipLaunchKernelGGL(check_cu_seqlens_kernel, dim3(grid_for((size_t)B + 1)), dim3(256), 0, stream, cu, B, T,
                           max_seqlen, false);
    });
}

hipError_t debug_check_prompts(const int32_t *cu, int R, int T, int max_len, bool need_nonempty, hipStream_t stream,
                               uint32_t *violations)
{
    return run_check(stream, violations, [&] {
        hipLaunchKernelGGL(check_cu_seqlens_kernel, dim3(grid_for((size_t)R + 1)), dim3(256), 0, stream, cu, R, T,
                           max_len, need_nonempty);
    });
}

hipError_t debug_check_parents(const int32_t *parent, int n, int W, hipStream_t stream, uint32_t *violations)
{
    return run_check(stream, violations, [&] {
        hipLaunchKernelGGL(check_parents_kernel, dim3(grid_for((size_t)n)), dim3(256), 0, stream, parent, n, W);
    });
}

hipError_t debug_check_logits(const uint16_t *x, size_t n, hipStream_t stream, uint32_t *violations)
{
    return run_check(stream, violations, [&] {
        hipLaunchKernelGGL(check_logits_kernel, dim3(grid_for(n)), dim3(256), 0, stream, x, n);
    });
}

}  // namespace bga

#endif  // BGA_DEBUG
