// Last valid token of every packed sequence, for gfx950.
//
// Article section 3.1: after packed attention the model takes, through the same
// sequence boundary, each sequence's last-position hidden state (the input of
// the per-sample score or label head). Row i of dst is row cu[i+1]-1 of src; a
// zero-length sequence has no last token and gets a row of zeros.
//
// A workgroup copies one 16 KB piece of one row (256 lanes x 4 chunks of 16
// bytes); grid = (sequences, pieces per row). The source row index is clamped to
// [0, T) so that even a corrupt cu_seqlens never reads outside src.
#include "device_common.hpp"
#include "internal.hpp"

namespace bga {

__global__ __launch_bounds__(256) void last_token_gather_kernel(const u32x4 *__restrict__ src,
                                                                const int32_t *__restrict__ cu, int T,
                                                                int64_t row16, u32x4 *__restrict__ dst)
{
    const int i = blockIdx.x;
    const int start = cu[i], end = cu[i + 1];
    const bool empty = end <= start;
    const int64_t last = min(max(end - 1, 0), T - 1);
    const u32x4 *s = src + last * row16;
    u32x4 *d = dst + (int64_t)i * row16;
    constexpr int U = 4;
    const int64_t base = (int64_t)blockIdx.y * (U * 256) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = base + u * 256;
        v[u] = (!empty && c < row16) ? s[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t c = base + u * 256;
        if (c < row16) d[c] = v[u];
    }
}

hipError_t launch_last_token_gather(const void *src, const int32_t *cu, int num_seqs, int T, int64_t row_bytes,
                                    void *dst, hipStream_t stream)
{
    const int64_t row16 = row_bytes / 16;
    const int64_t pieces = (row16 + 1023) / 1024;
    dim3 grid((unsigned)num_seqs, (unsigned)pieces), block(256);
    hipLaunchKernelGGL(last_token_gather_kernel, grid, block, 0, stream, (const u32x4 *)src, cu, T, row16,
                       (u32x4 *)dst);
    return hipGetLastError();
}

}  // namespace bga
