// Packed variable-length causal GQA prefill for gfx950.
//
// Article section 3.1 ("变长样本的 Packed Prefill"): sequences are packed back to
// back as Q [T, Nq, D], K/V [T, Nkv, D]; the sequence boundary (cu_seqlens)
// implies a block-diagonal causal mask; the kernel never expands GQA K/V heads
// and never materialises the score matrix; for each query block it derives the
// valid K/V range from the boundary and scans it blockwise with an fp32 online
// softmax.
//
// Rows. For a (sequence, kv head g) the query rows are the pairs (token t,
// head h of the group), n = t * G + h, t < L. A workgroup of NW waves takes
// 32 * NW consecutive rows; every wave takes 32 of them. All G heads of a token
// sit in the same block, so one K/V tile staged in LDS serves the whole group,
// and a block is full whatever G is (no idle head slots).
//
// Keys. The workgroup scans the sequence's keys from its first token up to its
// last row's token, 64 at a time. A wave computes only the tiles up to its own
// last row's token (it still takes part in the copies and barriers of the
// later ones) and masks only the tiles that reach past its first row's token.
//
// Grid = (pairs rounded up to a multiple of 8, row blocks). Pair = (sequence,
// kv head). Dispatch order over the row blocks: block 0 (one key tile, the
// shortest) first, then the rest longest first. When the grid exceeds what the
// GPU holds at once, the block-0 workgroups finish early and free their slots
// for the overflow, and the long blocks start at once. Consecutive workgroups
// are dealt round-robin over the 8 XCDs, so the pair index in x, padded to a
// multiple of 8, keeps every block of one (sequence, kv head) on one XCD and
// its L2.
#include "attn_core.hpp"
#include "internal.hpp"

namespace bga {

using namespace core;

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2))) void packed_prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ cu, int num_pairs, int blocks_y, int nq, int nkv, int group, float scale,
    uint16_t *__restrict__ out, float *__restrict__ lse)
{
    using G = Geo<D>;
    constexpr int ROWS = 32 * NW;
    extern __shared__ __align__(16) uint16_t smem[];

    const int pair = group_id_x();
    if (pair >= num_pairs) return;
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    const int seq = uni(pair / nkv), g = pair - seq * nkv;
    const int s0 = cu[seq];
    const int nrows = (cu[seq + 1] - s0) * group;
    // row block of this workgroup: y = 0 -> block 0, y = 1 .. -> blocks_y - 1 down to 1
    const int y = group_id_y();
    const int blk = y == 0 ? 0 : blocks_y - y;
    const int n0 = blk * ROWS;
    if (n0 >= nrows) return;   // uniform over the workgroup

    const int wave = uni(thread_id() >> 6);
    const int lane = lane_id(), col = lane & 31;
    const uint32_t lds_base = (uint32_t)(size_t)(const BGA_LDS char *)smem;
    const uint32_t rbytes = (uint32_t)(nkv * D * 2);
    const uint64_t kbase = uni64((uint64_t)(size_t)(k + ((size_t)s0 * nkv + g) * D));
    const uint64_t vbase = uni64((uint64_t)(size_t)(v + ((size_t)s0 * nkv + g) * D));
    const float c2 = scale * kLog2e;
    Copier<D, NW> cp;
    cp.init(wave, rbytes);
    Reads<D> rd;
    rd.init(lds_base);

    // Rows [n0, n0 + ROWS) of the sequence. Wave-uniform values come from
    // integer division on the vector ALU, so they are read back from the first
    // lane to keep the control flow scalar.
    // keys [0, kend) of the sequence; tiles [0, nkt)
    const int kend = uni((min(n0 + ROWS, nrows) - 1) / group + 1);
    const int nkt = uni((kend + G::BN - 1) / G::BN);
    // this wave: rows [wr0, wr_last], tiles [0, nkt_w), masked from tile kt_mask on
    const int wr0 = n0 + wave * 32;
    const int wr_last = min(wr0 + 31, nrows - 1);
    const int nkt_w = uni(wr0 < nrows ? (wr_last / group) / G::BN + 1 : 0);
    const int kt_mask = uni((wr0 / group + 1) / G::BN);
    // this lane's row (rows past the end duplicate the last row; not stored)
    const int n = min(wr0 + col, nrows - 1);
    const int tok = n / group, h = n - tok * group;
    const size_t qrow = ((size_t)(s0 + tok) * nq + (size_t)g * group + h);

    first_copies<D, NW>(cp, lds_base, kbase, vbase, kend, nkt);
    bf16x8 qop[D / 16];
    load_q<D>(qop, q + qrow * D);
    wait_copies_and_sync();
    Wave<D> st;
    st.reset();
    scan<D, NW>(st, rd, cp, qop, lds_base, kbase, vbase, kend, nkt, nkt_w, tok, kt_mask, c2, true);
    __syncthreads();   // every wave is done with the K/V slots: they stage the output rows now
    if (nkt_w > 0)
        st.finish(out, (uint32_t)qrow, lse ? lse + qrow : nullptr, wr0 + col < nrows, scale,
                  lds_base + (uint32_t)(wave * 32 * G::ROWB));
}

template <int D, int NW>
static hipError_t launch_prefill_d(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *cu,
                                   int num_seqs, int max_seqlen, int nq, int nkv, float scale, uint16_t *out,
                                   float *lse, hipStream_t stream)
{
    const int group = nq / nkv;
    const int pairs = num_seqs * nkv;
    const int xdim = (pairs + 7) / 8 * 8;
    const int blocks_y = (int)(((int64_t)max_seqlen * group + 32 * NW - 1) / (32 * NW));
    const size_t smem = Geo<D>::SMEM;
    const void *kern = (const void *)packed_prefill_kernel<D, NW>;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    dim3 grid(xdim, blocks_y), block(64 * NW);
    hipLaunchKernelGGL((packed_prefill_kernel<D, NW>), grid, block, smem, stream, q, k, v, cu, pairs, blocks_y, nq,
                       nkv, group, scale, out, lse);
    return hipGetLastError();
}

hipError_t launch_packed_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *cu,
                                 int num_seqs, int max_seqlen, int nq, int nkv, int d, float scale, uint16_t *out,
                                 float *lse, hipStream_t stream)
{
    if (d == 64) return launch_prefill_d<64, 4>(q, k, v, cu, num_seqs, max_seqlen, nq, nkv, scale, out, lse, stream);
    return launch_prefill_d<128, 4>(q, k, v, cu, num_seqs, max_seqlen, nq, nkv, scale, out, lse, stream);
}

}  // namespace bga
