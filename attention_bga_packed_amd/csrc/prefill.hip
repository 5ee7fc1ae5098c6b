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
// kv head). The row-block index is reversed, so the longest (last) blocks of
// every sequence are dispatched first. Consecutive workgroups are dealt
// round-robin over the 8 XCDs, so the pair index in x, padded to a multiple of
// 8, keeps every block of one (sequence, kv head) on one XCD and its L2.
#include <type_traits>

#include "attn_core.hpp"
#include "internal.hpp"

namespace bga {

using namespace core;

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2))) void packed_prefill_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ cu, int num_pairs, int nq, int nkv, int group, float scale,
    uint16_t *__restrict__ out, float *__restrict__ lse)
{
    using G = Geo<D>;
    constexpr int ROWS = 32 * NW;
    extern __shared__ __align__(16) uint16_t smem[];

    const int pair = blockIdx.x;
    if (pair >= num_pairs) return;
    const int seq = __builtin_amdgcn_readfirstlane(pair / nkv), g = pair - seq * nkv;
    const int s0 = cu[seq];
    const int nrows = (cu[seq + 1] - s0) * group;
    const int n0 = (gridDim.y - 1 - blockIdx.y) * ROWS;
    if (n0 >= nrows) return;   // uniform over the workgroup

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63, col = lane & 31;

    // Wave-uniform values: integer division runs on the vector ALU, so the
    // quotients are read back from the first lane to keep the control flow scalar.
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
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

    bf16x8 qop[D / 16];
    const uint32_t lds_base = (uint32_t)(size_t)(const BGA_LDS char *)smem;
    const uint32_t rbytes = (uint32_t)(nkv * D * 2);
    const uint64_t kbase = uni64((uint64_t)(size_t)(k + ((size_t)s0 * nkv + g) * D));
    const uint64_t vbase = uni64((uint64_t)(size_t)(v + ((size_t)s0 * nkv + g) * D));
    const uint64_t tile_bytes = (uint64_t)G::BN * rbytes;
    auto last_row = [&](int kt) { return kt * G::BN + G::BN > kend ? kend - 1 - kt * G::BN : -1; };

    Copier<D, NW> cp;
    cp.init(wave, rbytes);
    cp.template issue<false>(lds_base + G::kslot(0), kbase, last_row(0));
    cp.template issue<true>(lds_base + G::vslot(0), vbase, last_row(0));
    load_q<D>(qop, q + qrow * D);

    Reads<D> rd;
    rd.init(lds_base);
    Wave<D> st;
    st.reset();
    const float c2 = scale * kLog2e;

    wait_copies_and_sync();
    if (nkt > 1) cp.template issue<false>(lds_base + G::kslot(1), kbase + tile_bytes, last_row(1));

    f32x16 sa[2], sb[2];
    if (nkt_w > 0) {
        Wave<D>::scores(rd, qop, G::kslot(0), sa);
        if (kt_mask == 0) Wave<D>::mask(sa, tok);
        st.m = Wave<D>::rowmax(sa);
        st.mc = st.m * c2;
    }

    // Tile kt: K(kt) and V(kt) sit in slot kt & 1. Every tile starts with a
    // barrier after which K(kt+2) and V(kt+1) are copied into the slots that
    // K(kt) and V(kt-1) held.
    auto sync_and_copy = [&](int kt) {
        wait_copies_and_sync();   // K(kt+1), V(kt) landed; K(kt), V(kt-1) no longer read
        const uint32_t p = (uint32_t)(kt & 1);
        if (kt + 2 < nkt)
            cp.template issue<false>(lds_base + p * G::KBYTES, kbase + (uint64_t)(kt + 2) * tile_bytes,
                                     last_row(kt + 2));
        if (kt + 1 < nkt)
            cp.template issue<true>(lds_base + G::vslot(0) + (1 - p) * G::KBYTES,
                                    vbase + (uint64_t)(kt + 1) * tile_bytes, last_row(kt + 1));
    };
    // all but the wave's last tile: exponentials and P*V of tile kt, scores of kt+1
    auto step = [&](int kt, auto parity, f32x16(&sc)[2], f32x16(&sn)[2]) {
        constexpr int P = decltype(parity)::value;
        sync_and_copy(kt);
        float mx = st.step(rd, qop, sc, sn, G::kslot(1 - P), G::vslot(P), c2);
        if (kt + 1 >= kt_mask) {   // the next tile reaches past this wave's first row
            Wave<D>::mask(sn, tok - (kt + 1) * G::BN);
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

    if (nkt_w == 0) return;
    st.finish(out + qrow * D, lse ? lse + qrow : nullptr, wr0 + col < nrows, scale);
}

template <int D, int NW>
static hipError_t launch_prefill_d(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *cu,
                                   int num_seqs, int max_seqlen, int nq, int nkv, float scale, uint16_t *out,
                                   float *lse, hipStream_t stream)
{
    const int group = nq / nkv;
    const int pairs = num_seqs * nkv;
    const int xdim = (pairs + 7) / 8 * 8;
    const int blocks = (int)(((int64_t)max_seqlen * group + 32 * NW - 1) / (32 * NW));
    const size_t smem = Geo<D>::SMEM;
    const void *kern = (const void *)packed_prefill_kernel<D, NW>;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    dim3 grid(xdim, blocks), block(64 * NW);
    hipLaunchKernelGGL((packed_prefill_kernel<D, NW>), grid, block, smem, stream, q, k, v, cu, pairs, nq, nkv, group,
                       scale, out, lse);
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
