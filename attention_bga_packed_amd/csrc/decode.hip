// Shared-prefix beam decode attention for gfx950.
//
// Article section 3.2 ("请求内共享前缀的 K/V 布局"): one prompt K/V per request
// [L_p, Nkv, D], a short suffix K/V per beam [W, L_s, Nkv, D], one query token
// per beam [W, Nq, D], and O_b = Attention(Q_b, [prefix_K; suffix_K[b]],
// [prefix_V; suffix_V[b]]) computed in a single fp32 online-softmax state
// without any concatenated tensor.
//
// The prefix segment is the dense part: for a (request, kv head) all W beams'
// G query heads form a [W*G, D] block (rows n = beam * G + head) that multiplies
// the same [L_p, D] prefix, so it runs on MFMA exactly like a prefill tile, with
// no mask except the ragged end of the prefix. A workgroup takes 128 of those
// query rows (4 waves x 32) and streams the prefix through LDS once; the prefix
// is therefore read from HBM once per (request, kv head) and from L2 by the
// other row blocks. The suffix segment is a handful of per-beam keys: each lane
// pair (lanes l and l^32, one query row) forms the dot products with its own
// beam's suffix keys from the d-halves it already holds and folds them into the
// same (m, l, O) state. Every row takes the same order (prefix, then suffix), so
// a row's result does not depend on which workgroup holds it.
//
// Grid = (R*Nkv, row blocks). Consecutive workgroups are dealt round-robin over
// the 8 XCDs, so with R*Nkv a multiple of 8 every row block of one
// (request, kv head) lands on the same XCD and shares its L2 copy of the prefix.
//
// Prompt layout. Either every request has a prompt of Lp tokens at
// [R, Lp, Nkv, D], or (prefix_cu given) the prompts are packed back to back,
// exactly as the packed prefill leaves its K/V: request r's prompt is rows
// prefix_cu[r] .. prefix_cu[r+1]-1 of [T_p, Nkv, D], each of its own length.
#include "attn_core.hpp"
#include "internal.hpp"

namespace bga {

using namespace core;

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void shared_prefix_decode_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ pk, const uint16_t *__restrict__ pv,
    const int32_t *__restrict__ pcu, const uint16_t *__restrict__ sk, const uint16_t *__restrict__ sv, int W,
    int Lp_uniform, int Ls, int Ls_cap, int nq, int nkv, int group, float scale, uint16_t *__restrict__ out,
    float *__restrict__ lse)
{
    using G = Geo<D>;
    constexpr int NW = 4;
    extern __shared__ __align__(16) uint16_t smem[];

    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    const int rg = group_id_x();
    const int r = uni(rg / nkv), g = rg - r * nkv;
    const int wave = uni(thread_id() >> 6);
    const int lane = lane_id(), col = lane & 31, half = lane >> 5;
    const int rows = W * group;
    const int wr0 = group_id_y() * 128 + wave * 32;
    const bool wave_active = wr0 < rows;

    // this lane's row (rows past the end duplicate the last row; not stored)
    const int n = min(wr0 + col, rows - 1);
    const int beam = n / group, h = n - beam * group;
    const size_t qrow = ((size_t)r * W + beam) * nq + (size_t)g * group + h;

    const uint32_t lds_base = (uint32_t)(size_t)(const BGA_LDS char *)smem;
    const uint32_t rbytes = (uint32_t)(nkv * D * 2);
    // this request's prompt: rows p0 .. p0 + Lp - 1 (wave-uniform scalar loads)
    const int p0 = pcu ? uni(pcu[r]) : r * Lp_uniform;
    const int Lp = pcu ? uni(pcu[r + 1]) - p0 : Lp_uniform;
    const size_t pofs = ((size_t)p0 * nkv + g) * D;
    const uint64_t kbase = uni64((uint64_t)(size_t)(pk + pofs));
    const uint64_t vbase = uni64((uint64_t)(size_t)(pv + pofs));
    const int nkt = (Lp + G::BN - 1) / G::BN;
    const int nkt_w = wave_active ? nkt : 0;

    Copier<D, NW> cp;
    cp.init(wave, rbytes);
    if (nkt > 0) first_copies<D, NW>(cp, lds_base, kbase, vbase, Lp, nkt);
    bf16x8 qop[D / 16];
    load_q<D>(qop, q + qrow * D);

    Reads<D> rd;
    rd.init(lds_base);
    Wave<D> st;
    st.reset();
    const float c2 = scale * kLog2e;
    wait_copies_and_sync();

    // Suffix rows. For one position j the suffix K (or V) rows of this
    // workgroup's beams lie a constant stride apart, so they are copied like a
    // key tile: global -> LDS with the copier, into the K/V slots (the K chunk
    // swizzle for both), up to 64 beams per slot. With at most 64 beams a
    // position takes one K and one V slot and two positions are in flight:
    // position 0 goes into the slots that the last prompt tile leaves idle,
    // during that tile; each later one is copied as soon as the position two
    // before it has been read. With more beams a position takes all four
    // slots and positions are copied one at a time.
    const int bfirst = uni(group_id_y() * 128 / group);
    const int nbeam = uni(min(group_id_y() * 128 + 127, rows - 1) / group) - bfirst + 1;   // 1 .. 128
    const int tp = nbeam > G::BN ? 2 : 1;   // 64-row slots per position (K, and as many for V)
    const uint32_t sstride = (uint32_t)(Ls_cap * nkv * D * 2);   // bytes from one beam's row to the next
    const uint32_t pos_bytes = (uint32_t)(nkv * D * 2);          // bytes from one position to the next
    const size_t sofs = (((size_t)r * W + bfirst) * Ls_cap * nkv + g) * D;
    const uint64_t skb = uni64((uint64_t)(size_t)(sk + sofs));
    const uint64_t svb = uni64((uint64_t)(size_t)(sv + sofs));
    Copier<D, NW> scp;
    scp.init(wave, sstride);
    auto issue_pos = [&](int j, int set) {   // position j into slot set `set` (tp == 1) or all slots
        for (int t = 0; t < tp; ++t) {
            const int nrow = min(G::BN, nbeam - t * G::BN);
            const uint64_t off = (uint64_t)j * pos_bytes + (uint64_t)t * G::BN * sstride;
            const int slot = tp == 1 ? set : t;
            scp.template issue<false>(lds_base + G::kslot(slot), skb + off, nrow < G::BN ? nrow - 1 : -1);
            scp.template issue<false>(lds_base + G::vslot(slot), svb + off, nrow < G::BN ? nrow - 1 : -1);
        }
    };
    // slot set of the last prompt tile's K/V; position 0 goes into the other one
    const int s0 = tp == 1 ? (nkt > 0 ? 1 - ((nkt - 1) & 1) : 0) : 0;
    const bool pos0_in_scan = tp == 1 && Ls > 0 && nkt > 0;
    auto extra = [&](int kt) {
        if (pos0_in_scan && kt == nkt - 1) issue_pos(0, s0);
    };

    // ---- prefix segment: MFMA tiles through LDS, shared by the 4 waves
    if (nkt > 0)
        scan<D, NW>(st, rd, cp, qop, lds_base, kbase, vbase, Lp, nkt, nkt_w, Lp - 1, Lp / G::BN, c2, true, extra);

    // ---- suffix segment: this beam's own keys, folded into the same state
    __syncthreads();   // every wave is done with the last prompt tile's slots
    if (Ls > 0 && !pos0_in_scan) issue_pos(0, s0);
    if (tp == 1 && Ls > 1) issue_pos(1, 1 - s0);
    constexpr int kPerPos = 2 * Copier<D, NW>::N;   // copies of one position per wave (tp == 1)
    static_assert(kPerPos < 16, "vmcnt immediate");
    const int brow = beam - bfirst, bt = brow >> 6, rt = brow & (G::BN - 1);
    const int sw = G::swk(rt);
    for (int j = 0; j < Ls; ++j) {
        const int set = (j & 1) ? 1 - s0 : s0;   // slot set of position j (tp == 1; wave-uniform)
        const int rset = tp == 1 ? set : bt;      // the slot this lane's beam row is in
        if (tp == 1 && j + 1 < Ls)
            __builtin_amdgcn_s_waitcnt(0x0f70 | kPerPos);   // position j landed (j + 1 may be in flight)
        else
            __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();
        if (wave_active) {
            const uint32_t kb = lds_base + G::kslot(rset) + (uint32_t)(rt * G::ROWB);
            const uint32_t vb = lds_base + G::vslot(rset) + (uint32_t)(rt * G::ROWB);
            u32x4 kx[D / 16];
            u32x2 vx[D / 32][4];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                kx[ks] = *(const BGA_LDS u32x4 *)(size_t)(kb + (uint32_t)(((ks * 2 + half) ^ sw) << 4));
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
#pragma unroll
                for (int rgi = 0; rgi < 4; ++rgi)
                    vx[b][rgi] =
                        *(const BGA_LDS u32x2 *)(size_t)(vb + (uint32_t)((((b * 4 + rgi) ^ sw) << 4) + half * 8));
            float part = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const u32x4 qv = __builtin_bit_cast(u32x4, qop[ks]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    part = __builtin_fmaf(bf16_lo(qv[e]), bf16_lo(kx[ks][e]), part);
                    part = __builtin_fmaf(bf16_hi(qv[e]), bf16_hi(kx[ks][e]), part);
                }
            }
            const float s = pair_sum(part);
            const float m_new = fmaxf(st.m, s);
            const float alpha = __builtin_amdgcn_exp2f((st.m - m_new) * c2);   // 0 while no key was seen (m = -inf)
            const float p = __builtin_amdgcn_exp2f((s - m_new) * c2);
            st.l = st.l * alpha + (half == 0 ? p : 0.f);
            st.ln = st.ln * alpha + (half == 0 ? p : 0.f);   // the suffix weights p exactly (fp32)
            st.m = m_new;
#pragma unroll
            for (int b = 0; b < D / 32; ++b)
#pragma unroll
                for (int rgi = 0; rgi < 4; ++rgi) {
                    const u32x2 vv = vx[b][rgi];
                    st.o[b][rgi * 4 + 0] = __builtin_fmaf(st.o[b][rgi * 4 + 0], alpha, p * bf16_lo(vv[0]));
                    st.o[b][rgi * 4 + 1] = __builtin_fmaf(st.o[b][rgi * 4 + 1], alpha, p * bf16_hi(vv[0]));
                    st.o[b][rgi * 4 + 2] = __builtin_fmaf(st.o[b][rgi * 4 + 2], alpha, p * bf16_lo(vv[1]));
                    st.o[b][rgi * 4 + 3] = __builtin_fmaf(st.o[b][rgi * 4 + 3], alpha, p * bf16_hi(vv[1]));
                }
        }
        if (j + 1 < Ls) {
            __syncthreads();   // every wave has read position j's slots
            if (tp == 1) {
                if (j + 2 < Ls) issue_pos(j + 2, set);
            } else {
                issue_pos(j + 1, 0);
            }
        }
    }
    __syncthreads();   // every wave is done with the prefix slots: they stage the output rows now
    if (wave_active)
        st.finish(out, (uint32_t)qrow, lse ? lse + qrow : nullptr, wr0 + col < rows, scale,
                  lds_base + (uint32_t)(wave * 32 * G::ROWB));
}

template <int D>
static hipError_t launch_decode_d(const uint16_t *q, const uint16_t *pk, const uint16_t *pv, const int32_t *pcu,
                                  const uint16_t *sk, const uint16_t *sv, int R, int W, int Lp, int Ls, int Ls_cap,
                                  int nq, int nkv, float scale, uint16_t *out, float *lse, hipStream_t stream)
{
    const int group = nq / nkv;
    const int rows = W * group;
    const size_t smem = Geo<D>::SMEM;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = dynamic_lds_once((const void *)shared_prefix_decode_kernel<D>, (int)smem, lds_set);
    if (e != hipSuccess) return e;
    dim3 grid(R * nkv, (rows + 127) / 128), block(256);
    hipLaunchKernelGGL(shared_prefix_decode_kernel<D>, grid, block, smem, stream, q, pk, pv, pcu, sk, sv, W, Lp,
                       Ls, Ls_cap, nq, nkv, group, scale, out, lse);
    return hipGetLastError();
}

hipError_t launch_shared_prefix_decode(const uint16_t *q, const uint16_t *pk, const uint16_t *pv,
                                       const int32_t *prefix_cu, const uint16_t *sk, const uint16_t *sv, int R,
                                       int W, int Lp, int Ls, int Ls_cap, int nq, int nkv, int d, float scale,
                                       uint16_t *out, float *lse, hipStream_t stream)
{
    if (d == 64)
        return launch_decode_d<64>(q, pk, pv, prefix_cu, sk, sv, R, W, Lp, Ls, Ls_cap, nq, nkv, scale, out, lse,
                                   stream);
    return launch_decode_d<128>(q, pk, pv, prefix_cu, sk, sv, R, W, Lp, Ls, Ls_cap, nq, nkv, scale, out, lse,
                                stream);
}

}  // namespace bga
