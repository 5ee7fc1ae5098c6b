/*
 * Plain, slow, fp64 CPU oracle for the attention hot path of the
 * bounded-generation SLM engine ("SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化").
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. It shares no code, header,
 * table or helper with the HIP library; each side decodes bf16 on its own.
 *
 * Every function is the plain definition written out: no tiling, no online
 * rescaling, no fusion. Loops over independent units (sequence x head,
 * request x beam, beam row) are spread over OpenMP threads; each unit is
 * computed exactly as it would be serially.
 *
 * Inputs are raw bf16 bit patterns (uint16), widened exactly to double.
 * Return value: 0 on success, nonzero on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double widen(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float widen_f(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int pick_threads(int32_t n)
{
#ifdef _OPENMP
    return n > 0 ? n : omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

int32_t oracle_num_threads(int32_t requested) { return pick_threads(requested); }

/*
 * Softmax attention of one query over an explicit key/value list (article
 * section 3.1 for the prefill form, section 3.2 for the shared-prefix form):
 *   s_u = scale * <q, k_u>;  m = max_u s_u;  l = sum_u exp(s_u - m)
 *   o   = sum_u exp(s_u - m) * v_u / l;  lse = m + ln l
 * q has length d (double); keys/values are n rows of d doubles.
 */
static void attend(const double *q, const double *keys, const double *vals, int64_t n, int32_t d,
                   double scale, double *s, double *o, double *lse)
{
    double m = -INFINITY;
    for (int64_t u = 0; u < n; ++u) {
        double acc = 0.0;
        for (int32_t e = 0; e < d; ++e) acc += q[e] * keys[u * d + e];
        s[u] = scale * acc;
        if (s[u] > m) m = s[u];
    }
    double l = 0.0;
    for (int32_t e = 0; e < d; ++e) o[e] = 0.0;
    for (int64_t u = 0; u < n; ++u) {
        double p = exp(s[u] - m);
        l += p;
        for (int32_t e = 0; e < d; ++e) o[e] += p * vals[u * d + e];
    }
    for (int32_t e = 0; e < d; ++e) o[e] /= l;
    *lse = m + log(l);
}

/*
 * Packed variable-length causal GQA prefill (article section 3.1).
 * q [T, nq, d], k/v [T, nkv, d], cu_seqlens [num_seqs+1] (host).
 * Query position t of sequence i sees keys u of the same sequence with u <= t
 * ("not later than itself"). Query head h reads K/V head h / (nq/nkv).
 * out [T, nq, d] and lse [T, nq] are fp64.
 */
int32_t oracle_packed_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              const int32_t *cu_seqlens, int32_t num_seqs, int32_t nq, int32_t nkv,
                              int32_t d, double scale, double *out, double *lse, int32_t nthreads)
{
    if (!q || !k || !v || !cu_seqlens || !out || !lse) return 1;
    if (num_seqs < 0 || nq <= 0 || nkv <= 0 || d <= 0 || nq % nkv) return 2;
    const int32_t group = nq / nkv;
    const int64_t units = (int64_t)num_seqs * nq;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(pick_threads(nthreads)) reduction(| : bad)
    for (int64_t unit = 0; unit < units; ++unit) {
        const int32_t i = (int32_t)(unit / nq), h = (int32_t)(unit % nq), g = h / group;
        const int64_t start = cu_seqlens[i], len = (int64_t)cu_seqlens[i + 1] - cu_seqlens[i];
        if (len < 0) { bad |= 1; continue; }
        if (len == 0) continue;
        double *keys = malloc(sizeof(double) * len * d), *vals = malloc(sizeof(double) * len * d);
        double *qq = malloc(sizeof(double) * d), *s = malloc(sizeof(double) * len);
        double *o = malloc(sizeof(double) * d);
        for (int64_t u = 0; u < len; ++u)
            for (int32_t e = 0; e < d; ++e) {
                keys[u * d + e] = widen(k[((start + u) * nkv + g) * d + e]);
                vals[u * d + e] = widen(v[((start + u) * nkv + g) * d + e]);
            }
        for (int64_t t = 0; t < len; ++t) {
            const int64_t row = (start + t) * nq + h;
            for (int32_t e = 0; e < d; ++e) qq[e] = widen(q[row * d + e]);
            /* keys 0..t of this sequence: the causal, block-diagonal mask */
            attend(qq, keys, vals, t + 1, d, scale, s, o, &lse[row]);
            for (int32_t e = 0; e < d; ++e) out[row * d + e] = o[e];
        }
        free(keys); free(vals); free(qq); free(s); free(o);
    }
    return bad ? 2 : 0;
}

/*
 * Shared-prefix beam decode (article section 3.2, the equation
 * O_b = Attention(Q_b, [prefix_K; suffix_K[b]], [prefix_V; suffix_V[b]])).
 * The concatenated K/V is materialised explicitly here, per (request, beam,
 * kv head). q [R, W, nq, d]; prefix [R, Lp, nkv, d]; suffix [R, W, ls_cap, nkv, d]
 * of which the first ls positions are used. No mask: every key precedes the query.
 */
int32_t oracle_shared_prefix_decode(const uint16_t *q, const uint16_t *pk, const uint16_t *pv,
                                    const uint16_t *sk, const uint16_t *sv, int32_t R, int32_t W,
                                    int32_t Lp, int32_t Ls, int32_t Ls_cap, int32_t nq, int32_t nkv,
                                    int32_t d, double scale, double *out, double *lse, int32_t nthreads)
{
    if (!q || !pk || !pv || !out || !lse) return 1;
    if (Ls > 0 && (!sk || !sv)) return 1;
    if (R < 0 || W < 0 || Lp < 0 || Ls < 0 || Ls > Ls_cap || nq <= 0 || nkv <= 0 || nq % nkv || d <= 0)
        return 2;
    if (Lp + Ls == 0) return 2;
    const int32_t group = nq / nkv;
    const int64_t n = (int64_t)Lp + Ls;
    const int64_t units = (int64_t)R * W * nkv;
#pragma omp parallel for schedule(dynamic, 4) num_threads(pick_threads(nthreads))
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t r = unit / ((int64_t)W * nkv), b = (unit / nkv) % W, g = unit % nkv;
        double *kc = malloc(sizeof(double) * n * d), *vc = malloc(sizeof(double) * n * d);
        double *qq = malloc(sizeof(double) * d), *s = malloc(sizeof(double) * n), *o = malloc(sizeof(double) * d);
        for (int64_t u = 0; u < Lp; ++u)
            for (int32_t e = 0; e < d; ++e) {
                kc[u * d + e] = widen(pk[((r * Lp + u) * nkv + g) * d + e]);
                vc[u * d + e] = widen(pv[((r * Lp + u) * nkv + g) * d + e]);
            }
        for (int64_t j = 0; j < Ls; ++j)
            for (int32_t e = 0; e < d; ++e) {
                const int64_t src = (((r * W + b) * Ls_cap + j) * nkv + g) * d + e;
                kc[(Lp + j) * d + e] = widen(sk[src]);
                vc[(Lp + j) * d + e] = widen(sv[src]);
            }
        for (int32_t hg = 0; hg < group; ++hg) {
            const int64_t row = (r * W + b) * nq + g * group + hg;
            for (int32_t e = 0; e < d; ++e) qq[e] = widen(q[row * d + e]);
            attend(qq, kc, vc, n, d, scale, s, o, &lse[row]);
            for (int32_t e = 0; e < d; ++e) out[row * d + e] = o[e];
        }
        free(kc); free(vc); free(qq); free(s); free(o);
    }
    return 0;
}

/*
 * Shared-prefix beam decode where every request has a prompt of its own length,
 * the prompt K/V kept packed exactly as the packed prefill leaves it (article
 * section 3.2 equation; the packed layout of section 3.1). Request r's prompt is
 * rows prefix_cu[r] .. prefix_cu[r+1]-1 of pk/pv [T_p, nkv, d]; q, suffix, out
 * and lse as in oracle_shared_prefix_decode. The concatenation
 * [prompt of r; suffix of (r, b)] is again built explicitly.
 */
int32_t oracle_shared_prefix_decode_packed(const uint16_t *q, const uint16_t *pk, const uint16_t *pv,
                                           const int32_t *prefix_cu, const uint16_t *sk, const uint16_t *sv,
                                           int32_t R, int32_t W, int32_t Ls, int32_t Ls_cap, int32_t nq,
                                           int32_t nkv, int32_t d, double scale, double *out, double *lse,
                                           int32_t nthreads)
{
    if (!q || !prefix_cu || !out || !lse) return 1;
    if (Ls > 0 && (!sk || !sv)) return 1;
    if (R < 0 || W < 0 || Ls < 0 || Ls > Ls_cap || nq <= 0 || nkv <= 0 || nq % nkv || d <= 0) return 2;
    for (int32_t r = 0; r < R; ++r) {
        const int64_t lp = (int64_t)prefix_cu[r + 1] - prefix_cu[r];
        if (lp < 0 || lp + Ls == 0) return 2;
        if (lp > 0 && (!pk || !pv)) return 1;
    }
    const int32_t group = nq / nkv;
    const int64_t units = (int64_t)R * W * nkv;
#pragma omp parallel for schedule(dynamic, 4) num_threads(pick_threads(nthreads))
    for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t r = unit / ((int64_t)W * nkv), b = (unit / nkv) % W, g = unit % nkv;
        const int64_t p0 = prefix_cu[r], lp = (int64_t)prefix_cu[r + 1] - p0, n = lp + Ls;
        double *kc = malloc(sizeof(double) * n * d), *vc = malloc(sizeof(double) * n * d);
        double *qq = malloc(sizeof(double) * d), *s = malloc(sizeof(double) * n), *o = malloc(sizeof(double) * d);
        for (int64_t u = 0; u < lp; ++u)
            for (int32_t e = 0; e < d; ++e) {
                kc[u * d + e] = widen(pk[((p0 + u) * nkv + g) * d + e]);
                vc[u * d + e] = widen(pv[((p0 + u) * nkv + g) * d + e]);
            }
        for (int64_t j = 0; j < Ls; ++j)
            for (int32_t e = 0; e < d; ++e) {
                const int64_t at = (((r * W + b) * Ls_cap + j) * nkv + g) * d + e;
                kc[(lp + j) * d + e] = widen(sk[at]);
                vc[(lp + j) * d + e] = widen(sv[at]);
            }
        for (int32_t hg = 0; hg < group; ++hg) {
            const int64_t row = (r * W + b) * nq + g * group + hg;
            for (int32_t e = 0; e < d; ++e) qq[e] = widen(q[row * d + e]);
            attend(qq, kc, vc, n, d, scale, s, o, &lse[row]);
            for (int32_t e = 0; e < d; ++e) out[row * d + e] = o[e];
        }
        free(kc); free(vc); free(qq); free(s); free(o);
    }
    return 0;
}

/*
 * The last valid token of every packed sequence (article section 3.1: after
 * packed attention the same sequence boundary selects each sequence's
 * last-position hidden state). Row i of dst is row cu[i+1]-1 of src (rows of
 * row_bytes bytes); a zero-length sequence has no last token and gets a row of
 * zeros. Pure copy.
 */
int32_t oracle_last_token_gather(const uint8_t *src, const int32_t *cu, int32_t num_seqs, int64_t row_bytes,
                                 uint8_t *dst)
{
    if (!cu || !dst || (num_seqs > 0 && !src)) return 1;
    if (num_seqs < 0 || row_bytes < 0) return 2;
    for (int32_t i = 0; i < num_seqs; ++i) {
        const int64_t len = (int64_t)cu[i + 1] - cu[i];
        if (len < 0) return 2;
        if (len == 0) {
            memset(dst + (int64_t)i * row_bytes, 0, (size_t)row_bytes);
            continue;
        }
        const int64_t last = (int64_t)cu[i + 1] - 1;
        memcpy(dst + (int64_t)i * row_bytes, src + last * row_bytes, (size_t)row_bytes);
    }
    return 0;
}

/*
 * Parent-index reorder (article sections 3.2 and 3.3): new beam b takes the
 * suffix K/V (first Ls positions) and the token history of beam parent[r, b].
 * The prompt K/V is not touched. Pure copy.
 */
int32_t oracle_suffix_reorder(const uint16_t *src_k, const uint16_t *src_v, uint16_t *dst_k, uint16_t *dst_v,
                              const int32_t *parent, const int32_t *src_tok, int32_t *dst_tok, int32_t R,
                              int32_t W, int32_t Ls, int32_t Ls_cap, int32_t nkv, int32_t d, int32_t ntok,
                              int32_t tok_cap)
{
    if (!parent) return 1;
    const int64_t row = (int64_t)nkv * d;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t b = 0; b < W; ++b) {
            const int32_t p = parent[r * W + b];
            if (p < 0 || p >= W) return 2;
            for (int64_t j = 0; j < Ls; ++j)
                for (int64_t e = 0; e < row; ++e) {
                    dst_k[((r * W + b) * Ls_cap + j) * row + e] = src_k[((r * W + p) * Ls_cap + j) * row + e];
                    dst_v[((r * W + b) * Ls_cap + j) * row + e] = src_v[((r * W + p) * Ls_cap + j) * row + e];
                }
            if (src_tok && dst_tok)
                for (int64_t t = 0; t < ntok; ++t)
                    dst_tok[(r * W + b) * tok_cap + t] = src_tok[(r * W + p) * tok_cap + t];
        }
    return 0;
}

/* ---- beam top-K (article section 3.3) ---------------------------------- */

typedef struct { float x; int32_t id; } by_logit;
typedef struct { float s; int32_t f; } by_score;

/* larger logit first; equal logits (including -0 == +0): lower token id first */
static int cmp_logit(const void *a, const void *b)
{
    const by_logit *p = a, *q = b;
    if (p->x > q->x) return -1;
    if (p->x < q->x) return 1;
    return (p->id > q->id) - (p->id < q->id);
}

/* larger score first; equal scores: lower flattened index first */
static int cmp_score(const void *a, const void *b)
{
    const by_score *p = a, *q = b;
    if (p->s > q->s) return -1;
    if (p->s < q->s) return 1;
    return (p->f > q->f) - (p->f < q->f);
}

/*
 * Row log-sum-exp over the full vocabulary in fp64: lse = m + ln sum exp(x - m).
 */
static double row_lse64(const uint16_t *x, int32_t V)
{
    double m = -INFINITY;
    for (int32_t v = 0; v < V; ++v) { double t = widen(x[v]); if (t > m) m = t; }
    double l = 0.0;
    for (int32_t v = 0; v < V; ++v) l += exp(widen(x[v]) - m);
    return m + log(l);
}

/*
 * Two-stage candidate selection of one beam step (article section 3.3):
 *  stage 1, per beam row b: token ids ranked by bf16 logit (ties: lower id),
 *    first k_local kept; their fp32 log-probability lp = x - lse32 with lse32
 *    the fp32 rounding of the full-vocabulary fp64 log-sum-exp; score
 *    s = cum[b] + lp in fp32.
 *  stage 2, per request: the W_in*k_local candidates flattened as
 *    f = b*k_local + j, ranked by score (ties: lower f), first k_global kept;
 *    parent = f / k_local, token = local id at (parent, f % k_local).
 * cum may be NULL (all zero). local_* / row_lse* outputs may be NULL.
 */
/* Same selection with each row's fp32 log-sum-exp supplied by the caller
 * (lse_in[R * W_in]) instead of computed: where floating point decides the
 * integer result, this lets a test make that decision from the same fp32 row
 * log-sum-exp on both sides. row_lse / row_lse_f64 then echo lse_in. */
int32_t oracle_beam_topk_given_lse(const uint16_t *logits, const float *cum, const float *lse_in, int32_t R,
                                   int32_t W_in, int32_t V, int32_t k_local, int32_t k_global, int32_t *out_tokens,
                                   int32_t *out_parents, float *out_scores, int32_t *local_tokens,
                                   float *local_scores, float *row_lse, double *row_lse_f64, int32_t nthreads);

int32_t oracle_beam_topk(const uint16_t *logits, const float *cum, int32_t R, int32_t W_in, int32_t V,
                         int32_t k_local, int32_t k_global, int32_t *out_tokens, int32_t *out_parents,
                         float *out_scores, int32_t *local_tokens, float *local_scores, float *row_lse,
                         double *row_lse_f64, int32_t nthreads)
{
    return oracle_beam_topk_given_lse(logits, cum, NULL, R, W_in, V, k_local, k_global, out_tokens, out_parents,
                                      out_scores, local_tokens, local_scores, row_lse, row_lse_f64, nthreads);
}

int32_t oracle_beam_topk_given_lse(const uint16_t *logits, const float *cum, const float *lse_in, int32_t R,
                                   int32_t W_in, int32_t V, int32_t k_local, int32_t k_global, int32_t *out_tokens,
                                   int32_t *out_parents, float *out_scores, int32_t *local_tokens,
                                   float *local_scores, float *row_lse, double *row_lse_f64, int32_t nthreads)
{
    if (!logits || !out_tokens || !out_parents || !out_scores) return 1;
    if (R < 0 || W_in <= 0 || V <= 0 || k_local <= 0 || k_local > V || k_global <= 0 ||
        (int64_t)k_global > (int64_t)W_in * k_local)
        return 2;
    const int64_t rows = (int64_t)R * W_in;
    int32_t *ltok = malloc(sizeof(int32_t) * rows * k_local);
    float *lsc = malloc(sizeof(float) * rows * k_local);
    const int nt = pick_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t row = 0; row < rows; ++row) {
        const uint16_t *x = logits + row * V;
        const double lse64 = lse_in ? (double)lse_in[row] : row_lse64(x, V);
        const float lse32 = lse_in ? lse_in[row] : (float)lse64;
        by_logit *e = malloc(sizeof(by_logit) * V);
        for (int32_t v = 0; v < V; ++v) { e[v].x = widen_f(x[v]); e[v].id = v; }
        qsort(e, (size_t)V, sizeof *e, cmp_logit);
        const float c = cum ? cum[row] : 0.0f;
        for (int32_t j = 0; j < k_local; ++j) {
            volatile float lp = e[j].x - lse32;   /* one fp32 subtraction */
            volatile float s = c + lp;            /* one fp32 addition */
            ltok[row * k_local + j] = e[j].id;
            lsc[row * k_local + j] = s;
        }
        if (row_lse) row_lse[row] = lse32;
        if (row_lse_f64) row_lse_f64[row] = lse64;
        free(e);
    }
    if (local_tokens) memcpy(local_tokens, ltok, sizeof(int32_t) * rows * k_local);
    if (local_scores) memcpy(local_scores, lsc, sizeof(float) * rows * k_local);
    const int64_t nc = (int64_t)W_in * k_local;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t r = 0; r < R; ++r) {
        by_score *c = malloc(sizeof(by_score) * nc);
        for (int64_t f = 0; f < nc; ++f) { c[f].s = lsc[r * nc + f]; c[f].f = (int32_t)f; }
        qsort(c, (size_t)nc, sizeof *c, cmp_score);
        for (int32_t i = 0; i < k_global; ++i) {
            const int32_t parent = c[i].f / k_local, j = c[i].f % k_local;
            out_parents[r * k_global + i] = parent;
            out_tokens[r * k_global + i] = ltok[(r * W_in + parent) * k_local + j];
            out_scores[r * k_global + i] = c[i].s;
        }
        free(c);
    }
    free(ltok);
    free(lsc);
    return 0;
}

/* ---- selective FP8: fused SwiGLU requantisation (article section 3.4) ---- */

/*
 * OCP FP8 E4M3 ("e4m3fn") code of x: 1 sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits; no infinities; the all-ones exponent with mantissa 111 is
 * NaN, so the largest finite magnitude is 1.75 * 2^8 = 448; subnormals are
 * m/8 * 2^-6. Round to nearest, ties to even; magnitudes that round above 448
 * saturate to 448 (the requantisation never produces NaN).
 */
uint8_t oracle_e4m3_encode(double x)
{
    const uint8_t sign = (x < 0 || (x == 0 && signbit(x))) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a >= 464.0) return sign | 0x7E;   /* 464 is the midpoint between 448 and the next step, 480 */
    int e = a > 0 ? (int)floor(log2(a)) : -6;
    if (e < -6) e = -6;
    /* a / 2^(e-3) is exact in double; rint rounds to nearest even */
    double q = rint(ldexp(a, 3 - e));
    if (q >= 16.0) {   /* rounded up to the next binade */
        q = 8.0;
        e += 1;
    }
    if (q < 8.0) return sign | (uint8_t)q;                 /* subnormal (e == -6) or zero */
    if (e > 8 || (e == 8 && q > 14.0)) return sign | 0x7E;  /* above 448: saturate */
    return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

/* oracle_e4m3_encode over an array (for the tests) */
int32_t oracle_e4m3_encode_array(const double *x, int64_t n, uint8_t *out)
{
    if (!x || !out || n < 0) return 1;
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
    return 0;
}

/* value of an E4M3 code (for the tests) */
double oracle_e4m3_decode(uint8_t c)
{
    const double s = (c & 0x80) ? -1.0 : 1.0;
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return s * ldexp(m / 8.0, -6);
    return s * ldexp(1.0 + m / 8.0, e - 7);
}

/*
 * Per token (one row of the Gate/Up projection's output [T, 2I], gate in
 * columns 0..I-1 and up in I..2I-1): h = SiLU(gate) * up = gate / (1 + e^-gate)
 * * up; amax = max |h|; scale = max(amax, 1e-12) / 448; codes = E4M3(h /
 * scale). fp64 throughout (the definition; the kernel computes in fp32). Also
 * returns h and h / scale for the tests.
 */
int32_t oracle_swiglu_quant(const uint16_t *gate_up, int32_t T, int32_t I, uint8_t *codes, double *scale,
                            double *h_out, double *x_out, int32_t nthreads)
{
    if (!gate_up || !codes || !scale) return 1;
    if (T < 0 || I <= 0) return 2;
#pragma omp parallel for schedule(dynamic, 16) num_threads(pick_threads(nthreads))
    for (int32_t t = 0; t < T; ++t) {
        const uint16_t *row = gate_up + (int64_t)t * 2 * I;
        double *h = malloc(sizeof(double) * I);
        double amax = 0.0;
        for (int32_t j = 0; j < I; ++j) {
            const double g = widen(row[j]), u = widen(row[I + j]);
            h[j] = g / (1.0 + exp(-g)) * u;
            if (fabs(h[j]) > amax) amax = fabs(h[j]);
        }
        const double sc = (amax > 1e-12 ? amax : 1e-12) / 448.0;
        scale[t] = sc;
        for (int32_t j = 0; j < I; ++j) {
            const double x = h[j] / sc;
            codes[(int64_t)t * I + j] = oracle_e4m3_encode(x);
            if (h_out) h_out[(int64_t)t * I + j] = h[j];
            if (x_out) x_out[(int64_t)t * I + j] = x;
        }
        free(h);
    }
    return 0;
}
