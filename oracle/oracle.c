/*
 * Dynamic Bifocal RoPE attention -- plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link,
 * load or call this file; only the tests, the smoke check and the CPU
 * baseline leg of the benchmark do. It shares no code, header, table or
 * constant with the HIP library.
 *
 * What it evaluates is the per-pair piecewise definition of bifocal
 * attention, written out directly, with no tiling, no online softmax and
 * no merge trick:
 *
 *   s(L)  = max(1, ceil(L / w_pre))
 *           [Jet-Long promo script, papers.ananclaw.com, section 4
 *            storyboard, scene-2: the dynamic factor formula; ai-feeds.com
 *            summary, "方法 / 关键模块" items 1-2: s(L) = 1 while L is short,
 *            growing with L]
 *   local pair (i - j < w0): the model's original RoPE
 *           [ai-feeds.com summary, "方法 / 关键模块" item 1: a window of
 *            size w0 keeps unmodified RoPE]
 *   far pair: RoPE with positions replaced by phi(p)
 *           [same item: the long-range window uses the factor s(L)];
 *           phi(p) = p / s   (frequency interpolation, all frequencies / s)
 *           phi(p) = floor(p / s)   (position aliasing)
 *           [ai-feeds.com summary, "实验 / 关键发现", ablation bullet: the two
 *            long-branch strategies; mufans.github.io wiki, "Dynamic Bifocal
 *            RoPE 解决方案": far frequencies are the base frequencies times a
 *            factor below one]
 *   every causal pair counted exactly once, softmax over j <= i
 *           [seventnews.com (FR), paragraph on the fusion: local and long
 *            scores are combined without double counting]
 *
 * Readings taken where the pages are silent (each listed in the design
 * notes): inputs q', k' already carry original RoPE at their absolute
 * positions (the cache form); rotary pairs are half-split (m, m + D/2);
 * theta_m = base^(-2m/D); the softmax scale is the same in both branches;
 * one s per sequence, s = s(L) with L the sequence length; positions and s
 * restart per packed sequence; query head h reads KV head h / (Hq/Hkv).
 *
 * Route: every vector is first brought back to its raw (un-rotated) form
 * with R(-p*theta), and the far copy is then rotated to R(phi(p)*theta).
 * The oracle never forms the correction angle (phi(p) - p)*theta.
 * All arithmetic is fp64; inputs arrive as fp32 (bf16 inputs are widened
 * exactly before the call). sin/cos come from libm, which reduces large
 * arguments accurately.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD -1
#define ORC_NOMEM -2

/* ------------------------------------------------------------------ */
/* s(L): promo script, storyboard scene-2 formula.                     */
int64_t oracle_s_of_L(int64_t L, int64_t w_pre)
{
    if (L < 1 || w_pre < 1) return -1;
    int64_t q = L / w_pre;                 /* floor(L / w_pre)           */
    int64_t ceil_q = (q * w_pre == L) ? q : q + 1;
    return ceil_q > 1 ? ceil_q : 1;
}

/* phi(p) for the far branch; mode 0 = frequency interpolation (p / s),
 * mode 1 = position aliasing (floor(p / s)). */
double oracle_phi(int64_t p, int64_t s, int32_t mode)
{
    if (mode == 1) return (double)(p / s);      /* p >= 0, so / is floor */
    return (double)p / (double)s;
}

/* Half-split rotary rotation of one D-vector by angles pos * theta_m:
 *   y[m]       = x[m] cos a - x[m+H] sin a
 *   y[m+H]     = x[m+H] cos a + x[m] sin a,   a = pos * theta_m, H = D/2.
 * This is the standard RoPE rotation (reading: half-split pairing).      */
void oracle_rope_rotate(const double* x, double* y, int64_t D, double pos, double theta_base)
{
    int64_t H = D / 2;
    for (int64_t m = 0; m < H; ++m) {
        double th = pow(theta_base, -2.0 * (double)m / (double)D);
        double a = pos * th;
        double c = cos(a), s = sin(a);
        double x0 = x[m], x1 = x[m + H];
        y[m] = x0 * c - x1 * s;
        y[m + H] = x1 * c + x0 * s;
    }
}

/* far copy of an original-RoPE vector at position p: R(phi(p)) R(-p) x'  */
static void far_vector(const double* xp, double* out, int64_t D, int64_t p, int64_t s,
                       int32_t mode, double theta_base, double* tmp)
{
    oracle_rope_rotate(xp, tmp, D, -(double)p, theta_base);          /* raw */
    oracle_rope_rotate(tmp, out, D, oracle_phi(p, s, mode), theta_base);
}

/* Band-edge continuity shift (long-mode flag 4, off by default): the far
 * query is placed at phi(p) + delta with delta = w0 - phi(w0), so that a far
 * pair at distance exactly w0 sees relative position w0, as the band does
 * one step closer. FI: delta = w0 (s - 1) / s; PA: delta = w0 - floor(w0 / s)
 * (the offset of Self-Extend's grouped attention). The pages say the
 * correction rotation re-aligns the phases of the two branches without
 * fixing a constant [seventnews.com (FR), fusion paragraph; promo script,
 * "工程拐点" bullet: on-the-fly phase compensation]; the flag makes this
 * reading available next to the default (no shift).                      */
static double far_shift(int64_t w0, int64_t s, int32_t mode)
{
    return (double)w0 - oracle_phi(w0, s, mode);
}

static void far_query(const double* xp, double* out, int64_t D, int64_t p, int64_t s,
                      int32_t mode, double shift, double theta_base, double* tmp)
{
    oracle_rope_rotate(xp, tmp, D, -(double)p, theta_base);          /* raw */
    oracle_rope_rotate(tmp, out, D, oracle_phi(p, s, mode) + shift, theta_base);
}

static double dot(const double* a, const double* b, int64_t D)
{
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += a[d] * b[d];
    return acc;
}

static int64_t seq_of_token(const int64_t* cu, int64_t B, int64_t t)
{
    for (int64_t b = 0; b < B; ++b)
        if (t >= cu[b] && t < cu[b + 1]) return b;
    return -1;
}

/* ------------------------------------------------------------------ */
/* One query row: the direct piecewise definition with an exact two-pass
 * softmax.  kv_orig / kv_far point at position 0 of this sequence for the
 * query's KV head; qo / qf are the original and far query vectors.
 * band_only drops the far pairs altogether (mode 2: the band-only special
 * case, sliding-window attention over the w0 most recent keys with original
 * RoPE, as in the sliding-window layers of a hybrid model) [ai-feeds.com
 * summary, "关键模块" item 1: the w0 window keeps original RoPE; "核心洞察",
 * third bullet, and seventnews.com (FR), "Généralisation aux architectures
 * d'attention hybrides": hybrid designs where sliding-window and global
 * attention layers coexist].                                             */
static void one_row(const double* qo, const double* qf,
                    const double* k_orig, const double* k_far, const double* v,
                    int64_t i, int64_t D, int64_t w0, double scale, int band_only,
                    double* score_buf, double* o_out, double* lse_out)
{
    double M = -INFINITY;
    for (int64_t j = 0; j <= i; ++j) {
        double sc;
        if (i - j < w0)     sc = scale * dot(qo, k_orig + j * D, D);   /* local   */
        else if (band_only) sc = -INFINITY;                           /* dropped */
        else                sc = scale * dot(qf, k_far + j * D, D);    /* far     */
        score_buf[j] = sc;
        if (sc > M) M = sc;
    }
    double Z = 0.0;
    for (int64_t d = 0; d < D; ++d) o_out[d] = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        double e = exp(score_buf[j] - M);
        Z += e;
        const double* vj = v + j * D;
        for (int64_t d = 0; d < D; ++d) o_out[d] += e * vj[d];
    }
    for (int64_t d = 0; d < D; ++d) o_out[d] /= Z;
    *lse_out = M + log(Z);
}

/* Same row computed through the three partials of the inclusion-exclusion
 * reading: A = scaled branch over every causal pair, B = scaled branch over
 * the band, C = original branch over the band, all against one common max;
 * o = (N_A - N_B + N_C) / (Z_A - Z_B + Z_C).
 * [seventnews.com (FR), fusion paragraph; ai-feeds.com summary, "关键模块"
 *  item 3: inclusion-exclusion merge of the two windows]                 */
static void one_row_inclexcl(const double* qo, const double* qf,
                             const double* k_orig, const double* k_far, const double* v,
                             int64_t i, int64_t D, int64_t w0, double scale,
                             double* sfar, double* sloc, double* num, double* o_out,
                             double* lse_out)
{
    double M = -INFINITY;
    for (int64_t j = 0; j <= i; ++j) {
        sfar[j] = scale * dot(qf, k_far + j * D, D);
        if (sfar[j] > M) M = sfar[j];
        if (i - j < w0) {
            sloc[j] = scale * dot(qo, k_orig + j * D, D);
            if (sloc[j] > M) M = sloc[j];
        }
    }
    double ZA = 0.0, ZB = 0.0, ZC = 0.0;
    double* NA = num;
    double* NB = num + D;
    double* NC = num + 2 * D;
    for (int64_t d = 0; d < 3 * D; ++d) num[d] = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        const double* vj = v + j * D;
        double ea = exp(sfar[j] - M);
        ZA += ea;
        for (int64_t d = 0; d < D; ++d) NA[d] += ea * vj[d];
        if (i - j < w0) {
            double eb = ea;
            double ec = exp(sloc[j] - M);
            ZB += eb;
            ZC += ec;
            for (int64_t d = 0; d < D; ++d) { NB[d] += eb * vj[d]; NC[d] += ec * vj[d]; }
        }
    }
    double Z = ZA - ZB + ZC;
    for (int64_t d = 0; d < D; ++d) o_out[d] = (NA[d] - NB[d] + NC[d]) / Z;
    *lse_out = M + log(Z);
}

/* ------------------------------------------------------------------ */
/* Prefill over a packed ragged batch, evaluated at a chosen set of query
 * rows (global token indices).
 *   q_rows [Hq][n_rows][D]  query vectors of those rows (original RoPE)
 *   k, v   [Hkv][T][D]      packed keys / values, T = cu[B]
 *   cu     [B+1]            sequence offsets; positions restart per sequence
 *   o      [Hq][n_rows][D], lse [Hq][n_rows]  (natural log)
 *   mode 0 = FI, 1 = PA, 2 = band only (far pairs dropped); 4 | 0 and
 *   4 | 1 add the band-edge continuity shift to FI / PA.
 *   variant 0 = direct definition, 1 = inclusion-exclusion partials.
 * Returns 0, or a negative code for bad arguments / no memory.           */
int oracle_prefill_rows(const float* q_rows, const float* k, const float* v,
                        const int64_t* cu, int64_t B, const int64_t* rows, int64_t n_rows,
                        int64_t Hq, int64_t Hkv, int64_t D, int64_t w0, int64_t w_pre,
                        double theta_base, int32_t mode, double scale, int32_t variant,
                        double* o, double* lse)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 2 || D % 2 != 0 || D > 1024) return ORC_BAD;
    const int32_t shift_on = mode & 4;
    mode &= ~4;
    if (w0 < 0 || w_pre < 1 || mode < 0 || mode > 2 || (mode == 2 && (w0 < 1 || shift_on))) return ORC_BAD;
    if (variant == 1 && mode == 2) return ORC_BAD;  /* no scaled branch to subtract */
    for (int64_t b = 0; b < B; ++b)
        if (cu[b + 1] <= cu[b]) return ORC_BAD;
    const int64_t T = cu[B];
    const int64_t G = Hq / Hkv;

    /* For every sequence that has a requested row, build fp64 original and
     * far copies of the keys it needs (positions 0 .. max requested row). */
    int64_t* need = (int64_t*)calloc((size_t)B, sizeof(int64_t));  /* rows needed per seq */
    if (!need) return ORC_NOMEM;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b = seq_of_token(cu, B, rows[r]);
        if (b < 0) { free(need); return ORC_BAD; }
        int64_t i = rows[r] - cu[b];
        if (i + 1 > need[b]) need[b] = i + 1;
    }
    int64_t total_need = 0;
    int64_t* base = (int64_t*)calloc((size_t)B + 1, sizeof(int64_t));
    if (!base) { free(need); return ORC_NOMEM; }
    for (int64_t b = 0; b < B; ++b) { base[b] = total_need; total_need += need[b]; }
    base[B] = total_need;

    size_t nk = (size_t)Hkv * (size_t)total_need * (size_t)D;
    double* ko = (double*)malloc((nk ? nk : 1) * sizeof(double));
    double* kf = (double*)malloc((nk ? nk : 1) * sizeof(double));
    double* vv = (double*)malloc((nk ? nk : 1) * sizeof(double));
    if (!ko || !kf || !vv) { free(ko); free(kf); free(vv); free(need); free(base); return ORC_NOMEM; }

    for (int64_t b = 0; b < B; ++b) {
        if (!need[b]) continue;
        int64_t L = cu[b + 1] - cu[b];
        int64_t s = oracle_s_of_L(L, w_pre);
        #pragma omp parallel for collapse(2) schedule(static)
        for (int64_t h = 0; h < Hkv; ++h)
            for (int64_t p = 0; p < need[b]; ++p) {
                double tmp[1024];
                double xo[1024];
                size_t src = ((size_t)h * (size_t)T + (size_t)(cu[b] + p)) * (size_t)D;
                size_t dst = ((size_t)h * (size_t)total_need + (size_t)(base[b] + p)) * (size_t)D;
                for (int64_t d = 0; d < D; ++d) {
                    xo[d] = (double)k[src + d];
                    ko[dst + d] = xo[d];
                    vv[dst + d] = (double)v[src + d];
                }
                far_vector(xo, kf + dst, D, p, s, mode, theta_base, tmp);
            }
    }

    int64_t maxL = 0;
    for (int64_t b = 0; b < B; ++b) if (need[b] > maxL) maxL = need[b];
    int err = ORC_OK;

    #pragma omp parallel
    {
        double* buf = (double*)malloc((size_t)(2 * maxL + 4 * D + 2048) * sizeof(double));
        if (!buf) {
            #pragma omp atomic write
            err = ORC_NOMEM;
        } else {
            double* s1 = buf;
            double* s2 = buf + maxL;
            double* num = buf + 2 * maxL;
            double* qo = num + 3 * D;
            double* qf = qo + 1024;
            double tmp[1024];
            #pragma omp for collapse(2) schedule(dynamic, 1)
            for (int64_t h = 0; h < Hq; ++h)
                for (int64_t r = 0; r < n_rows; ++r) {
                    int64_t t = rows[r];
                    int64_t b = seq_of_token(cu, B, t);
                    int64_t i = t - cu[b];
                    int64_t L = cu[b + 1] - cu[b];
                    int64_t s = oracle_s_of_L(L, w_pre);
                    const double shift = shift_on ? far_shift(w0, s, mode) : 0.0;
                    int64_t hk = h / G;
                    const float* qsrc = q_rows + ((size_t)h * (size_t)n_rows + (size_t)r) * (size_t)D;
                    for (int64_t d = 0; d < D; ++d) qo[d] = (double)qsrc[d];
                    far_query(qo, qf, D, i, s, mode, shift, theta_base, tmp);
                    size_t kb = ((size_t)hk * (size_t)total_need + (size_t)base[b]) * (size_t)D;
                    double* orow = o + ((size_t)h * (size_t)n_rows + (size_t)r) * (size_t)D;
                    double* lrow = lse + (size_t)h * (size_t)n_rows + (size_t)r;
                    if (variant == 1)
                        one_row_inclexcl(qo, qf, ko + kb, kf + kb, vv + kb, i, D, w0, scale,
                                         s1, s2, num, orow, lrow);
                    else
                        one_row(qo, qf, ko + kb, kf + kb, vv + kb, i, D, w0, scale, mode == 2, s1,
                                orow, lrow);
                }
            free(buf);
        }
    }
    free(ko); free(kf); free(vv); free(need); free(base);
    return err;
}

/* ------------------------------------------------------------------ */
/* Single-token decode over a KV cache: row N-1 of the prefill definition
 * with L = N, where N = seqlens[b] counts every valid key including the new
 * token's own (reading: the new token's K/V is appended before attention).
 *   q [B][Hq][D], k_cache / v_cache [B][Hkv][cap][D], o [B][Hq][D], lse [B][Hq]
 * [promo script, voice-over: single-batch generation; ai-feeds.com
 *  summary, "关键模块" item 3: correction applied to cached keys]         */
int oracle_decode(const float* q, const float* k_cache, const float* v_cache,
                  const int64_t* seqlens, int64_t B, int64_t cap, int64_t Hq, int64_t Hkv,
                  int64_t D, int64_t w0, int64_t w_pre, double theta_base, int32_t mode,
                  double scale, double* o, double* lse)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 2 || D % 2 != 0 || D > 1024) return ORC_BAD;
    const int32_t shift_on = mode & 4;
    mode &= ~4;
    if (w0 < 0 || w_pre < 1 || mode < 0 || mode > 2 || (mode == 2 && (w0 < 1 || shift_on))) return ORC_BAD;
    int64_t maxN = 0;
    for (int64_t b = 0; b < B; ++b) {
        if (seqlens[b] < 1 || seqlens[b] > cap) return ORC_BAD;
        if (seqlens[b] > maxN) maxN = seqlens[b];
    }
    const int64_t G = Hq / Hkv;
    int err = ORC_OK;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t N = seqlens[b];
        const int64_t s = oracle_s_of_L(N, w_pre);
        const double shift = shift_on ? far_shift(w0, s, mode) : 0.0;
        size_t nk = (size_t)Hkv * (size_t)N * (size_t)D;
        double* ko = (double*)malloc(nk * sizeof(double));
        double* kf = (double*)malloc(nk * sizeof(double));
        double* vv = (double*)malloc(nk * sizeof(double));
        if (!ko || !kf || !vv) { free(ko); free(kf); free(vv); return ORC_NOMEM; }
        #pragma omp parallel for collapse(2) schedule(static)
        for (int64_t h = 0; h < Hkv; ++h)
            for (int64_t p = 0; p < N; ++p) {
                double tmp[1024];
                size_t src = (((size_t)b * (size_t)Hkv + (size_t)h) * (size_t)cap + (size_t)p) * (size_t)D;
                size_t dst = ((size_t)h * (size_t)N + (size_t)p) * (size_t)D;
                for (int64_t d = 0; d < D; ++d) {
                    ko[dst + d] = (double)k_cache[src + d];
                    vv[dst + d] = (double)v_cache[src + d];
                }
                far_vector(ko + dst, kf + dst, D, p, s, mode, theta_base, tmp);
            }
        #pragma omp parallel
        {
            double* sb = (double*)malloc((size_t)(N + 3 * D) * sizeof(double));
            if (!sb) {
                #pragma omp atomic write
                err = ORC_NOMEM;
            } else {
                double qo[1024], qf[1024], tmp[1024];
                #pragma omp for schedule(dynamic, 1)
                for (int64_t h = 0; h < Hq; ++h) {
                    int64_t hk = h / G;
                    const float* qs = q + ((size_t)b * (size_t)Hq + (size_t)h) * (size_t)D;
                    for (int64_t d = 0; d < D; ++d) qo[d] = (double)qs[d];
                    far_query(qo, qf, D, N - 1, s, mode, shift, theta_base, tmp);
                    size_t kb = (size_t)hk * (size_t)N * (size_t)D;
                    one_row(qo, qf, ko + kb, kf + kb, vv + kb, N - 1, D, w0, scale, mode == 2, sb,
                            o + ((size_t)b * (size_t)Hq + (size_t)h) * (size_t)D,
                            lse + (size_t)b * (size_t)Hq + (size_t)h);
                }
                free(sb);
            }
        }
        free(ko); free(kf); free(vv);
        if (err) return err;
    }
    return err;
}

/* ------------------------------------------------------------------ */
/* Multi-token queries over a KV cache (chunked prefill): sequence b holds
 * N_b = seqlens[b] keys in the cache and its Lq_b = cu_q[b+1] - cu_q[b]
 * queries are the last Lq_b positions N_b - Lq_b .. N_b - 1. A query at
 * position i is the prefill row i of that sequence with L = s_len[b]
 * (N_b when s_len is NULL), evaluated at the chosen packed query rows.
 *   q_rows [Hq][n_rows][D]  query vectors of those rows (original RoPE)
 *   k_cache, v_cache [B][Hkv][cap][D]
 *   o [Hq][n_rows][D], lse [Hq][n_rows]
 * [mufans.github.io wiki, Jet-Long Dynamic RoPE, "可执行建议": use with
 *  prompt caching; ai-feeds.com summary, "关键模块" item 3: correction of
 *  cached keys]                                                          */
int oracle_chunk_rows(const float* q_rows, const float* k_cache, const float* v_cache,
                      const int64_t* cu_q, const int64_t* seqlens, const int64_t* s_len,
                      int64_t B, int64_t cap, const int64_t* rows, int64_t n_rows,
                      int64_t Hq, int64_t Hkv, int64_t D, int64_t w0, int64_t w_pre,
                      double theta_base, int32_t mode, double scale, double* o, double* lse)
{
    if (B < 1 || cap < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 2 || D % 2 != 0 || D > 1024)
        return ORC_BAD;
    const int32_t shift_on = mode & 4;
    mode &= ~4;
    if (w0 < 0 || w_pre < 1 || mode < 0 || mode > 2 || (mode == 2 && (w0 < 1 || shift_on))) return ORC_BAD;
    if (cu_q[0] != 0) return ORC_BAD;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t Lq = cu_q[b + 1] - cu_q[b];
        if (Lq < 1 || seqlens[b] < Lq || seqlens[b] > cap) return ORC_BAD;
        if (s_len && s_len[b] < seqlens[b]) return ORC_BAD;
    }
    const int64_t G = Hq / Hkv;
    /* keys each sequence needs: positions 0 .. largest requested position */
    int64_t* need = (int64_t*)calloc((size_t)B, sizeof(int64_t));
    int64_t* base = (int64_t*)calloc((size_t)B + 1, sizeof(int64_t));
    if (!need || !base) { free(need); free(base); return ORC_NOMEM; }
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t b = seq_of_token(cu_q, B, rows[r]);
        if (b < 0) { free(need); free(base); return ORC_BAD; }
        const int64_t i = seqlens[b] - (cu_q[b + 1] - cu_q[b]) + (rows[r] - cu_q[b]);
        if (i + 1 > need[b]) need[b] = i + 1;
    }
    for (int64_t b = 0; b < B; ++b) base[b + 1] = base[b] + need[b];
    const int64_t total = base[B];
    const size_t nk = (size_t)Hkv * (size_t)total * (size_t)D;
    double* ko = (double*)malloc((nk ? nk : 1) * sizeof(double));
    double* kf = (double*)malloc((nk ? nk : 1) * sizeof(double));
    double* vv = (double*)malloc((nk ? nk : 1) * sizeof(double));
    if (!ko || !kf || !vv) { free(ko); free(kf); free(vv); free(need); free(base); return ORC_NOMEM; }
    for (int64_t b = 0; b < B; ++b) {
        if (!need[b]) continue;
        const int64_t s = oracle_s_of_L(s_len ? s_len[b] : seqlens[b], w_pre);
        #pragma omp parallel for collapse(2) schedule(static)
        for (int64_t h = 0; h < Hkv; ++h)
            for (int64_t p = 0; p < need[b]; ++p) {
                double tmp[1024];
                const size_t src = (((size_t)b * (size_t)Hkv + (size_t)h) * (size_t)cap + (size_t)p) * (size_t)D;
                const size_t dst = ((size_t)h * (size_t)total + (size_t)(base[b] + p)) * (size_t)D;
                for (int64_t d = 0; d < D; ++d) {
                    ko[dst + d] = (double)k_cache[src + d];
                    vv[dst + d] = (double)v_cache[src + d];
                }
                far_vector(ko + dst, kf + dst, D, p, s, mode, theta_base, tmp);
            }
    }
    int64_t maxn = 0;
    for (int64_t b = 0; b < B; ++b) if (need[b] > maxn) maxn = need[b];
    int err = ORC_OK;
    #pragma omp parallel
    {
        double* sb = (double*)malloc((size_t)(maxn + 1) * sizeof(double));
        if (!sb) {
            #pragma omp atomic write
            err = ORC_NOMEM;
        } else {
            double qo[1024], qf[1024], tmp[1024];
            #pragma omp for collapse(2) schedule(dynamic, 1)
            for (int64_t h = 0; h < Hq; ++h)
                for (int64_t r = 0; r < n_rows; ++r) {
                    const int64_t b = seq_of_token(cu_q, B, rows[r]);
                    const int64_t i = seqlens[b] - (cu_q[b + 1] - cu_q[b]) + (rows[r] - cu_q[b]);
                    const int64_t s = oracle_s_of_L(s_len ? s_len[b] : seqlens[b], w_pre);
                    const double shift = shift_on ? far_shift(w0, s, mode) : 0.0;
                    const float* qs = q_rows + ((size_t)h * (size_t)n_rows + (size_t)r) * (size_t)D;
                    for (int64_t d = 0; d < D; ++d) qo[d] = (double)qs[d];
                    far_query(qo, qf, D, i, s, mode, shift, theta_base, tmp);
                    const size_t kb = ((size_t)(h / G) * (size_t)total + (size_t)base[b]) * (size_t)D;
                    one_row(qo, qf, ko + kb, kf + kb, vv + kb, i, D, w0, scale, mode == 2, sb,
                            o + ((size_t)h * (size_t)n_rows + (size_t)r) * (size_t)D,
                            lse + (size_t)h * (size_t)n_rows + (size_t)r);
                }
            free(sb);
        }
    }
    free(ko); free(kf); free(vv); free(need); free(base);
    return err;
}

/* Classification of one pair, for the integer pins: returns 1 for a local
 * pair (original RoPE), 2 for a far pair (scaled RoPE), 0 for a pair the
 * causal mask removes (j > i).                                           */
int32_t oracle_pair_branch(int64_t i, int64_t j, int64_t w0)
{
    if (j > i) return 0;
    return (i - j < w0) ? 1 : 2;
}

/* Original RoPE of packed rows (the raw-input pre-step): row (h, t) of
 * x [H][T][D] is the raw vector of a token at position pos[t], and y gets
 * the model's own rotation of it, R(pos[t] * theta) x, in fp64.
 * [mufans.github.io wiki, Jet-Long Dynamic RoPE, "关键实现 / 推理流程":
 *  the flow starts by computing RoPE for the input tokens]               */
int oracle_rope_rows(const float* x, double* y, int64_t H, int64_t T, int64_t D,
                     const int64_t* pos, double theta_base)
{
    if (H < 1 || T < 1 || D < 2 || (D & 1)) return ORC_BAD;
    double* row = (double*)malloc(sizeof(double) * (size_t)D);
    if (!row) return ORC_NOMEM;
    for (int64_t h = 0; h < H; ++h)
        for (int64_t t = 0; t < T; ++t) {
            const float* xr = x + (h * T + t) * D;
            for (int64_t d = 0; d < D; ++d) row[d] = (double)xr[d];
            oracle_rope_rotate(row, y + (h * T + t) * D, D, (double)pos[t], theta_base);
        }
    free(row);
    return ORC_OK;
}
