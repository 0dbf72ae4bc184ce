/*
 * fp64 CPU oracle for MLA decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header or
 * constant with the GPU library; the product path never calls it.
 *
 * What it computes is plain softmax attention as the FlashMLA-ETAP summary
 * states it in "Mecanismo Central": scores S = Q K^T (times the softmax scale),
 * P = softmax(S) along the key axis, O = P V; with the max-subtracted softmax
 * the blog page shows under "数值稳定性增强" (without its epsilon in the
 * denominator), evaluated in double precision as the pages' accuracy figure
 * uses a double-precision reference ("Estabilidade Numerica").  The cache row
 * is the MLA latent plus the shared RoPE key (GQLA summary, "Arquitetura",
 * absorbed-MQA path): 576 dims, of which the first 512 are the value.
 *
 * The log-sum-exp (natural log, scale included) is returned with O so that
 * partial results over disjoint key sets can be merged; a row that sees no
 * key returns O = 0 and LSE = -inf.
 *
 * Parity pins (brute force, closed forms, invariants) live in the tests; the
 * ORACLE_PLANTED_MISTAKE hooks below exist only so those tests can check that
 * each pin catches a plausible bug.  A normal build defines none of them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_PLANTED_MISTAKE
#define ORACLE_PLANTED_MISTAKE 0
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_PAGE (-2)
#define ORACLE_ERR_NOMEM (-3)

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Softmax attention over one query row given its n scores (already scaled).
 * Turns scores[] into unnormalised weights e_j = exp(s_j - max) and returns
 * l = sum_j e_j and the max through *m.
 */
static double softmax_weights(double *scores, int64_t n, double *m)
{
    double mx = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (scores[j] > mx)
            mx = scores[j];
#if ORACLE_PLANTED_MISTAKE == 3
    mx = -mx; /* planted: wrong sign in the max subtraction */
#endif
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        scores[j] = exp(scores[j] - mx);
        l += scores[j];
    }
    *m = mx;
    return l;
}

static double finish_lse(double m, double l)
{
#if ORACLE_PLANTED_MISTAKE == 4
    return m + log2(l); /* planted: base-2 log */
#else
    return m + log(l);
#endif
}

/*
 * Dense attention: q [n_q][d_k], k [n_k][d_k], v [n_k][d_v] (row-major fp64).
 * Outputs o [n_q][d_v], lse [n_q] and, if p is not NULL, the probabilities
 * p [n_q][n_k].
 */
int oracle_attention_f64(int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v,
                         const double *q, const double *k, const double *v, double scale,
                         double *o, double *lse, double *p)
{
    if (n_q < 0 || n_k < 0 || d_k <= 0 || d_v <= 0 || !q || !o || !lse || (n_k > 0 && (!k || !v)))
        return ORACLE_ERR_ARG;
    double *w = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
    if (!w)
        return ORACLE_ERR_NOMEM;
    for (int64_t r = 0; r < n_q; ++r) {
        double *orow = o + r * d_v;
        for (int64_t d = 0; d < d_v; ++d)
            orow[d] = 0.0;
        if (n_k == 0) {
            lse[r] = -INFINITY;
            continue;
        }
        for (int64_t j = 0; j < n_k; ++j) {
            double s = 0.0;
            for (int64_t d = 0; d < d_k; ++d) {
#if ORACLE_PLANTED_MISTAKE == 5
                s += q[r * d_k + d] * k[d * n_k + j]; /* planted: K read transposed */
#else
                s += q[r * d_k + d] * k[j * d_k + d];
#endif
            }
#if ORACLE_PLANTED_MISTAKE == 1
            w[j] = s; /* planted: scale dropped */
#else
            w[j] = scale * s;
#endif
        }
        double m;
        double l = softmax_weights(w, n_k, &m);
        for (int64_t j = 0; j < n_k; ++j) {
            for (int64_t d = 0; d < d_v; ++d)
                orow[d] += w[j] * v[j * d_v + d];
            if (p)
                p[r * n_k + j] = w[j] / l;
        }
        for (int64_t d = 0; d < d_v; ++d)
            orow[d] /= l;
        lse[r] = finish_lse(m, l);
    }
    free(w);
    return ORACLE_OK;
}

/*
 * MLA decode over a paged bf16 latent cache.
 *   q           bf16 bits [batch][s_q][heads][d_k]
 *   cache       bf16 bits [num_pages][page_size][d_k]; the value of a key is its
 *               first d_v dims
 *   block_table int32 [batch][bt_stride]: logical page p of sequence b lives in
 *               pool page block_table[b][p]
 *   seqlens     int32 [batch]: context length L_b, counting the s_q new tokens
 *   causal      query token i sees keys 0 .. L_b - s_q + i (bottom-right
 *               aligned); otherwise every query token sees all L_b keys
 *   rows        optional list of flattened rows (b*s_q + i)*heads + h; NULL
 *               means every row in that order
 *   o, lse      fp64 [n_rows][d_v], [n_rows]
 * Returns ORACLE_ERR_PAGE if a page a visible key needs is outside the pool.
 */
static int decode_rows(const uint16_t *q, const uint16_t *cache, const int32_t *block_table,
                       int64_t bt_stride, const int32_t *seqlens, int64_t batch, int64_t s_q,
                       int64_t heads, int64_t num_pages, int64_t page_size, int64_t d_k,
                       int64_t d_v, double scale, int causal, const int64_t *rows,
                       int64_t n_rows, double *o, double *o_abs, double *lse, int n_threads);

int oracle_mla_decode(const uint16_t *q, const uint16_t *cache, const int32_t *block_table,
                      int64_t bt_stride, const int32_t *seqlens, int64_t batch, int64_t s_q,
                      int64_t heads, int64_t num_pages, int64_t page_size, int64_t d_k,
                      int64_t d_v, double scale, int causal, const int64_t *rows,
                      int64_t n_rows, double *o, double *lse, int n_threads)
{
    return decode_rows(q, cache, block_table, bt_stride, seqlens, batch, s_q, heads, num_pages,
                       page_size, d_k, d_v, scale, causal, rows, n_rows, o, NULL, lse, n_threads);
}

/*
 * The same, with a second output o_abs[n_rows][d_v] = sum_j p_j |v_j| (the attention of the
 * absolute values under the same weights).  It is the scale of the error that rounding the
 * weights p_j (to a short format, before the weighted sum) can cause in O, so the tests derive
 * their per-element tolerance from it; it bounds |O| elementwise and equals it when every value
 * is nonnegative.
 */
int oracle_mla_decode_with_scale(const uint16_t *q, const uint16_t *cache, const int32_t *block_table,
                                 int64_t bt_stride, const int32_t *seqlens, int64_t batch, int64_t s_q,
                                 int64_t heads, int64_t num_pages, int64_t page_size, int64_t d_k,
                                 int64_t d_v, double scale, int causal, const int64_t *rows,
                                 int64_t n_rows, double *o, double *o_abs, double *lse, int n_threads)
{
    if (!o_abs)
        return ORACLE_ERR_ARG;
    return decode_rows(q, cache, block_table, bt_stride, seqlens, batch, s_q, heads, num_pages,
                       page_size, d_k, d_v, scale, causal, rows, n_rows, o, o_abs, lse, n_threads);
}

static int decode_rows(const uint16_t *q, const uint16_t *cache, const int32_t *block_table,
                       int64_t bt_stride, const int32_t *seqlens, int64_t batch, int64_t s_q,
                       int64_t heads, int64_t num_pages, int64_t page_size, int64_t d_k,
                       int64_t d_v, double scale, int causal, const int64_t *rows,
                       int64_t n_rows, double *o, double *o_abs, double *lse, int n_threads)
{
    if (!q || !cache || !block_table || !seqlens || !o || !lse || batch <= 0 || s_q <= 0 ||
        heads <= 0 || num_pages <= 0 || page_size <= 0 || d_k <= 0 || d_v <= 0 || d_v > d_k ||
        bt_stride <= 0)
        return ORACLE_ERR_ARG;
    const int64_t total_rows = batch * s_q * heads;
    if (!rows)
        n_rows = total_rows;
    for (int64_t b = 0; b < batch; ++b)
        if (seqlens[b] < 0 || (seqlens[b] + page_size - 1) / page_size > bt_stride)
            return ORACLE_ERR_ARG;
    for (int64_t t = 0; t < n_rows; ++t)
        if (rows && (rows[t] < 0 || rows[t] >= total_rows))
            return ORACLE_ERR_ARG;
    int status = ORACLE_OK;
    (void)n_threads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int64_t t = 0; t < n_rows; ++t) {
        const int64_t row = rows ? rows[t] : t;
        const int64_t h = row % heads;
        const int64_t i = (row / heads) % s_q;
        const int64_t b = row / (heads * s_q);
        const int64_t L = seqlens[b];
#if ORACLE_PLANTED_MISTAKE == 6
        int64_t n = causal ? L - s_q + i : L; /* planted: off-by-one causal rule */
#else
        int64_t n = causal ? L - s_q + 1 + i : L;
#endif
        if (n < 0)
            n = 0;
        if (n > L)
            n = L;
        double *orow = o + t * d_v;
        double *arow = o_abs ? o_abs + t * d_v : NULL;
        for (int64_t d = 0; d < d_v; ++d)
            orow[d] = 0.0;
        if (arow)
            for (int64_t d = 0; d < d_v; ++d)
                arow[d] = 0.0;
        if (n == 0) {
            lse[t] = -INFINITY;
            continue;
        }
        const uint16_t *qrow = q + ((b * s_q + i) * heads + h) * d_k;
        double *w = (double *)malloc(sizeof(double) * (size_t)n);
        const uint16_t **keys = (const uint16_t **)malloc(sizeof(void *) * (size_t)n);
        if (!w || !keys) {
            free(w);
            free((void *)keys);
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
            continue;
        }
        int bad = 0;
        for (int64_t j = 0; j < n; ++j) {
#if ORACLE_PLANTED_MISTAKE == 7
            /* planted: pages taken as contiguous after the first table entry */
            int64_t page = block_table[b * bt_stride] + j / page_size;
            int64_t slot = j % page_size;
#else
            int64_t page = block_table[b * bt_stride + j / page_size];
            int64_t slot = j % page_size;
#endif
            if (page < 0 || page >= num_pages) {
                bad = 1;
                break;
            }
            keys[j] = cache + (page * page_size + slot) * d_k;
            double s = 0.0;
            for (int64_t d = 0; d < d_k; ++d)
                s += bf16_to_f64(qrow[d]) * bf16_to_f64(keys[j][d]);
#if ORACLE_PLANTED_MISTAKE == 1
            w[j] = s; /* planted: scale dropped */
#else
            w[j] = scale * s;
#endif
        }
        if (bad) {
            free(w);
            free((void *)keys);
#pragma omp atomic write
            status = ORACLE_ERR_PAGE;
            continue;
        }
        double m;
        double l = softmax_weights(w, n, &m);
        for (int64_t j = 0; j < n; ++j) {
#if ORACLE_PLANTED_MISTAKE == 2
            const uint16_t *vrow = keys[j] + (d_k - d_v); /* planted: value = last d_v dims */
#else
            const uint16_t *vrow = keys[j];
#endif
            for (int64_t d = 0; d < d_v; ++d)
                orow[d] += w[j] * bf16_to_f64(vrow[d]);
            if (arow)
                for (int64_t d = 0; d < d_v; ++d)
                    arow[d] += w[j] * fabs(bf16_to_f64(vrow[d]));
        }
        for (int64_t d = 0; d < d_v; ++d)
            orow[d] /= l;
        if (arow)
            for (int64_t d = 0; d < d_v; ++d)
                arow[d] /= l;
        lse[t] = finish_lse(m, l);
        free(w);
        free((void *)keys);
    }
    return status;
}

int oracle_planted_mistake(void) { return ORACLE_PLANTED_MISTAKE; }
