/*
 * Plain fp64 attention oracle in C, with OpenMP over output rows.
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the library.
 *
 * Definition followed: lecompute.fr, "FlashAttention-4 : limites du calcul
 * matriciel", section "Entre deux multiplications il faut fabriquer les
 * poids" -- scores from query/key dot products, a softmax that makes
 * positive weights summing to one, then a weighted mix of the values.  The
 * causal reach follows section "Le FP4 ajoute un compromis numérique" of the
 * same page, read with bottom-right alignment (query i sees key j iff
 * j <= i + Skv - Sq).
 *
 * Each requested row materialises its whole score row in fp64, subtracts the
 * row maximum, exponentiates with libm exp, sums, mixes V and divides.  Inputs
 * are bfloat16 bit patterns, widened exactly to double.  A row with no allowed
 * key yields O = 0 and LSE = -inf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One output row: q_row[d]; keys/values are n_ok rows at stride kv_stride
 * elements; scores is scratch of n_ok doubles. */
static void one_row(const uint16_t *q_row, const uint16_t *k0, const uint16_t *v0,
                    int64_t kv_stride, int n_ok, int d, double scale,
                    double *scores, double *o, double *lse) {
    int c, j;
    if (n_ok <= 0) {
        for (c = 0; c < d; ++c) o[c] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (j = 0; j < n_ok; ++j) {
        const uint16_t *kr = k0 + (int64_t)j * kv_stride;
        double acc = 0.0;
        for (c = 0; c < d; ++c) acc += bf16_to_double(q_row[c]) * bf16_to_double(kr[c]);
        scores[j] = scale * acc;
        if (scores[j] > m) m = scores[j];
    }
    double l = 0.0;
    for (j = 0; j < n_ok; ++j) {
        scores[j] = exp(scores[j] - m);
        l += scores[j];
    }
    for (c = 0; c < d; ++c) o[c] = 0.0;
    for (j = 0; j < n_ok; ++j) {
        const uint16_t *vr = v0 + (int64_t)j * kv_stride;
        for (c = 0; c < d; ++c) o[c] += scores[j] * bf16_to_double(vr[c]);
    }
    for (c = 0; c < d; ++c) o[c] /= l;
    *lse = m + log(l);
}

/*
 * Fixed-batch layout: q [B,Sq,Hq,d], k/v [B,Skv,Hkv,d] (bf16 bits).
 * rows: n triples (b, h, i).  o: n x d doubles, lse: n doubles.
 * Query head h reads KV head h / (Hq / Hkv).  nthreads <= 0: OpenMP default.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int B, int Hq, int Hkv, int Sq, int Skv, int d, double scale,
                     int causal, const int64_t *rows, int64_t n, double *o, double *lse,
                     int nthreads) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || d < 1 || Hq % Hkv) return -1;
    for (int64_t r = 0; r < n; ++r) {
        int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Sq) return -1;
    }
    int grp = Hq / Hkv;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)Skv);
        if (!scores) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < n; ++r) {
                int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
                int64_t hk = h / grp;
                int64_t lim = causal ? i + (Skv - Sq) + 1 : Skv;
                int n_ok = (int)(lim < 0 ? 0 : (lim > Skv ? Skv : lim));
                const uint16_t *qr = q + (((b * Sq + i) * Hq + h) * d);
                const uint16_t *k0 = k + ((b * Skv) * Hkv + hk) * d;
                const uint16_t *v0 = v + ((b * Skv) * Hkv + hk) * d;
                one_row(qr, k0, v0, (int64_t)Hkv * d, n_ok, d, scale, scores,
                        o + r * d, lse + r);
            }
            free(scores);
        }
    }
    return err ? -1 : 0;
}

/*
 * Packed ragged layout: q [Tq,Hq,d], k/v [Tk,Hkv,d]; sequence s owns query
 * rows cu_q[s]..cu_q[s+1]-1 and keys cu_k[s]..cu_k[s+1]-1.
 * rows: n triples (s, h, i) with i local to the sequence.
 */
int oracle_attn_varlen_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const int32_t *cu_q, const int32_t *cu_k, int nseq, int Hq,
                            int Hkv, int d, double scale, int causal, const int64_t *rows,
                            int64_t n, double *o, double *lse, int nthreads) {
    if (nseq < 1 || Hq < 1 || Hkv < 1 || d < 1 || Hq % Hkv) return -1;
    int maxk = 0;
    for (int s = 0; s < nseq; ++s) {
        if (cu_q[s + 1] < cu_q[s] || cu_k[s + 1] < cu_k[s]) return -1;
        if (cu_k[s + 1] - cu_k[s] > maxk) maxk = cu_k[s + 1] - cu_k[s];
    }
    for (int64_t r = 0; r < n; ++r) {
        int64_t s = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (s < 0 || s >= nseq || h < 0 || h >= Hq || i < 0 || i >= cu_q[s + 1] - cu_q[s])
            return -1;
    }
    int grp = Hq / Hkv;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)(maxk > 0 ? maxk : 1));
        if (!scores) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < n; ++r) {
                int64_t s = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
                int64_t hk = h / grp;
                int64_t sq = cu_q[s + 1] - cu_q[s], skv = cu_k[s + 1] - cu_k[s];
                int64_t lim = causal ? i + (skv - sq) + 1 : skv;
                int n_ok = (int)(lim < 0 ? 0 : (lim > skv ? skv : lim));
                const uint16_t *qr = q + (((int64_t)cu_q[s] + i) * Hq + h) * d;
                const uint16_t *k0 = k + ((int64_t)cu_k[s] * Hkv + hk) * d;
                const uint16_t *v0 = v + ((int64_t)cu_k[s] * Hkv + hk) * d;
                one_row(qr, k0, v0, (int64_t)Hkv * d, n_ok, d, scale, scores,
                        o + r * d, lse + r);
            }
            free(scores);
        }
    }
    return err ? -1 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_num_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        t = omp_get_num_threads();
    }
    return t;
#else
    (void)nthreads;
    return 1;
#endif
}
