/*
 * Drives the C oracle (oracle/oracle_cpu.c) through its edge cases under
 * AddressSanitizer and UndefinedBehaviorSanitizer (built by
 * tests/test_host_sanitizers.py): rows with no allowed key, empty ragged
 * sequences, more query rows than keys under the bottom-right causal mask,
 * grouped heads, out-of-range row requests, 1 and 4 OpenMP threads.  Values
 * are checked against closed forms: a row that sees one key returns that
 * key's value row and LSE = scale * q.k; a row whose scores are all zero
 * returns the mean of the value rows it sees and LSE = log(count).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int Hq,
                     int Hkv, int Sq, int Skv, int d, double scale, int causal,
                     const int64_t *rows, int64_t n, double *o, double *lse, int nthreads);
int oracle_attn_varlen_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const int32_t *cu_q, const int32_t *cu_k, int nseq, int Hq, int Hkv,
                            int d, double scale, int causal, const int64_t *rows, int64_t n,
                            double *o, double *lse, int nthreads);

static int g_checks = 0, g_fail = 0;
#define CHECK(cond)                                                         \
    do {                                                                    \
        ++g_checks;                                                         \
        if (!(cond)) {                                                      \
            ++g_fail;                                                       \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);       \
        }                                                                   \
    } while (0)

/* bf16 bits of small integers and halves (exact in bf16) */
static uint16_t bf(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return (uint16_t)(u >> 16);
}
static double val(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

int main(void) {
    enum { B = 2, Hq = 4, Hkv = 2, Sq = 5, Skv = 3, D = 8 };
    static uint16_t q[B * Sq * Hq * D], k[B * Skv * Hkv * D], v[B * Skv * Hkv * D];
    srand(7);
    for (int i = 0; i < B * Sq * Hq * D; ++i) q[i] = bf((float)(rand() % 9 - 4) * 0.5f);
    for (int i = 0; i < B * Skv * Hkv * D; ++i) k[i] = bf((float)(rand() % 9 - 4) * 0.5f);
    for (int i = 0; i < B * Skv * Hkv * D; ++i) v[i] = bf((float)(rand() % 9 - 4));
    const double scale = 0.25;

    /* every row of the fixed batch, causal with Sq > Skv: rows 0, 1 see no
     * key, row 2 sees exactly key 0 */
    int64_t rows[B * Hq * Sq * 3];
    int64_t n = 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h)
            for (int i = 0; i < Sq; ++i) {
                rows[3 * n] = b, rows[3 * n + 1] = h, rows[3 * n + 2] = i;
                ++n;
            }
    double o1[B * Hq * Sq * D], l1[B * Hq * Sq], o4[B * Hq * Sq * D], l4[B * Hq * Sq];
    CHECK(oracle_attn_rows(q, k, v, B, Hq, Hkv, Sq, Skv, D, scale, 1, rows, n, o1, l1, 1) == 0);
    CHECK(oracle_attn_rows(q, k, v, B, Hq, Hkv, Sq, Skv, D, scale, 1, rows, n, o4, l4, 4) == 0);
    CHECK(memcmp(o1, o4, sizeof o1) == 0 && memcmp(l1, l4, sizeof l1) == 0);
    for (int64_t r = 0; r < n; ++r) {
        const int b = (int)rows[3 * r], h = (int)rows[3 * r + 1], i = (int)rows[3 * r + 2];
        const int hk = h / (Hq / Hkv);
        if (i < 2) {
            CHECK(isinf(l1[r]) && l1[r] < 0);
            for (int c = 0; c < D; ++c) CHECK(o1[r * D + c] == 0.0);
        } else if (i == 2) {
            double dot = 0;
            for (int c = 0; c < D; ++c)
                dot += val(q[((b * Sq + i) * Hq + h) * D + c]) * val(k[((b * Skv) * Hkv + hk) * D + c]);
            CHECK(fabs(l1[r] - scale * dot) < 1e-12);
            for (int c = 0; c < D; ++c)
                CHECK(o1[r * D + c] == val(v[((b * Skv) * Hkv + hk) * D + c]));
        }
    }
    /* zero queries: uniform weights over the allowed keys */
    static uint16_t qz[B * Sq * Hq * D];
    double oz[B * Hq * Sq * D], lz[B * Hq * Sq];
    CHECK(oracle_attn_rows(qz, k, v, B, Hq, Hkv, Sq, Skv, D, scale, 0, rows, n, oz, lz, 0) == 0);
    for (int64_t r = 0; r < n; ++r) {
        const int b = (int)rows[3 * r], hk = (int)rows[3 * r + 1] / (Hq / Hkv);
        CHECK(fabs(lz[r] - log((double)Skv)) < 1e-12);
        for (int c = 0; c < D; ++c) {
            double m = 0;
            for (int j = 0; j < Skv; ++j) m += val(v[((b * Skv + j) * Hkv + hk) * D + c]);
            CHECK(fabs(oz[r * D + c] - m / Skv) < 1e-12);
        }
    }
    /* bad arguments and rows out of range */
    int64_t bad[3] = {0, Hq, 0}, bad2[3] = {0, 0, Sq};
    CHECK(oracle_attn_rows(q, k, v, B, Hq, Hkv, Sq, Skv, D, scale, 0, bad, 1, o1, l1, 1) == -1);
    CHECK(oracle_attn_rows(q, k, v, B, Hq, Hkv, Sq, Skv, D, scale, 0, bad2, 1, o1, l1, 1) == -1);
    CHECK(oracle_attn_rows(q, k, v, B, 3, Hkv, Sq, Skv, D, scale, 0, rows, 1, o1, l1, 1) == -1);
    CHECK(oracle_attn_rows(q, k, v, B, Hq, Hkv, Sq, Skv, D, scale, 0, rows, 0, o1, l1, 1) == 0);

    /* ragged: sequence 1 has no queries, sequence 2 no keys, sequence 3 more
     * queries than keys */
    const int32_t cq[5] = {0, 2, 2, 5, 9}, ck[5] = {0, 3, 6, 6, 8};
    static uint16_t vq[9 * Hq * D], vk[8 * Hkv * D], vv[8 * Hkv * D];
    for (int i = 0; i < 9 * Hq * D; ++i) vq[i] = bf((float)(rand() % 7 - 3) * 0.5f);
    for (int i = 0; i < 8 * Hkv * D; ++i) vk[i] = bf((float)(rand() % 7 - 3) * 0.5f);
    for (int i = 0; i < 8 * Hkv * D; ++i) vv[i] = bf((float)(rand() % 7 - 3));
    int64_t vr[9 * Hq * 3];
    int64_t vn = 0;
    const int seq_of[9] = {0, 0, 2, 2, 2, 3, 3, 3, 3};
    for (int t = 0; t < 9; ++t)
        for (int h = 0; h < Hq; ++h) {
            vr[3 * vn] = seq_of[t], vr[3 * vn + 1] = h, vr[3 * vn + 2] = t - cq[seq_of[t]];
            ++vn;
        }
    double vo[9 * Hq * D], vl[9 * Hq], vo4[9 * Hq * D], vl4[9 * Hq];
    for (int causal = 0; causal < 2; ++causal) {
        CHECK(oracle_attn_varlen_rows(vq, vk, vv, cq, ck, 4, Hq, Hkv, D, scale, causal, vr, vn,
                                      vo, vl, 1) == 0);
        CHECK(oracle_attn_varlen_rows(vq, vk, vv, cq, ck, 4, Hq, Hkv, D, scale, causal, vr, vn,
                                      vo4, vl4, 4) == 0);
        CHECK(memcmp(vo, vo4, sizeof vo) == 0 && memcmp(vl, vl4, sizeof vl) == 0);
        for (int64_t r = 0; r < vn; ++r) {
            const int s = (int)vr[3 * r], i = (int)vr[3 * r + 2];
            /* sequence 2: no keys; sequence 3 (4 queries, 2 keys) causal:
             * local rows 0, 1 see none, row 2 sees key 0 only */
            const int none = s == 2 || (causal && s == 3 && i < 2);
            if (none) {
                CHECK(isinf(vl[r]) && vl[r] < 0);
                for (int c = 0; c < D; ++c) CHECK(vo[r * D + c] == 0.0);
            } else {
                CHECK(isfinite(vl[r]));
            }
            if (causal && s == 3 && i == 2) {
                const int hk = (int)vr[3 * r + 1] / (Hq / Hkv);
                for (int c = 0; c < D; ++c) CHECK(vo[r * D + c] == val(vv[(6 * Hkv + hk) * D + c]));
            }
        }
    }
    const int32_t cbad[3] = {0, 3, 2};
    int64_t one[3] = {0, 0, 0}, past[3] = {1, 0, 0};
    CHECK(oracle_attn_varlen_rows(vq, vk, vv, cq, cbad, 2, Hq, Hkv, D, scale, 0, one, 1, vo, vl,
                                  1) == -1);
    CHECK(oracle_attn_varlen_rows(vq, vk, vv, cq, ck, 4, Hq, Hkv, D, scale, 0, past, 1, vo, vl,
                                  1) == -1);   /* sequence 1 has no rows */
    printf("oracle: %d checks, %d failed\n", g_checks, g_fail);
    return g_fail ? 1 : 0;
}
