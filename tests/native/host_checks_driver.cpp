// Drives every host-side argument check and sizing function of the C ABI
// through its edge cases (sizes at the int limits, overflowing products,
// NULL and misaligned pointers, malformed offsets), checking each result.
// Built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py, so that any overflow, out-of-bounds read or
// undefined shift in these paths aborts the run.  Pointers are only compared
// and tested for alignment here, never dereferenced (except offset arrays).
#include <limits.h>
#include <math.h>
#include <stdio.h>

#include "fastdiv.h"
#include "host_checks.h"

using namespace attn::host;

static int g_checks = 0, g_fail = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        ++g_checks;                                                   \
        if (!(cond)) {                                                \
            ++g_fail;                                                 \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond); \
        }                                                             \
    } while (0)

alignas(64) static char buf[256];

int main() {
    const void *p = buf, *mis = buf + 2;   // 16-byte aligned, and not
    const float *lse = (const float *)(buf + 64);
    const int IM = INT_MAX;

    // ceil_div at the top of the int range
    CHECK(ceil_div(0, 7) == 0);
    CHECK(ceil_div(IM, 1) == IM);
    CHECK(ceil_div(IM, 2) == 1073741824);
    CHECK(ceil_div(IM, 256) == 8388608);
    CHECK(ceil_div(IM - 64, 32) == 67108862);
    CHECK(d_ok(64) && d_ok(128) && !d_ok(96) && !d_ok(0));
    CHECK(scale_ok(0.1f) && !scale_ok(0.f) && !scale_ok(-1.f) && !scale_ok(NAN) &&
          !scale_ok(INFINITY));

    // the kernels' division by launch-fixed divisors: every divisor up to
    // 70000 and powers of two and their neighbours up to 2^31 - 1, against
    // numerators at the edges (0, multiples of d and their neighbours, the
    // top of the 31-bit range) and a spread in between
    {
        long long bad = 0;
        auto check_d = [&](uint32_t d) {
            const attn::FastDiv f = attn::make_fastdiv(d);
            auto one = [&](uint32_t n) {
                if (attn::fastdiv_apply(n, f) != n / d) ++bad;
            };
            for (uint32_t n = 0; n < 2048; ++n) one(n);
            for (uint64_t k = 1; k * d < 0x7fffffffull && k < 4096; k = k * 3 + 1) {
                const uint32_t n = (uint32_t)(k * d);
                one(n - 1);
                one(n);
                if (n + 1 <= 0x7fffffffu) one(n + 1);
            }
            for (uint32_t n = 0x7fffffffu; n > 0x7fffffffu - 4096; --n) one(n);
            uint32_t x = d * 2654435761u;
            for (int i = 0; i < 64; ++i) {
                x = x * 1664525u + 1013904223u;
                one(x & 0x7fffffffu);
            }
        };
        for (uint32_t d = 1; d <= 70000; ++d) check_d(d);
        for (int e = 17; e <= 31; ++e)
            for (long long dd = (1ll << e) - 3; dd <= (1ll << e) + 3; ++dd)
                if (dd >= 1 && dd < 0x7fffffffll) check_d((uint32_t)dd);
        check_d(0x7ffffffeu);
        CHECK(bad == 0);
    }

    // decode sizing: split counts stay in [1, keys / 512] and chunks in int
    for (int skv : {1, 31, 32, 33, 511, 512, 4096, 1 << 20, IM - 64}) {
        for (int b : {1, 7, 64, 1 << 16}) {
            const int s = pick_splits(b, 32, 8, skv);
            CHECK(s >= 1 && s <= ceil_div(skv, 512));
            const DecodeShape sh = decode_shape(b, 32, 8, skv, 0);
            CHECK(sh.nsplit == s && sh.chunk % 32 == 0 && sh.chunk >= 32 && sh.ncb == 1);
            CHECK((long long)sh.chunk * sh.nsplit >= skv);
        }
    }
    CHECK(decode_shape(1, 256, 1, IM - 64, 1).chunk == 2147483584);
    CHECK(decode_shape(1, 256, 1, 100, 7).ncb == 8);
    CHECK(decode_ws_bytes(1, 1, 128, 1) == 0);
    CHECK(decode_ws_bytes(65536, 256, 128, 65536) ==
          (size_t)65536 * 65536 * 256 * 129 * sizeof(float));
    // split by the lengths: eligibility (list size, tile positions in an
    // int with room for the runs), header and workspace bytes
    CHECK(decode_list_ok(64, 32, 8, 32768) && decode_list_ok(1, 1, 1, 1));
    CHECK(decode_list_ok(2048, 64, 1, 1024) && !decode_list_ok(2049, 64, 1, 1024));
    CHECK(!decode_list_ok(2048, 8, 1, IM - 64) && !decode_list_ok(2048, 256, 1, 1 << 22));
    CHECK(decode_list_ok(2048, 256, 1, 1 << 20));
    CHECK(decode_list_ok(1, 1, 1, IM - 64));
    CHECK(decode_list_hdr_bytes(1) == 32 && decode_list_hdr_bytes(3) == 32 &&
          decode_list_hdr_bytes(4) == 48 && decode_list_hdr_bytes(2048) == 16 + 8208);
    CHECK(decode_list_ws_bytes(64, 32, 8, 128) ==
          decode_list_hdr_bytes(64) + (size_t)(64 * 32 + 1024 * 4) * 129 * sizeof(float));
    CHECK(decode_list_ws_bytes(2048, 256, 1, 128) ==
          decode_list_hdr_bytes(2048) + (size_t)(2048 * 256 + 1024 * 32) * 129 * sizeof(float));
    CHECK(decode_sizes_ok(64, 32, 8, 4096, 128));
    CHECK(!decode_sizes_ok(64, 32, 8, IM, 128) && !decode_sizes_ok(0, 32, 8, 4096, 128));
    CHECK(!decode_sizes_ok(IM, IM, IM, IM - 64, 128));

    // decode argument checks, one failure at a time, in their fixed order
    const Fp8Scales f8{0.5f, 2.f}, f8bad{0.5f, NAN}, f8huge{1e30f, 1.f};
    CHECK(decode_args_status(p, p, p, p, lse, 64, 32, 8, 4096, 128, 0.09f, 0, nullptr) == ATTN_OK);
    CHECK(decode_args_status(p, p, p, p, nullptr, 64, 32, 8, 4096, 128, 0.09f, 8, &f8) == ATTN_OK);
    CHECK(decode_args_status(nullptr, p, p, p, lse, 64, 32, 8, 4096, 128, 0.09f, 0, nullptr) ==
          ATTN_ERR_NULLPTR);
    CHECK(decode_args_status(p, p, p, p, lse, 0, 32, 8, 4096, 128, 0.09f, 0, nullptr) ==
          ATTN_ERR_SHAPE);
    CHECK(decode_args_status(p, p, p, p, lse, 64, 32, 8, IM, 128, 0.09f, 0, nullptr) ==
          ATTN_ERR_SHAPE);
    CHECK(decode_args_status(p, p, p, p, lse, 64, 32, 8, 4096, 96, 0.09f, 0, nullptr) ==
          ATTN_ERR_UNSUPPORTED_D);
    CHECK(decode_args_status(p, p, p, p, lse, 64, 30, 8, 4096, 128, 0.09f, 0, nullptr) ==
          ATTN_ERR_GQA_RATIO);
    CHECK(decode_args_status(p, p, p, p, lse, 64, 32, 8, 4096, 128, NAN, 0, nullptr) ==
          ATTN_ERR_SCALE);
    CHECK(decode_args_status(p, p, p, p, lse, 64, 32, 8, 4096, 128, 0.09f, 0, &f8bad) ==
          ATTN_ERR_SCALE);
    CHECK(decode_args_status(p, p, p, p, lse, 64, 32, 8, 4096, 128, 1e30f, 0, &f8huge) ==
          ATTN_ERR_SCALE);
    CHECK(decode_args_status(p, p, p, p, lse, 64, 32, 8, 4096, 128, 0.09f, 70000, nullptr) ==
          ATTN_ERR_SHAPE);
    CHECK(decode_args_status(mis, p, p, p, lse, 64, 32, 8, 4096, 128, 0.09f, 0, nullptr) ==
          ATTN_ERR_ALIGNMENT);
    CHECK(decode_args_status(p, p, p, p, (const float *)(buf + 1), 64, 32, 8, 4096, 128, 0.09f,
                             0, nullptr) == ATTN_ERR_ALIGNMENT);
    // work items past the int range: B * Hkv * blocks * splits
    CHECK(decode_args_status(p, p, p, p, lse, 1 << 16, 1 << 10, 1 << 10, 1 << 8, 64, 0.09f,
                             65536, nullptr) == ATTN_ERR_SHAPE);
    CHECK(workspace_status(nullptr, 0, 0) == ATTN_OK);
    CHECK(workspace_status(nullptr, 100, 16) == ATTN_ERR_WORKSPACE);
    CHECK(workspace_status(p, 15, 16) == ATTN_ERR_WORKSPACE);
    CHECK(workspace_status(mis, 64, 16) == ATTN_ERR_ALIGNMENT);
    CHECK(workspace_status(p, 16, 16) == ATTN_OK);

    // split-KV prefill sizing
    CHECK(fwd_pick_splits(1, 1, 1, 1, false) == 1);
    CHECK(fwd_pick_splits(1, 32, 512, 8192, false) >= 2);
    CHECK(fwd_pick_splits(1, 1, IM, IM, true) >= 1);
    CHECK(fwd_pick_splits(1, 1, IM, 1, true) == 1);
    CHECK(fwd_ws_bytes(1, 1, 1, 128, 1) == 0);
    CHECK(fwd_ws_bytes(2, 3, 5, 64, 4) == (size_t)4 * 2 * 3 * 5 * 65 * sizeof(float));

    // fixed-batch prefill checks
    int nt = -1;
    CHECK(fwd_args_status(p, p, p, p, lse, 4, 16, 16, 2048, 2048, 128, 0.09f, &nt) == ATTN_OK &&
          nt == 8);
    CHECK(fwd_args_status(p, p, p, p, nullptr, 1, 1, 1, 257, 1, 64, 0.09f, &nt) == ATTN_OK &&
          nt == 2);
    CHECK(fwd_args_status(p, nullptr, p, p, lse, 4, 16, 16, 2048, 2048, 128, 0.09f, &nt) ==
          ATTN_ERR_NULLPTR);
    CHECK(fwd_args_status(p, p, p, p, lse, 4, 16, 16, 0, 2048, 128, 0.09f, &nt) ==
          ATTN_ERR_SHAPE);
    CHECK(fwd_args_status(p, p, p, p, lse, IM, IM, 1, IM, 1, 128, 0.09f, &nt) == ATTN_ERR_SHAPE);
    CHECK(fwd_args_status(p, p, p, p, lse, 4, 16, 16, 2048, 2048, 80, 0.09f, &nt) ==
          ATTN_ERR_UNSUPPORTED_D);
    CHECK(fwd_args_status(p, p, p, p, lse, 4, 16, 3, 2048, 2048, 128, 0.09f, &nt) ==
          ATTN_ERR_GQA_RATIO);
    CHECK(fwd_args_status(p, p, p, p, lse, 4, 16, 16, 2048, 2048, 128, -0.5f, &nt) ==
          ATTN_ERR_SCALE);
    CHECK(fwd_args_status(p, p, mis, p, lse, 4, 16, 16, 2048, 2048, 128, 0.09f, &nt) ==
          ATTN_ERR_ALIGNMENT);
    // tiles * B * Hq past the int range while every tensor stays under the cap
    CHECK(fwd_args_status(p, p, p, p, lse, 1 << 16, 1 << 16, 1, 1, 1, 64, 0.09f, &nt) ==
          ATTN_ERR_SHAPE);

    // ragged-batch prefill checks
    alignas(4) static int cu[5] = {0, 3, 3, 10, 12};
    CHECK(varlen_args_status(p, p, p, p, lse, cu, cu, 4, 12, 12, 7, 7, 8, 2, 128, 0.09f, &nt) ==
          ATTN_OK && nt == 1);
    CHECK(varlen_args_status(p, p, p, p, lse, nullptr, cu, 4, 12, 12, 7, 7, 8, 2, 128, 0.09f,
                             &nt) == ATTN_ERR_NULLPTR);
    CHECK(varlen_args_status(p, p, p, p, lse, cu, cu, IM, 12, 12, 7, 7, 8, 2, 128, 0.09f, &nt) ==
          ATTN_ERR_SHAPE);
    CHECK(varlen_args_status(p, p, p, p, lse, cu, cu, 4, 12, 12, 13, 7, 8, 2, 128, 0.09f, &nt) ==
          ATTN_ERR_SEQLENS);
    CHECK(varlen_args_status(p, p, p, p, lse, (const int *)(buf + 2), cu, 4, 12, 12, 7, 7, 8, 2,
                             128, 0.09f, &nt) == ATTN_ERR_ALIGNMENT);
    CHECK(varlen_args_status(p, p, p, p, lse, cu, cu, 1 << 20, IM, IM, IM, IM, 1 << 10, 1, 64,
                             0.09f, &nt) == ATTN_ERR_SHAPE);
    int mx = -1;
    CHECK(varlen_check(cu, 4, 12, &mx) == ATTN_OK && mx == 7);
    CHECK(varlen_check(cu, 4, 12, nullptr) == ATTN_OK);
    CHECK(varlen_check(cu, 4, 11, &mx) == ATTN_ERR_SEQLENS);
    CHECK(varlen_check(cu, 0, 0, &mx) == ATTN_ERR_SEQLENS);
    CHECK(varlen_check(nullptr, 4, 12, &mx) == ATTN_ERR_NULLPTR);
    alignas(4) static int dec[4] = {0, 5, 4, 9}, nz[3] = {1, 2, 3};
    alignas(4) static int big[3] = {0, IM - 1, IM};
    CHECK(varlen_check(dec, 3, 9, &mx) == ATTN_ERR_SEQLENS);
    CHECK(varlen_check(nz, 2, 3, &mx) == ATTN_ERR_SEQLENS);
    CHECK(varlen_check(big, 2, IM, &mx) == ATTN_OK && mx == IM - 1);

    // paged-cache extras and k-means
    CHECK(paged_args_status(cu, cu, 4, 8, 128, 16, 4, 64) == ATTN_OK);
    CHECK(paged_args_status(nullptr, cu, 4, 8, 128, 16, 4, 64) == ATTN_ERR_NULLPTR);
    CHECK(paged_args_status(cu, cu, 4, 8, 128, 8, 4, 64) == ATTN_ERR_SHAPE);
    CHECK(paged_args_status(cu, cu, 4, 8, 128, 24, 4, 64) == ATTN_ERR_SHAPE);
    CHECK(paged_args_status(cu, cu, 4, 8, 128, 1 << 16, 1 << 16, 64) == ATTN_ERR_SHAPE);
    CHECK(paged_args_status(cu, cu, IM, 8, 128, 16, 4, 64) == ATTN_ERR_SHAPE);
    CHECK(paged_args_status(cu, cu, 4, IM, IM, 16, 4, IM) == ATTN_ERR_SHAPE);
    CHECK(paged_args_status(cu, (const int *)(buf + 1), 4, 8, 128, 16, 4, 64) ==
          ATTN_ERR_ALIGNMENT);
    CHECK(kmeans_args_status(p, p, cu, lse, 1000, 16, 128) == ATTN_OK);
    CHECK(kmeans_args_status(p, p, nullptr, lse, 1000, 16, 128) == ATTN_ERR_NULLPTR);
    CHECK(kmeans_args_status(p, p, cu, lse, 0, 16, 128) == ATTN_ERR_SHAPE);
    CHECK(kmeans_args_status(p, p, cu, lse, IM, IM, 128) == ATTN_OK);   // 2^38 elements
    CHECK(kmeans_args_status(p, p, cu, lse, IM, 16, IM) == ATTN_ERR_SHAPE);
    CHECK(kmeans_args_status(p, p, cu, lse, 1000, 16, 32) == ATTN_ERR_UNSUPPORTED_D);
    CHECK(kmeans_args_status(mis, p, cu, lse, 1000, 16, 128) == ATTN_ERR_ALIGNMENT);

    // the bounded product itself
    CHECK(prod_le(10, {2, 5}) && !prod_le(10, {11}) && !prod_le(10, {2, 3, 2}));
    CHECK(prod_le(kMaxElems, {IM, IM, IM, 0}) && !prod_le(kMaxElems, {IM, IM, IM, IM}));
    CHECK(!prod_le(0x7fffffff, {-1, 1}) && prod_le(0x7fffffff, {}));

    printf("host checks: %d checks, %d failed\n", g_checks, g_fail);
    return g_fail ? 1 : 0;
}
