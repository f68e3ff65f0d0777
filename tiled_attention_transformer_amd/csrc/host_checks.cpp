// Host-side argument checks and sizing of the C ABI (see host_checks.h).
// Plain C++: built into libattn.so, and on its own under the host
// sanitizers by the tests.
#include "host_checks.h"

#include <math.h>

#include <initializer_list>

#include "tile_config.h"

namespace attn {
namespace host {

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool d_ok(int d) { return d == 64 || d == 128; }

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

// a / b rounded up, for a >= 0 and b >= 1 (no intermediate a + b - 1,
// which overflows for a near INT_MAX)
int ceil_div(int a, int b) { return a / b + (a % b != 0); }

// Whether the product of non-negative factors is at most lim (lim >= 0),
// without forming any product above lim: four int factors near INT_MAX
// would overflow even int64.
bool prod_le(int64_t lim, std::initializer_list<int64_t> factors) {
    for (const int64_t f : factors)
        if (f < 0) return false;
    for (const int64_t f : factors)
        if (f == 0) return true;
    int64_t acc = 1;
    for (const int64_t f : factors) {
        if (acc > lim / f) return false;
        acc *= f;
    }
    return true;
}

int pick_splits(int B, int Hq, int Hkv, int Skv) {
    // About one work item per compute unit (an MI355X has 256), but chunks of
    // at least 512 keys.  Measured on the decode kernels: more, shorter
    // chunks spend their time in per-item setup and in the merge of the
    // partials, fewer leave compute units idle.  Then balance: the workers
    // (the 256 workgroups, or the 1024 waves once there are that many split
    // items) take the items in rounds, and a last round that is mostly empty
    // leaves the GPU idle for its length (384 groups: 1.5 items per
    // workgroup, the second round half empty); of s0 .. max(2 s0, s0 + 3)
    // chunks the one with the fullest rounds wins, if it fills them by 0.15
    // more than s0.
    const int ncb = ceil_div(Hq / Hkv, kDecCols);
    const int64_t base = (int64_t)B * Hkv * ncb;
    const int64_t max_by_len = ceil_div(Skv, 512);
    int64_t s0 = (256 + base - 1) / base;
    if (s0 > max_by_len) s0 = max_by_len;
    if (s0 < 1) s0 = 1;
    auto fill = [&](int64_t s) {
        const int64_t items = base * s;
        const int64_t workers = (s > 1 && items >= 1024) ? 1024 : 256;
        const int64_t rounds = (items + workers - 1) / workers;
        return (double)items / (double)(rounds * workers);
    };
    int64_t best = s0;
    double fbest = fill(s0);
    const double f0 = fbest;
    const int64_t s_hi = 2 * s0 > s0 + 3 ? 2 * s0 : s0 + 3;
    for (int64_t s = s0 + 1; s <= s_hi && s <= max_by_len; ++s) {
        const double f = fill(s);
        if (f > fbest) {
            best = s;
            fbest = f;
        }
    }
    return (int)(fbest >= f0 + 0.15 ? best : s0);
}

DecodeShape decode_shape(int B, int Hq, int Hkv, int Skv, int num_splits) {
    DecodeShape sh;
    sh.nsplit = num_splits > 0 ? num_splits : pick_splits(B, Hq, Hkv, Skv);
    // chunks start on 32-key boundaries, so a kernel tile (32 keys, read as
    // two 16-key halves) never straddles a 16-key boundary -- in a paged
    // cache, never a page boundary; trailing chunks may be empty
    sh.chunk = ceil_div(ceil_div(Skv, sh.nsplit), 32) * 32;
    sh.ncb = ceil_div(Hq / Hkv, kDecCols);
    return sh;
}

size_t decode_ws_bytes(int B, int Hq, int d, int nsplit) {
    if (nsplit <= 1) return 0;
    const size_t o_bytes = (size_t)nsplit * B * Hq * d * sizeof(float);
    const size_t l_bytes = (size_t)nsplit * B * Hq * sizeof(float);
    return o_bytes + l_bytes;
}

bool decode_sizes_ok(int B, int Hq, int Hkv, int Skv, int d) {
    // Skv leaves room for the chunk rounding to 32 keys in an int
    return B >= 1 && Hq >= 1 && Hkv >= 1 && Skv >= 1 && d >= 1 && Skv <= 0x7fffffff - 64 &&
           prod_le(kMaxElems, {B, Skv, Hkv, d}) && prod_le(kMaxElems, {B, Hq, d});
}

attn_status_t decode_args_status(const void *q, const void *k_cache, const void *v_cache,
                                 const void *o, const float *lse, int B, int Hq, int Hkv, int Skv,
                                 int d, float scale, int num_splits, const Fp8Scales *fp8) {
    if (!q || !k_cache || !v_cache || !o) return ATTN_ERR_NULLPTR;
    if (!decode_sizes_ok(B, Hq, Hkv, Skv, d)) return ATTN_ERR_SHAPE;
    if (!d_ok(d)) return ATTN_ERR_UNSUPPORTED_D;
    if (Hq % Hkv) return ATTN_ERR_GQA_RATIO;
    if (!scale_ok(scale)) return ATTN_ERR_SCALE;
    if (fp8 && (!scale_ok(fp8->k_scale) || !scale_ok(fp8->v_scale) ||
                !scale_ok(scale * fp8->k_scale)))
        return ATTN_ERR_SCALE;
    if (num_splits > 65536) return ATTN_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
        (lse && !aligned(lse, 4)))
        return ATTN_ERR_ALIGNMENT;
    const DecodeShape sh = decode_shape(B, Hq, Hkv, Skv, num_splits);
    if (!prod_le(0x7fffffff, {B, Hkv, sh.ncb, sh.nsplit})) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

bool decode_list_ok(int B, int Hq, int Hkv, int Skv) {
    // a list that fits the kernel's LDS, and tile positions (sequences x
    // 32-key tiles x KV heads x query blocks, plus a run per wave) in an int
    const int ncb = ceil_div(Hq / Hkv, kDecCols);
    return B <= kDecListSeqs &&
           prod_le(0x7fffffff - (1 << 20), {B, ceil_div(Skv, 32), Hkv, ncb});
}

size_t decode_list_ws_bytes(int B, int Hq, int Hkv, int d) {
    // header (run length, per-sequence offsets), then fp32 partials and
    // their LSE values: a row per (sequence, query head) and ncm per wave
    const int ncm = Hq / Hkv < kDecCols ? Hq / Hkv : kDecCols;
    const size_t rows = (size_t)B * Hq + (size_t)kDecListWGs * 4 * ncm;
    return decode_list_hdr_bytes(B) + rows * (size_t)(d + 1) * sizeof(float);
}

size_t decode_list_hdr_bytes(int B) { return 16 + ((size_t)4 * (B + 1) + 15) / 16 * 16; }

attn_status_t workspace_status(const void *workspace, size_t workspace_bytes, size_t need) {
    if (need == 0) return ATTN_OK;
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_ALIGNMENT;
    return ATTN_OK;
}

// Split-KV prefill: about one work item per compute unit (an MI355X has
// 256), but shares that average at least 1024 keys: the shares' partial
// outputs cost a write and a read of fp32 rows, which only pays when each
// share still streams many key tiles.  Measured (d = 128): a 512-token chunk
// against 8192 keys splits 4 ways (2.3x faster), 256 tokens against 16384
// keys 8 ways (4.4x), a causal 4096-token prefill with 8 heads 2 ways
// (1.4x); a 1024-token prefill with 32 heads is faster unsplit, causal or
// not.
int fwd_pick_splits(int B, int Hq, int Sq, int Skv, bool causal) {
    const int64_t base = (int64_t)B * Hq * ceil_div(Sq, kFwdBr);
    int64_t s = (256 + base - 1) / base;
    // keys a query row sees on average (bottom-right causal alignment)
    int64_t avg = Skv;
    if (causal) avg = Sq <= Skv ? Skv - Sq / 2 : (int64_t)Skv * Skv / (2 * (int64_t)Sq);
    const int64_t cap = avg / 1024;
    if (s > cap) s = cap;
    return s < 1 ? 1 : (int)s;
}

size_t fwd_ws_bytes(int B, int Hq, int Sq, int d, int nsplit) {
    if (nsplit <= 1) return 0;
    return (size_t)nsplit * B * Hq * Sq * (d + 1) * sizeof(float);
}

attn_status_t fwd_args_status(const void *q, const void *k, const void *v, const void *o,
                              const float *lse, int B, int Hq, int Hkv, int Sq, int Skv, int d,
                              float scale, int *ntiles) {
    if (!q || !k || !v || !o) return ATTN_ERR_NULLPTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || d < 1) return ATTN_ERR_SHAPE;
    if (!prod_le(kMaxElems, {B, Sq, Hq, d}) || !prod_le(kMaxElems, {B, Skv, Hkv, d}))
        return ATTN_ERR_SHAPE;
    if (!d_ok(d)) return ATTN_ERR_UNSUPPORTED_D;
    if (Hq % Hkv) return ATTN_ERR_GQA_RATIO;
    if (!scale_ok(scale)) return ATTN_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        (lse && !aligned(lse, 4)))
        return ATTN_ERR_ALIGNMENT;
    const int nt = ceil_div(Sq, kFwdBr);
    if (!prod_le(0x7fffffff, {nt, B, Hq})) return ATTN_ERR_SHAPE;
    *ntiles = nt;
    return ATTN_OK;
}

attn_status_t varlen_args_status(const void *q, const void *k, const void *v, const void *o,
                                 const float *lse, const int *cu_q, const int *cu_k, int nseq,
                                 int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                                 int Hq, int Hkv, int d, float scale, int *ntiles) {
    if (!q || !k || !v || !o || !cu_q || !cu_k) return ATTN_ERR_NULLPTR;
    if (nseq < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 ||
        Hq < 1 || Hkv < 1 || d < 1)
        return ATTN_ERR_SHAPE;
    if (nseq == 0x7fffffff) return ATTN_ERR_SHAPE;   // nseq + 1 offsets must fit an int
    if (max_seqlen_q > total_q || max_seqlen_k > total_k) return ATTN_ERR_SEQLENS;
    if (!prod_le(kMaxElems, {total_q, Hq, d}) || !prod_le(kMaxElems, {total_k, Hkv, d}))
        return ATTN_ERR_SHAPE;
    if (!d_ok(d)) return ATTN_ERR_UNSUPPORTED_D;
    if (Hq % Hkv) return ATTN_ERR_GQA_RATIO;
    if (!scale_ok(scale)) return ATTN_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        (lse && !aligned(lse, 4)) || !aligned(cu_q, 4) || !aligned(cu_k, 4))
        return ATTN_ERR_ALIGNMENT;
    const int nt = ceil_div(max_seqlen_q, kFwdBr);
    if (!prod_le(0x7fffffff, {nt, nseq, Hq})) return ATTN_ERR_SHAPE;
    *ntiles = nt;
    return ATTN_OK;
}

attn_status_t varlen_check(const int *cu, int nseq, int total, int *max_seqlen) {
    if (!cu) return ATTN_ERR_NULLPTR;
    if (nseq < 1 || nseq == 0x7fffffff || total < 0 || cu[0] != 0 || cu[nseq] != total)
        return ATTN_ERR_SEQLENS;
    int mx = 0;
    for (int s = 0; s < nseq; ++s) {
        if (cu[s + 1] < cu[s]) return ATTN_ERR_SEQLENS;
        // non-decreasing from 0, so the difference cannot overflow
        if (cu[s + 1] - cu[s] > mx) mx = cu[s + 1] - cu[s];
    }
    if (max_seqlen) *max_seqlen = mx;
    return ATTN_OK;
}

attn_status_t paged_args_status(const int *block_table, const int *seqlens_k, int B, int Hkv,
                                int d, int page_size, int max_pages_per_seq, int num_pages) {
    if (!block_table || !seqlens_k) return ATTN_ERR_NULLPTR;
    if (page_size < 16 || page_size % 16 || max_pages_per_seq < 1 || num_pages < 1)
        return ATTN_ERR_SHAPE;
    if (!prod_le(0x7fffffff - 64, {max_pages_per_seq, page_size}) ||
        !prod_le(kMaxElems, {num_pages, page_size, Hkv, d}) ||
        !prod_le(0x7fffffff, {B, max_pages_per_seq}))
        return ATTN_ERR_SHAPE;
    if (!aligned(block_table, 4) || !aligned(seqlens_k, 4)) return ATTN_ERR_ALIGNMENT;
    return ATTN_OK;
}

attn_status_t kmeans_args_status(const void *x, const void *c, const int *idx, const float *dist,
                                 int N, int K, int d) {
    if (!x || !c || !idx) return ATTN_ERR_NULLPTR;
    if (N < 1 || K < 1 || !prod_le(kMaxElems, {N, d}) || !prod_le(kMaxElems, {K, d}))
        return ATTN_ERR_SHAPE;
    if (!d_ok(d)) return ATTN_ERR_UNSUPPORTED_D;
    if (!aligned(x, 16) || !aligned(c, 16) || !aligned(idx, 4) || (dist && !aligned(dist, 4)))
        return ATTN_ERR_ALIGNMENT;
    return ATTN_OK;
}

}  // namespace host
}  // namespace attn
