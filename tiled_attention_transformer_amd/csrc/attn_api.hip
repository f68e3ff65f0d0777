// C ABI of libattn.so (declared in include/attn.h): argument validation on
// the host, then the kernel launches.  No allocation, no global state.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/attn.h"
#include "kernels.h"

// Split partials of attn_decode_noalloc: a fixed array in device memory (one
// copy per GPU), so that entry point allocates nothing.  Host code never
// passes `scratch` itself (on the host the name is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;   // sanity cap on tensor sizes

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool d_ok(int d) { return d == 64 || d == 128; }

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

attn_status_t from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct DecodeShape {
    int nsplit, chunk, ncb;
};

int pick_splits(int B, int Hq, int Hkv, int Skv) {
    // About one work item per compute unit (an MI355X has 256), but chunks of
    // at least 512 keys.  Measured on the decode kernels: more, shorter
    // chunks spend their time in per-item setup and in the merge of the
    // partials, fewer leave compute units idle.
    const int ncb = ceil_div(Hq / Hkv, attn::kDecCols);
    const int64_t base = (int64_t)B * Hkv * ncb;
    int s = (int)((256 + base - 1) / base);
    const int max_by_len = ceil_div(Skv, 512);
    if (s > max_by_len) s = max_by_len;
    if (s < 1) s = 1;
    return s;
}

DecodeShape decode_shape(int B, int Hq, int Hkv, int Skv, int num_splits) {
    DecodeShape sh;
    sh.nsplit = num_splits > 0 ? num_splits : pick_splits(B, Hq, Hkv, Skv);
    // chunks start on 32-key boundaries, so a kernel tile (32 keys, read as
    // two 16-key halves) never straddles a 16-key boundary -- in a paged
    // cache, never a page boundary; trailing chunks may be empty
    sh.chunk = ceil_div(ceil_div(Skv, sh.nsplit), 32) * 32;
    sh.ncb = ceil_div(Hq / Hkv, attn::kDecCols);
    return sh;
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
    const int64_t base = (int64_t)B * Hq * ceil_div(Sq, attn::kFwdBr);
    int s = (int)((256 + base - 1) / base);
    // keys a query row sees on average (bottom-right causal alignment)
    int64_t avg = Skv;
    if (causal) avg = Sq <= Skv ? Skv - Sq / 2 : (int64_t)Skv * Skv / (2 * (int64_t)Sq);
    const int64_t cap = avg / 1024;
    if (s > cap) s = (int)cap;
    return s < 1 ? 1 : s;
}

size_t fwd_ws_bytes(int B, int Hq, int Sq, int d, int nsplit) {
    if (nsplit <= 1) return 0;
    return (size_t)nsplit * B * Hq * Sq * (d + 1) * sizeof(float);
}

attn_status_t fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                       int Hq, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                       int num_splits, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

size_t decode_ws_bytes(int B, int Hq, int d, int nsplit) {
    if (nsplit <= 1) return 0;
    const size_t o_bytes = (size_t)nsplit * B * Hq * d * sizeof(float);
    const size_t l_bytes = (size_t)nsplit * B * Hq * sizeof(float);
    return o_bytes + l_bytes;
}

bool decode_sizes_ok(int B, int Hq, int Hkv, int Skv, int d) {
    return B >= 1 && Hq >= 1 && Hkv >= 1 && Skv >= 1 && d >= 1 &&
           (int64_t)B * Skv * Hkv * d <= kMaxElems && (int64_t)B * Hq * d <= kMaxElems;
}

}  // namespace

extern "C" {

const char *attn_status_string(attn_status_t s) {
    switch (s) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULLPTR: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "a size is < 1 or too large";
        case ATTN_ERR_UNSUPPORTED_D: return "head dimension must be 64 or 128";
        case ATTN_ERR_GQA_RATIO: return "Hq must be a multiple of Hkv";
        case ATTN_ERR_ALIGNMENT: return "pointer not aligned (bf16 tensors 16 B, lse 4 B, workspace 16 B)";
        case ATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
        case ATTN_ERR_SEQLENS: return "malformed cumulative sequence offsets";
        case ATTN_ERR_HIP: return "HIP runtime error at launch";
        case ATTN_ERR_SCALE: return "scale must be finite and > 0";
        case ATTN_ERR_SCRATCH_LIMIT: return "the split partials need more than the fixed scratch of attn_decode_noalloc";
    }
    return "unknown status";
}

attn_status_t attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                       int Hq, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                       hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, scale, causal, 1, nullptr, 0, stream);
}

size_t attn_fwd_splitkv_workspace_bytes(int B, int Hq, int Sq, int Skv, int d, int causal,
                                        int num_splits) {
    if (B < 1 || Hq < 1 || Sq < 1 || Skv < 1 || !d_ok(d) || num_splits > 1024) return 0;
    if ((int64_t)B * Sq * Hq * d > kMaxElems) return 0;
    const int ns = num_splits > 0 ? num_splits : fwd_pick_splits(B, Hq, Sq, Skv, causal != 0);
    return fwd_ws_bytes(B, Hq, Sq, d, ns);
}

attn_status_t attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                               int B, int Hq, int Hkv, int Sq, int Skv, int d, float scale,
                               int causal, int num_splits, void *workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    if (num_splits > 1024) return ATTN_ERR_SHAPE;
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, scale, causal, num_splits, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"

namespace {

attn_status_t fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                       int Hq, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                       int num_splits, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    if (!q || !k || !v || !o) return ATTN_ERR_NULLPTR;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1 || d < 1) return ATTN_ERR_SHAPE;
    if ((int64_t)B * Sq * Hq * d > kMaxElems || (int64_t)B * Skv * Hkv * d > kMaxElems)
        return ATTN_ERR_SHAPE;
    if (!d_ok(d)) return ATTN_ERR_UNSUPPORTED_D;
    if (Hq % Hkv) return ATTN_ERR_GQA_RATIO;
    if (!scale_ok(scale)) return ATTN_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        (lse && !aligned(lse, 4)))
        return ATTN_ERR_ALIGNMENT;
    const int ntiles = ceil_div(Sq, attn::kFwdBr);
    if ((int64_t)ntiles * B * Hq > 0x7fffffff) return ATTN_ERR_SHAPE;
    attn::FwdParams p{};
    p.q = (const __bf16 *)q;
    p.k = (const __bf16 *)k;
    p.v = (const __bf16 *)v;
    p.o = (__bf16 *)o;
    p.lse = lse;
    p.nbatch = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.group = Hq / Hkv;
    p.Sq = Sq;
    p.Skv = Skv;
    p.ntiles = ntiles;
    p.c = scale * attn::kLog2e;
    const int ns = num_splits > 0 ? num_splits : fwd_pick_splits(B, Hq, Sq, Skv, causal != 0);
    if (ns <= 1) return from_hip(attn::launch_fwd(p, d, causal != 0, false, stream));
    const size_t need = fwd_ws_bytes(B, Hq, Sq, d, ns);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_ALIGNMENT;
    if ((int64_t)ntiles * B * Hq * ns > 0x7fffffff) return ATTN_ERR_SHAPE;
    p.nsplit = ns;
    p.ws_o = (float *)workspace;
    p.ws_lse = p.ws_o + (size_t)ns * B * Hq * Sq * d;
    return from_hip(attn::launch_fwd_split(p, d, causal != 0, stream));
}

}  // namespace

extern "C" {

attn_status_t attn_varlen_check(const int *cu, int nseq, int total, int *max_seqlen) {
    if (!cu) return ATTN_ERR_NULLPTR;
    if (nseq < 1 || total < 0 || cu[0] != 0 || cu[nseq] != total) return ATTN_ERR_SEQLENS;
    int mx = 0;
    for (int s = 0; s < nseq; ++s) {
        if (cu[s + 1] < cu[s]) return ATTN_ERR_SEQLENS;
        if (cu[s + 1] - cu[s] > mx) mx = cu[s + 1] - cu[s];
    }
    if (max_seqlen) *max_seqlen = mx;
    return ATTN_OK;
}

attn_status_t attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                              const int *cu_seqlens_q, const int *cu_seqlens_k, int nseq,
                              int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                              int Hq, int Hkv, int d, float scale, int causal,
                              hipStream_t stream) {
    if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k) return ATTN_ERR_NULLPTR;
    if (nseq < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 ||
        Hq < 1 || Hkv < 1 || d < 1)
        return ATTN_ERR_SHAPE;
    if (max_seqlen_q > total_q || max_seqlen_k > total_k) return ATTN_ERR_SEQLENS;
    if ((int64_t)total_q * Hq * d > kMaxElems || (int64_t)total_k * Hkv * d > kMaxElems)
        return ATTN_ERR_SHAPE;
    if (!d_ok(d)) return ATTN_ERR_UNSUPPORTED_D;
    if (Hq % Hkv) return ATTN_ERR_GQA_RATIO;
    if (!scale_ok(scale)) return ATTN_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        (lse && !aligned(lse, 4)) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
        return ATTN_ERR_ALIGNMENT;
    const int ntiles = ceil_div(max_seqlen_q, attn::kFwdBr);
    if ((int64_t)ntiles * nseq * Hq > 0x7fffffff) return ATTN_ERR_SHAPE;
    attn::FwdParams p{};
    p.q = (const __bf16 *)q;
    p.k = (const __bf16 *)k;
    p.v = (const __bf16 *)v;
    p.o = (__bf16 *)o;
    p.lse = lse;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.nbatch = nseq;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.group = Hq / Hkv;
    p.total_q = total_q;
    p.total_k = total_k;
    p.max_len = max_seqlen_q > max_seqlen_k ? max_seqlen_q : max_seqlen_k;
    p.ntiles = ntiles;
    p.c = scale * attn::kLog2e;
    return from_hip(attn::launch_fwd(p, d, causal != 0, true, stream));
}

int attn_decode_pick_splits(int B, int Hq, int Hkv, int Skv) {
    if (!decode_sizes_ok(B, Hq, Hkv, Skv, 64) || Hq % Hkv) return 0;
    return pick_splits(B, Hq, Hkv, Skv);
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Skv, int d, int num_splits) {
    if (!decode_sizes_ok(B, Hq, Hkv, Skv, d) || Hq % Hkv || !d_ok(d)) return 0;
    const DecodeShape sh = decode_shape(B, Hq, Hkv, Skv, num_splits);
    return decode_ws_bytes(B, Hq, d, sh.nsplit);
}

}  // extern "C"

namespace {

struct PagedCache {
    const int *block_table;
    int page_size, max_pages, num_pages;
};

// An fp8 (e4m3fn) cache: stored codes times a per-tensor scale.
struct Fp8Cache {
    float k_scale, v_scale;
};

// The argument checks of every decode entry point, in their fixed order
// (everything but the workspace).
attn_status_t decode_args_status(const void *q, const void *k_cache, const void *v_cache,
                                 const void *o, const float *lse, int B, int Hq, int Hkv, int Skv,
                                 int d, float scale, int num_splits, const Fp8Cache *fp8) {
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
    return ATTN_OK;
}

attn_status_t decode_impl(const void *q, const void *k_cache, const void *v_cache, void *o,
                          float *lse, const int *seqlens, int B, int Hq, int Hkv, int Skv, int d,
                          float scale, int num_splits, void *workspace, size_t workspace_bytes,
                          hipStream_t stream, const PagedCache *paged = nullptr,
                          const Fp8Cache *fp8 = nullptr) {
    const attn_status_t st = decode_args_status(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d,
                                                scale, num_splits, fp8);
    if (st != ATTN_OK) return st;
    const DecodeShape sh = decode_shape(B, Hq, Hkv, Skv, num_splits);
    const size_t need = decode_ws_bytes(B, Hq, d, sh.nsplit);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return ATTN_ERR_ALIGNMENT;
    }
    if ((int64_t)B * Hkv * sh.ncb * sh.nsplit > 0x7fffffff) return ATTN_ERR_SHAPE;
    attn::DecParams p{};
    p.q = (const __bf16 *)q;
    p.k = k_cache;
    p.v = v_cache;
    p.o = (__bf16 *)o;
    p.lse = lse;
    p.seqlens = seqlens;
    if (paged != nullptr) {
        p.block_table = paged->block_table;
        p.page_size = paged->page_size;
        p.max_pages = paged->max_pages;
        p.num_pages = paged->num_pages;
    }
    if (need > 0) {
        p.ws_o = (float *)workspace;
        p.ws_lse = p.ws_o + (size_t)sh.nsplit * B * Hq * d;
    }
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.group = Hq / Hkv;
    p.Skv = Skv;
    p.ncb = sh.ncb;
    p.nsplit = sh.nsplit;
    p.chunk = sh.chunk;
    p.c = scale * attn::kLog2e;
    p.v_scale = 1.f;
    if (fp8) {
        // scores use the stored key codes: the key scale joins the softmax
        // scale; the value scale multiplies the output
        p.c = scale * fp8->k_scale * attn::kLog2e;
        p.v_scale = fp8->v_scale;
    }
    return from_hip(attn::launch_decode(p, d, fp8 != nullptr, stream));
}

}  // namespace

extern "C" {

attn_status_t attn_decode(const void *q, const void *k_cache, const void *v_cache, void *o,
                          float *lse, int B, int Hq, int Hkv, int Skv, int d, float scale,
                          int num_splits, void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
    return decode_impl(q, k_cache, v_cache, o, lse, nullptr, B, Hq, Hkv, Skv, d, scale,
                       num_splits, workspace, workspace_bytes, stream);
}

attn_status_t attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  void *o, float *lse, int B, int Hq, int Hkv, int Skv, int d,
                                  float scale, int num_splits, hipStream_t stream) {
    const attn_status_t st = decode_args_status(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d,
                                                scale, num_splits, nullptr);
    if (st != ATTN_OK) return st;
    // the partials must fit the fixed scratch
    const size_t need = decode_ws_bytes(B, Hq, d, decode_shape(B, Hq, Hkv, Skv, num_splits).nsplit);
    if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    if (need > 0) {
        // the device address of this GPU's copy of `scratch`, looked up on
        // the first call on the device (with it current) and kept
        static std::mutex mu;
        static void *addr[64] = {};
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ATTN_ERR_HIP;
        std::lock_guard<std::mutex> lock(mu);
        if (addr[dev] == nullptr) {
            void *p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return ATTN_ERR_HIP;
            addr[dev] = p;
        }
        ws = addr[dev];
    }
    return decode_impl(q, k_cache, v_cache, o, lse, nullptr, B, Hq, Hkv, Skv, d, scale,
                       num_splits, ws, ws ? (size_t)ATTN_NOALLOC_SCRATCH_BYTES : 0, stream);
}

attn_status_t attn_decode_varlen(const void *q, const void *k_cache, const void *v_cache,
                                 void *o, float *lse, const int *seqlens_k, int B, int Hq,
                                 int Hkv, int Skv_max, int d, float scale, int num_splits,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!seqlens_k) return ATTN_ERR_NULLPTR;
    if (!aligned(seqlens_k, 4)) return ATTN_ERR_ALIGNMENT;
    return decode_impl(q, k_cache, v_cache, o, lse, seqlens_k, B, Hq, Hkv, Skv_max, d, scale,
                       num_splits, workspace, workspace_bytes, stream);
}

attn_status_t attn_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                                void *o, float *lse, const int *block_table,
                                const int *seqlens_k, int B, int Hq, int Hkv, int d,
                                int page_size, int max_pages_per_seq, int num_pages, float scale,
                                int num_splits, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    if (!block_table || !seqlens_k) return ATTN_ERR_NULLPTR;
    if (page_size < 16 || page_size % 16 || max_pages_per_seq < 1 || num_pages < 1)
        return ATTN_ERR_SHAPE;
    if ((int64_t)max_pages_per_seq * page_size > 0x7fffffff ||
        (int64_t)num_pages * page_size * Hkv * d > kMaxElems ||
        (int64_t)B * max_pages_per_seq > 0x7fffffff)
        return ATTN_ERR_SHAPE;
    if (!aligned(block_table, 4) || !aligned(seqlens_k, 4)) return ATTN_ERR_ALIGNMENT;
    const PagedCache pc{block_table, page_size, max_pages_per_seq, num_pages};
    // each sequence can hold max_pages_per_seq * page_size keys; the
    // checks and key chunking below treat that as the cache capacity
    return decode_impl(q, k_pages, v_pages, o, lse, seqlens_k, B, Hq, Hkv,
                       max_pages_per_seq * page_size, d, scale, num_splits, workspace,
                       workspace_bytes, stream, &pc);
}

attn_status_t attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache, void *o,
                              float *lse, const int *seqlens_k, int B, int Hq, int Hkv,
                              int Skv, int d, float scale, float k_scale, float v_scale,
                              int num_splits, void *workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    if (seqlens_k && !aligned(seqlens_k, 4)) return ATTN_ERR_ALIGNMENT;
    const Fp8Cache f{k_scale, v_scale};
    return decode_impl(q, k_cache, v_cache, o, lse, seqlens_k, B, Hq, Hkv, Skv, d, scale,
                       num_splits, workspace, workspace_bytes, stream, nullptr, &f);
}

attn_status_t attn_kmeans_assign(const void *x, const void *c, int *idx, float *dist, int N, int K,
                                 int d, hipStream_t stream) {
    if (!x || !c || !idx) return ATTN_ERR_NULLPTR;
    if (N < 1 || K < 1 || (int64_t)N * d > kMaxElems || (int64_t)K * d > kMaxElems)
        return ATTN_ERR_SHAPE;
    if (!d_ok(d)) return ATTN_ERR_UNSUPPORTED_D;
    if (!aligned(x, 16) || !aligned(c, 16) || !aligned(idx, 4) || (dist && !aligned(dist, 4)))
        return ATTN_ERR_ALIGNMENT;
    attn::AssignParams p{};
    p.x = (const __bf16 *)x;
    p.c = (const __bf16 *)c;
    p.idx = idx;
    p.dist = dist;
    p.N = N;
    p.K = K;
    return from_hip(attn::launch_kmeans_assign(p, d, stream));
}

}  // extern "C"
