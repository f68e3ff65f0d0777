// C ABI of libattn.so (declared in include/attn.h): the host-side argument
// checks (host_checks.cpp), then the kernel launches.  No allocation; the
// only state kept between calls is the per-device compute-unit count and
// the device address of the no-allocation scratch.
//
// ATTN_DEBUG (environment, read on every call; bits, default 0):
//   1  synchronise the stream after every launch and report any error of
//      the kernels as ATTN_ERR_HIP (a fault or a failed launch surfaces at
//      the call that caused it);
//   2  fixed-batch prefill: fill every retired LDS stage with NaN bit
//      patterns before its next tile loads (a read of a stage outside its
//      lifetime then shows up as NaN in the output);
//   4  fixed-batch prefill: a 3-stage K/V ring instead of 4 (the shallowest
//      the pipeline allows; it must give the same bits as the 4-stage ring).
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/attn.h"
#include "host_checks.h"
#include "kernels.h"

// Split partials of attn_decode_noalloc: a fixed array in device memory (one
// copy per GPU), so that entry point allocates nothing.  Host code never
// passes `scratch` itself (on the host the name is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace attn::host;

int debug_flags() {
    const char *e = getenv("ATTN_DEBUG");
    return e ? atoi(e) : 0;
}

// The status of a launch (and, in debug mode, of the kernels it started).
attn_status_t finish(hipError_t e, hipStream_t stream) {
    if (e != hipSuccess) return ATTN_ERR_HIP;
    if (debug_flags() & 1) {
        if (hipStreamSynchronize(stream) != hipSuccess) return ATTN_ERR_HIP;
        if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

attn_status_t fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                       int Hq, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                       int num_splits, void *workspace, size_t workspace_bytes,
                       hipStream_t stream, int exp2_poly = 0) {
    int ntiles = 0;
    const attn_status_t st = fwd_args_status(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, scale,
                                             &ntiles);
    if (st != ATTN_OK) return st;
    if (exp2_poly != 0 && exp2_poly != 4 && exp2_poly != 8 && exp2_poly != 16) return ATTN_ERR_OPTION;
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
    p.debug = debug_flags();
    const int ns = num_splits > 0 ? num_splits : fwd_pick_splits(B, Hq, Sq, Skv, causal != 0);
    if (ns <= 1) return finish(attn::launch_fwd(p, d, causal != 0, false, stream, exp2_poly), stream);
    const attn_status_t ws = workspace_status(workspace, workspace_bytes,
                                              fwd_ws_bytes(B, Hq, Sq, d, ns));
    if (ws != ATTN_OK) return ws;
    if ((int64_t)ntiles * B * Hq * ns > 0x7fffffff) return ATTN_ERR_SHAPE;
    p.nsplit = ns;
    p.ws_o = (float *)workspace;
    p.ws_lse = p.ws_o + (size_t)ns * B * Hq * Sq * d;
    return finish(attn::launch_fwd_split(p, d, causal != 0, stream), stream);
}

struct PagedCache {
    const int *block_table;
    int page_size, max_pages, num_pages;
};

attn_status_t decode_impl(const void *q, const void *k_cache, const void *v_cache, void *o,
                          float *lse, const int *seqlens, int B, int Hq, int Hkv, int Skv, int d,
                          float scale, int num_splits, void *workspace, size_t workspace_bytes,
                          hipStream_t stream, const PagedCache *paged = nullptr,
                          const Fp8Scales *fp8 = nullptr) {
    const attn_status_t st = decode_args_status(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d,
                                                scale, num_splits, fp8);
    if (st != ATTN_OK) return st;
    DecodeShape sh = decode_shape(B, Hq, Hkv, Skv, num_splits);
    size_t need = decode_ws_bytes(B, Hq, d, sh.nsplit);
    // Per-sequence key counts with the library's choice and a workspace
    // large enough: the kernel splits by the counts themselves (the groups'
    // key tiles end to end, an equal run per wave).  Otherwise the split is
    // by the capacity.
    const bool listed = seqlens != nullptr && num_splits <= 0 && decode_list_ok(B, Hq, Hkv, Skv) &&
                        workspace != nullptr &&
                        workspace_bytes >= decode_list_ws_bytes(B, Hq, Hkv, d);
    if (listed) need = decode_list_ws_bytes(B, Hq, Hkv, d);
    const attn_status_t ws = workspace_status(workspace, workspace_bytes, need);
    if (ws != ATTN_OK) return ws;
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
    if (listed) {
        // header (run length, per-sequence tile offsets), then the partials:
        // a row per (sequence, query head), then ncm rows per wave
        p.listed = 1;
        p.ncm = Hq / Hkv < attn::kDecCols ? Hq / Hkv : attn::kDecCols;
        p.ws_hdr = (int *)workspace;
        p.ws_o = (float *)((char *)workspace + decode_list_hdr_bytes(B));
        p.ws_lse = p.ws_o + ((size_t)B * Hq + (size_t)attn::kDecListWGs * 4 * p.ncm) * d;
        sh.nsplit = 0;
    } else if (need > 0) {
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
    return finish(attn::launch_decode(p, d, fp8 != nullptr, stream), stream);
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
        case ATTN_ERR_OPTION: return "an option is outside its documented set of values";
    }
    return "unknown status";
}

attn_status_t attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                       int Hq, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                       hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, scale, causal, 1, nullptr, 0, stream);
}

attn_status_t attn_fwd_exp2_poly(const void *q, const void *k, const void *v, void *o, float *lse,
                                 int B, int Hq, int Hkv, int Sq, int Skv, int d, float scale,
                                 int causal, int poly_per_32, hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, scale, causal, 1, nullptr, 0, stream,
                    poly_per_32);
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

attn_status_t attn_varlen_check(const int *cu, int nseq, int total, int *max_seqlen) {
    return varlen_check(cu, nseq, total, max_seqlen);
}

attn_status_t attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                              const int *cu_seqlens_q, const int *cu_seqlens_k, int nseq,
                              int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                              int Hq, int Hkv, int d, float scale, int causal,
                              hipStream_t stream) {
    int ntiles = 0;
    const attn_status_t st = varlen_args_status(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq,
                                                total_q, total_k, max_seqlen_q, max_seqlen_k, Hq,
                                                Hkv, d, scale, &ntiles);
    if (st != ATTN_OK) return st;
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
    p.debug = debug_flags();
    return finish(attn::launch_fwd(p, d, causal != 0, true, stream), stream);
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

size_t attn_decode_varlen_workspace_bytes(int B, int Hq, int Hkv, int Skv_max, int d) {
    if (!decode_sizes_ok(B, Hq, Hkv, Skv_max, d) || Hq % Hkv || !d_ok(d)) return 0;
    if (decode_list_ok(B, Hq, Hkv, Skv_max)) return decode_list_ws_bytes(B, Hq, Hkv, d);
    return decode_ws_bytes(B, Hq, d, decode_shape(B, Hq, Hkv, Skv_max, 0).nsplit);
}

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
            void *ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
                return ATTN_ERR_HIP;
            addr[dev] = ptr;
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
    const attn_status_t st = paged_args_status(block_table, seqlens_k, B, Hkv, d, page_size,
                                               max_pages_per_seq, num_pages);
    if (st != ATTN_OK) return st;
    const PagedCache pc{block_table, page_size, max_pages_per_seq, num_pages};
    // each sequence can hold max_pages_per_seq * page_size keys; the
    // checks and key chunking treat that as the cache capacity
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
    const Fp8Scales f{k_scale, v_scale};
    return decode_impl(q, k_cache, v_cache, o, lse, seqlens_k, B, Hq, Hkv, Skv, d, scale,
                       num_splits, workspace, workspace_bytes, stream, nullptr, &f);
}

attn_status_t attn_kmeans_assign(const void *x, const void *c, int *idx, float *dist, int N, int K,
                                 int d, hipStream_t stream) {
    const attn_status_t st = kmeans_args_status(x, c, idx, dist, N, K, d);
    if (st != ATTN_OK) return st;
    attn::AssignParams p{};
    p.x = (const __bf16 *)x;
    p.c = (const __bf16 *)c;
    p.idx = idx;
    p.dist = dist;
    p.N = N;
    p.K = K;
    return finish(attn::launch_kmeans_assign(p, d, stream), stream);
}

}  // extern "C"
