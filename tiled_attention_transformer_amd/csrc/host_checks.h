// Host-side argument checks and sizing of the C ABI: plain C++, no HIP
// device code, so the same source builds into libattn.so and, on its own,
// under the host sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/attn.h"

namespace attn {
namespace host {

constexpr int64_t kMaxElems = (int64_t)1 << 40;   // sanity cap on tensor sizes

bool aligned(const void *p, uintptr_t a);
bool d_ok(int d);
bool scale_ok(float s);
int ceil_div(int a, int b);
// product of non-negative factors <= lim, decided without overflow
bool prod_le(int64_t lim, std::initializer_list<int64_t> factors);

// Decode: split count, chunk length (keys) and blocks of <= 32 query heads.
struct DecodeShape {
    int nsplit, chunk, ncb;
};
int pick_splits(int B, int Hq, int Hkv, int Skv);
DecodeShape decode_shape(int B, int Hq, int Hkv, int Skv, int num_splits);
size_t decode_ws_bytes(int B, int Hq, int d, int nsplit);
bool decode_sizes_ok(int B, int Hq, int Hkv, int Skv, int d);
// every decode check but the workspace, in its fixed order (fp8: the key and
// value scales of an fp8 cache, or NULL)
struct Fp8Scales {
    float k_scale, v_scale;
};
attn_status_t decode_args_status(const void *q, const void *k_cache, const void *v_cache,
                                 const void *o, const float *lse, int B, int Hq, int Hkv, int Skv,
                                 int d, float scale, int num_splits, const Fp8Scales *fp8);
// Decode split by the per-sequence key counts: whether a batch can use it,
// its workspace bytes, and the bytes of the workspace's header (the run
// length and the per-sequence tile offsets, before the partials)
bool decode_list_ok(int B, int Hq, int Hkv, int Skv);
size_t decode_list_ws_bytes(int B, int Hq, int Hkv, int d);
size_t decode_list_hdr_bytes(int B);
// the workspace check of a decode call that needs `need` bytes
attn_status_t workspace_status(const void *workspace, size_t workspace_bytes, size_t need);

// Split-KV prefill: split count and workspace bytes.
int fwd_pick_splits(int B, int Hq, int Sq, int Skv, bool causal);
size_t fwd_ws_bytes(int B, int Hq, int Sq, int d, int nsplit);
// fixed-batch prefill checks, in their fixed order; *ntiles receives the
// number of query tiles per (batch, head)
attn_status_t fwd_args_status(const void *q, const void *k, const void *v, const void *o,
                              const float *lse, int B, int Hq, int Hkv, int Sq, int Skv, int d,
                              float scale, int *ntiles);
// ragged-batch prefill checks
attn_status_t varlen_args_status(const void *q, const void *k, const void *v, const void *o,
                                 const float *lse, const int *cu_q, const int *cu_k, int nseq,
                                 int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                                 int Hq, int Hkv, int d, float scale, int *ntiles);
// host copy of cumulative offsets
attn_status_t varlen_check(const int *cu, int nseq, int total, int *max_seqlen);
// paged-cache extras and k-means checks
attn_status_t paged_args_status(const int *block_table, const int *seqlens_k, int B, int Hkv,
                                int d, int page_size, int max_pages_per_seq, int num_pages);
attn_status_t kmeans_args_status(const void *x, const void *c, const int *idx, const float *dist,
                                 int N, int K, int d);

}  // namespace host
}  // namespace attn
