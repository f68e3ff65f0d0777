// Launch parameters and launchers of the gfx950 attention kernels.  Internal
// to libattn.so: the exported C ABI (include/attn.h) validates arguments and
// then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fastdiv.h"
#include "tile_config.h"

namespace attn {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Slack (log2 units) before the online softmax moves its reference max:
// weights exp2(s*c - m) stay <= 2^8, far from fp32/bf16 overflow.
constexpr float kRescaleSlack = 8.0f;

// n / d for 0 <= n < 2^31, with the constants make_fastdiv(d) (fastdiv.h)
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.s; }

// Compute units of the current device.  Cached per device after the first
// query: the attribute query costs host time on every launch otherwise,
// which shows up as idle GPU time between back-to-back calls.
inline hipError_t current_cu_count(int *cus) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < 64;
    if (cached) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (cached) cache[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return hipSuccess;
}

struct FwdParams {
    const __bf16 *q, *k, *v;
    __bf16 *o;
    float *lse;              // may be null
    const int *cu_q, *cu_k;  // varlen only (device)
    int nbatch;              // B, or nseq for varlen
    int Hq, Hkv, group;      // group = Hq / Hkv
    int Sq, Skv;             // fixed batch only
    int max_len;             // ragged batch: longest query or key sequence (launch choice)
    int total_q, total_k;    // varlen only
    int ntiles;              // query tiles per (batch, head)
    int nitems;              // ntiles * nbatch * Hq (* nsplit; set by the launcher)
    float c;                 // scale * log2(e)
    // split-KV prefill (fixed batches): each query tile's key tiles are cut
    // into nsplit shares; split s of a tile writes its normalised output and
    // natural-log LSE to ws_o [nsplit, B, Hq, Sq, d] and ws_lse [nsplit, B, Hq, Sq]
    int nsplit;
    float *ws_o, *ws_lse;
    // debug bits (host only, chosen at launch): 2 = NaN-poison retired LDS
    // stages, 4 = 3-stage K/V ring, 6 = both (fixed-batch prefill)
    int debug;
    // ragged batch on a persistent grid with a cost-sorted item list (set by
    // the launcher when the list fits the kSched* bounds)
    int compact;
    // the item decode's divisors (nbatch * Hq, Hq, group, nsplit), set by the
    // launcher
    FastDiv fd_bh, fd_hq, fd_group, fd_split;
};

struct DecParams {
    const __bf16 *q;
    const void *k, *v;       // bf16, or fp8 (e4m3fn) codes for an fp8 cache
    __bf16 *o;
    float *lse;              // may be null
    float *ws_o, *ws_lse;    // split partials (null when nsplit == 1)
    const int *seqlens;      // keys per sequence (device, clamped to [0, Skv]), or null: all Skv
    // paged caches (block_table non-null): k, v are [num_pages, page_size,
    // Hkv, d]; key j of sequence b is row j % page_size of page
    // block_table[b * max_pages + j / page_size]; Skv = max_pages * page_size
    const int *block_table;
    int page_size, max_pages, num_pages;
    int B, Hq, Hkv, group, Skv;
    int ncb;                 // blocks of <= 32 query heads per KV head
    int nsplit, chunk;       // key chunks and keys per chunk
    float c;                 // scale * log2(e) (times the key scale of an fp8 cache)
    float v_scale;           // value scale of an fp8 cache (unused for bf16)
    // split by the per-sequence key counts (seqlens given): the kernel lays
    // the groups' tiles end to end and gives every wave an equal run; it
    // writes the run length and the per-sequence tile offsets to ws_hdr
    // (ws_hdr[0], ws_hdr[4 + b]) for the merge.  Partial rows: B * Hq for
    // each group's first run, then ncm per wave for the run that continues a
    // group begun by an earlier wave (ncm = query heads of a block).
    int listed;
    int *ws_hdr;
    int ncm;
};

// k-means assignment: nearest centroid of every point
struct AssignParams {
    const __bf16 *x, *c;     // points [N, d], centroids [K, d]
    int *idx;                // [N]
    float *dist;             // [N], may be null
    int N, K;
};

// exp2_poly: for fixed batches, of each lane's 32 exponentials per key tile
// this many (0, 4, 8 or 16) by the polynomial of exp2_poly.h
hipError_t launch_fwd(const FwdParams &p, int d, bool causal, bool varlen, hipStream_t s,
                      int exp2_poly = 0);
hipError_t launch_fwd_split(const FwdParams &p, int d, bool causal, hipStream_t s);
hipError_t launch_decode(const DecParams &p, int d, bool fp8, hipStream_t s);
hipError_t launch_kmeans_assign(const AssignParams &p, int d, hipStream_t s);

}  // namespace attn
