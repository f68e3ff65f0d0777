/*
 * attn.h -- C ABI of the fused, tiled attention forward pass for AMD MI355X
 * (gfx950).  Library: tiled_attention_transformer_amd/libattn.so.
 *
 * What is computed (lecompute.fr, "FlashAttention-4 : limites du calcul
 * matriciel", section "Entre deux multiplications il faut fabriquer les
 * poids"): for every query row, scores against the keys, a softmax that turns
 * them into positive weights summing to one, and the weighted sum of the value
 * rows:
 *
 *     O[i] = sum_j softmax_j(scale * q_i . k_j) * v_j      (j over allowed keys)
 *     LSE[i] = log(sum_j exp(scale * q_i . k_j))          (natural log)
 *
 * The work is cut into query and key tiles and accumulated tile by tile with
 * an online softmax (same section, and section "Déplacer une partie des
 * exponentielles": one common scale for the old and the new contributions),
 * so the score matrix never reaches device memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Tensors are contiguous, row-major, bfloat16 (q, k, v, o) and float32
 *    (lse), passed as raw DEVICE pointers.  The caller allocates and owns
 *    every buffer; the library allocates nothing.  The only state it keeps
 *    between calls is a per-device cache of the compute-unit count (read
 *    once, a property of the device) and, for attn_decode_noalloc alone, its
 *    fixed device array and that array's per-device address (below); every
 *    other entry point is thread-safe.
 *  * Pointers to bf16 tensors must be 16-byte aligned; lse and the decode
 *    workspace 4- and 16-byte aligned respectively.
 *  * Head grouping (GQA/MQA): query head h reads KV head h / (Hq / Hkv);
 *    Hq must be a multiple of Hkv.
 *  * Head dimension d must be 64 or 128.  scale must be finite and > 0
 *    (typically 1/sqrt(d)).
 *  * Causal masking is bottom-right aligned: query row i (0-based) may see key
 *    j iff j <= i + (Skv - Sq).  With Sq == Skv this is the usual lower
 *    triangle (same page, section "Le FP4 ajoute un compromis numérique",
 *    on the causal mask).  A row with no allowed key gets O = 0 and
 *    LSE = -inf.
 *  * lse may be NULL, in which case it is not written.
 *  * Every call is asynchronous on `stream` (0 = the null stream) and never
 *    synchronises (outside debug mode 1, below).  Arguments are validated on the host BEFORE any launch; on
 *    a nonzero status nothing was launched and no output was written.  A
 *    launch failure returns ATTN_ERR_HIP (outputs then undefined).
 *  * Results are deterministic: the same inputs give bitwise the same
 *    outputs (fixed tile order, no atomics).
 *
 * Debug modes (environment variable ATTN_DEBUG, an integer of bit flags,
 * read at every call; unset or 0 in production)
 * ------------------------------------------------------------------------
 *  * 1: every call synchronises its stream before it returns and reports a
 *    kernel fault as ATTN_ERR_HIP, so a fault is charged to the call that
 *    caused it.
 *  * 2: fixed-batch prefill fills each LDS stage of the K/V ring with NaN
 *    before its tile loads are issued, so a read of a stage before its loads
 *    complete (or after the stage was handed back) turns the output NaN.
 *  * 4: fixed-batch prefill runs the shallowest K/V ring its pipeline allows
 *    (3 stages instead of 4), which leaves no slack for a missing wait.
 *  Modes 2 and 4 (and 6, both) change no arithmetic: correct kernels give the
 *  normal mode's outputs bit for bit, only slower.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULLPTR = 1,        /* a required pointer is NULL                   */
    ATTN_ERR_SHAPE = 2,          /* a size is < 1 or too large                   */
    ATTN_ERR_UNSUPPORTED_D = 3,  /* d is not 64 or 128                           */
    ATTN_ERR_GQA_RATIO = 4,      /* Hq is not a multiple of Hkv                  */
    ATTN_ERR_ALIGNMENT = 5,      /* a pointer is not suitably aligned            */
    ATTN_ERR_WORKSPACE = 6,      /* decode workspace missing or too small        */
    ATTN_ERR_SEQLENS = 7,        /* malformed cumulative sequence offsets        */
    ATTN_ERR_HIP = 8,            /* the HIP runtime reported an error on launch  */
    ATTN_ERR_SCALE = 9,          /* scale is not finite and > 0                  */
    ATTN_ERR_SCRATCH_LIMIT = 10, /* the sizes need more than the fixed scratch   */
    ATTN_ERR_OPTION = 11         /* an option is outside its documented values   */
} attn_status_t;

/* Size of the fixed device scratch that attn_decode_noalloc uses (bytes). */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * Prefill / full forward over a fixed batch.
 *   q, o : [B, Sq, Hq, d]  bf16        k, v : [B, Skv, Hkv, d]  bf16
 *   lse  : [B, Hq, Sq]     fp32 (or NULL)
 *   causal: 0 = every key, nonzero = bottom-right causal mask.
 * Query tiles of 256 rows, key tiles of 64 keys; under the causal mask the
 * key tiles above a query tile's diagonal are never loaded.
 */
attn_status_t attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                       int B, int Hq, int Hkv, int Sq, int Skv, int d, float scale,
                       int causal, hipStream_t stream);

/*
 * attn_fwd with part of the softmax's exponentials computed by a polynomial
 * on the fused multiply-add path instead of the hardware exponential
 * (lecompute.fr, "FlashAttention-4 : limites du calcul matriciel", section
 * "Déplacer une partie des exponentielles": moving a share of the
 * exponentials onto the FMA units so that both kinds of unit carry part of
 * the softmax).  Same arguments and layouts as attn_fwd, plus:
 *   poly_per_32 : of each lane's 32 exponentials per 64-key tile, how many
 *                 go to the polynomial: 0 (this is then attn_fwd exactly,
 *                 bit for bit), 4, 8 or 16; any other value returns
 *                 ATTN_ERR_OPTION before any launch.
 * The polynomial is exp2(x) = 2^floor(x) * p(x - floor(x)) with a cubic p,
 * p(0) = 1, fitted for the smallest maximum relative error on [0, 1) by
 * Remez's exchange (relative error at most 8.6e-5; the weights are rounded
 * to bfloat16, relative 2^-9, before the P V product).  Masked scores still
 * give weight exactly 0.  Every fixed batch runs the two-group (ping-pong)
 * kernel on this path, whatever its size; the debug modes 2 and 4 do not
 * apply to it.  Errors as attn_fwd, plus ATTN_ERR_OPTION.  On gfx950 the
 * hardware exponential is not the prefill's limit (the softmax phase is
 * bound by vector-instruction issue, and the polynomial takes 7 vector
 * instructions where the exponential takes one), so this is a lever, not
 * the default: measured slower than attn_fwd at every share (causal B4 H16
 * S2048 d128: 2.5 %, 4.3 % and 9.1 % at 4, 8 and 16; B1 H32 S16384: 3.4 %,
 * 6.3 % and 13.1 %).
 */
attn_status_t attn_fwd_exp2_poly(const void *q, const void *k, const void *v, void *o,
                                 float *lse, int B, int Hq, int Hkv, int Sq, int Skv, int d,
                                 float scale, int causal, int poly_per_32, hipStream_t stream);

/*
 * Prefill with the key range split across workgroups (split-KV), for shapes
 * with few query tiles (few sequences, heads or rows, e.g. a chunk of new
 * tokens against a long cache), where attn_fwd would leave compute units
 * idle.  Same arguments and result as attn_fwd (up to fp32 rounding
 * order), plus:
 *   num_splits : key shares per query tile (each tile's own key tiles, cut
 *                into num_splits runs of equal length); <= 0 lets the
 *                library choose (about one work item per compute unit, and
 *                shares that average at least 1024 keys -- otherwise the
 *                partials' traffic outweighs the gain; 1 when no split
 *                pays); 1 is attn_fwd exactly.
 *   workspace  : DEVICE scratch of at least
 *                attn_fwd_splitkv_workspace_bytes(...) bytes, 16-byte
 *                aligned, owned by the caller (NULL allowed when that is 0);
 *                it holds each share's normalised output (fp32) and
 *                log-sum-exp, merged by LSE = M + log(sum_s exp(lse_s - M)),
 *                O = sum_s exp(lse_s - LSE) O_s -- the same merge as decode.
 * Deterministic for given sizes and num_splits.  Errors as attn_fwd, plus
 * ATTN_ERR_WORKSPACE and ATTN_ERR_SHAPE for num_splits > 1024.  The
 * splitting is the decode's key-range split (lecompute.fr, "FlashAttention-4
 * : limites du calcul matriciel", section "Déplacer une partie des
 * exponentielles": partial results under their own scale, merged by a common
 * one) applied to prefill.
 */
attn_status_t attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                               int B, int Hq, int Hkv, int Sq, int Skv, int d, float scale,
                               int causal, int num_splits, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Bytes of attn_fwd_splitkv workspace for these sizes and mask (0 when
 * num_splits resolves to 1; num_splits <= 0 means the library's choice, which
 * depends on causal).  Returns 0 for invalid sizes. */
size_t attn_fwd_splitkv_workspace_bytes(int B, int Hq, int Sq, int Skv, int d, int causal,
                                        int num_splits);

/*
 * Forward over a packed ragged batch (variable lengths).
 *   q, o : [total_q, Hq, d] bf16      k, v : [total_k, Hkv, d] bf16
 *   lse  : [Hq, total_q] fp32 (or NULL)
 *   cu_seqlens_q, cu_seqlens_k : DEVICE int32 arrays of nseq+1 cumulative
 *   offsets (start at 0, non-decreasing, last = total).  Sequence s owns query
 *   rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 and keys cu_seqlens_k[s] ..
 *   cu_seqlens_k[s+1]-1; it never sees another sequence's keys, and the
 *   causal mask applies inside each sequence.
 *   max_seqlen_q must be >= every query length (it sizes the grid); rows of a
 *   longer sequence beyond it are not computed.  The kernels read the offsets
 *   on the device and treat a sequence whose offsets are decreasing or fall
 *   outside [0, total] as empty, so malformed offsets cannot cause an
 *   out-of-bounds access; use attn_varlen_check() on a host copy to reject
 *   them up front.
 */
attn_status_t attn_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                              const int *cu_seqlens_q, const int *cu_seqlens_k, int nseq,
                              int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                              int Hq, int Hkv, int d, float scale, int causal,
                              hipStream_t stream);

/*
 * Host-side check of a HOST copy of cumulative offsets: nseq >= 1,
 * cu[0] == 0, non-decreasing, cu[nseq] == total.  If max_seqlen is not NULL
 * it receives the largest length.  Returns ATTN_OK or ATTN_ERR_SEQLENS
 * (ATTN_ERR_NULLPTR for a NULL cu).  Touches no device.
 */
attn_status_t attn_varlen_check(const int *cu_seqlens_host, int nseq, int total,
                                int *max_seqlen);

/*
 * Split-KV decode: one query token per sequence against a KV cache.
 *   q, o : [B, Hq, d] bf16      k_cache, v_cache : [B, Skv, Hkv, d] bf16
 *   lse  : [B, Hq] fp32 (or NULL)
 * The query is the newest position, so all Skv cached keys are attended.
 * The cache is cut into num_splits chunks of ceil(Skv / num_splits) keys,
 * rounded up to a multiple of 32 (trailing chunks may then be empty); a
 * normalised partial output and its log-sum-exp are computed per (sequence,
 * KV head, chunk) -- every query head of a KV group shares one pass over that
 * chunk of K and V -- and the chunks are merged:
 * LSE = M + log(sum_s exp(lse_s - M)), O = sum_s exp(lse_s - LSE) * O_s.
 * A positive num_splits is honoured as given: with more than one chunk the
 * chunks spread over the workgroups, each writes a normalised fp32 partial
 * and its log-sum-exp into the workspace, and a second kernel merges them.
 * With one chunk (num_splits == 1) each workgroup takes whole sequences: its
 * four waves split the keys, their results are merged the same way inside
 * the kernel, and no workspace is used.  Either way the result is the same
 * log-sum-exp merge (up to fp32 rounding order), and it is deterministic for
 * given sizes and num_splits.
 * num_splits <= 0 lets the library choose (attn_decode_pick_splits): one
 * chunk when the (sequence, KV head, block of 32 query heads) groups alone
 * give each of an MI355X's 256 compute units a work item, else about one
 * work item per compute unit with chunks of at least 512 keys; then a few
 * more chunks when they fill the last round of work items much better (384
 * groups, 1.5 per compute unit, take 2 chunks).
 * workspace: DEVICE scratch of at least attn_decode_workspace_bytes(...)
 * bytes, 16-byte aligned, owned by the caller, may be reused between calls
 * on the same stream (not by calls that run concurrently).  When the split
 * count resolves to 1 no workspace is needed (may be NULL); the size needed
 * depends on the sizes and num_splits only.
 */
attn_status_t attn_decode(const void *q, const void *k_cache, const void *v_cache, void *o,
                          float *lse, int B, int Hq, int Hkv, int Skv, int d, float scale,
                          int num_splits, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * Decode against caches filled to different lengths: sequence b attends to
 * keys 0 .. seqlens_k[b]-1 of its cache rows.  Same layouts, chunking,
 * workspace and errors as attn_decode, with Skv_max the cache capacity
 * (the row count of k_cache and v_cache).  seqlens_k: DEVICE int32 [B],
 * 4-byte aligned, read by the kernels; values are clamped to
 * [0, Skv_max] on the device (the host never reads them).  A sequence of
 * length 0 gets O = 0 and LSE = -inf.  Chunks past a sequence's length read
 * no memory.  Serving keeps one KV cache per sequence, each filled to its
 * own length (lecompute.fr, "Flapping Airplanes, ThunderKittens and
 * megakernels", section "A benchmark that could test the broader promise").
 * Split by the lengths: with num_splits <= 0 and a workspace of at least
 * attn_decode_varlen_workspace_bytes(B, Hq, Hkv, Skv_max, d) bytes, the
 * kernel reads the lengths, lays the 32-key tiles of every (sequence, KV
 * head, block of 32 query heads) group end to end and gives each of the
 * 1024 waves of its grid an equal run of ceil(tiles / 1024) tiles (at least
 * 4), so a batch of mixed lengths (one long sequence among short ones)
 * spreads evenly over the whole GPU.  A group inside one run gets its result
 * directly; the runs of the others are merged as above.  With a smaller
 * workspace (attn_decode_workspace_bytes) or a positive num_splits the split
 * is by the capacity Skv_max, as in attn_decode.  The same holds for
 * attn_decode_paged and for attn_decode_fp8 with seqlens_k.  The runs depend
 * on the lengths, so the fp32 rounding order (not the result beyond it) may
 * change with them.  Up to 2048 sequences, and sequences x ceil(Skv_max / 32)
 * x Hkv x query-head blocks below 2^31 - 2^20; larger batches split by the
 * capacity.
 */
attn_status_t attn_decode_varlen(const void *q, const void *k_cache, const void *v_cache,
                                 void *o, float *lse, const int *seqlens_k, int B, int Hq,
                                 int Hkv, int Skv_max, int d, float scale, int num_splits,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode against a paged KV cache (blocks of page_size keys drawn from a
 * shared pool, as a serving system allocates them).
 *   k_pages, v_pages : [num_pages, page_size, Hkv, d] bf16 (DEVICE)
 *   block_table      : DEVICE int32 [B, max_pages_per_seq]; key j of sequence
 *                      b is row j % page_size of page
 *                      block_table[b * max_pages_per_seq + j / page_size]
 *   seqlens_k        : DEVICE int32 [B], keys per sequence, clamped on the
 *                      device to [0, max_pages_per_seq * page_size]
 *   q, o, lse, scale, num_splits, workspace: as attn_decode, with the cache
 *   capacity Skv = max_pages_per_seq * page_size (use that value for
 *   attn_decode_workspace_bytes / attn_decode_pick_splits).
 * page_size must be a positive multiple of 16.  Only table entries that
 * hold keys below a sequence's length are read; a page id outside
 * [0, num_pages) is read as zeros (no memory outside the pool is touched)
 * and the result for that sequence is then meaningless.  block_table and
 * seqlens_k are read by the kernels only (the host never reads them).
 * Returns ATTN_ERR_NULLPTR for a NULL table or lengths, ATTN_ERR_SHAPE for a
 * page size that is not a multiple of 16 or non-positive counts, and the
 * errors of attn_decode otherwise.  The per-sequence cache of the serving
 * note in lecompute.fr, "Flapping Airplanes, ThunderKittens and
 * megakernels", section "A benchmark that could test the broader promise",
 * stored in fixed-size pages.
 */
attn_status_t attn_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                                void *o, float *lse, const int *block_table,
                                const int *seqlens_k, int B, int Hq, int Hkv, int d,
                                int page_size, int max_pages_per_seq, int num_pages, float scale,
                                int num_splits, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Decode against an 8-bit floating-point KV cache: every cached element is
 * an OCP FP8 E4M3 ("e4m3fn": 1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, no infinities, codes 0x7F / 0xFF are NaN) code, one byte,
 * and the cache holds k = k_scale * code(K), v = v_scale * code(V) with one
 * positive fp32 scale per tensor.
 *   q, o : [B, Hq, d] bf16      k_cache, v_cache : [B, Skv, Hkv, d] uint8 codes
 *   lse  : [B, Hq] fp32 (or NULL)
 *   seqlens_k : DEVICE int32 [B] (4-byte aligned) as in attn_decode_varlen, or
 *   NULL to attend to all Skv keys of every sequence.
 * The result is the attention of attn_decode over the dequantised cache:
 * scores scale * k_scale * (q . code(k_j)), O = v_scale * sum_j p_j code(v_j).
 * Codes are widened to bf16 exactly (every E4M3 value is a bf16 value); the
 * scales are applied in fp32 to the scores and to the output.  Chunking,
 * workspace (attn_decode_workspace_bytes with the same sizes) and errors as
 * attn_decode; ATTN_ERR_SCALE also for a k_scale or v_scale that is not
 * finite and > 0.  Cache pointers must be 16-byte aligned.  Halving the
 * bytes per cached element halves the memory traffic that bounds decode
 * (lecompute.fr, "Flapping Airplanes, ThunderKittens and megakernels",
 * section "Follow the request instead of one utilization number"); each
 * generation of matrix units takes narrower formats, FP8 among them (same
 * page, section "ThunderKittens starts with tiles, not whole applications", glossary note
 * on Tensor Cores).
 */
attn_status_t attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache, void *o,
                              float *lse, const int *seqlens_k, int B, int Hq, int Hkv,
                              int Skv, int d, float scale, float k_scale, float v_scale,
                              int num_splits, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Fused k-means assignment (FlashAssign): for every point, the nearest
 * centroid in squared Euclidean distance, without writing the N x K
 * distance matrix (lefilia.fr, "Flash-KMeans : un K-Means exact et optimisé
 * pour les E/S, plus de 200 fois plus rapide que FAISS sur GPU", the
 * paragraph on the assignment phase).
 *   x    : [N, d] bf16 points          c : [K, d] bf16 centroids
 *   idx  : [N] int32, idx[n] = argmin_k |x_n - c_k|^2; among equal computed
 *          distances the lowest k
 *   dist : [N] fp32 (or NULL), |x_n - c_idx[n]|^2 (clamped at 0)
 * The distance is compared as |c_k|^2 - 2 x_n . c_k with fp32 accumulation
 * of bf16 products (|x_n|^2 is common to all k); dist adds |x_n|^2.  d must
 * be 64 or 128; N, K >= 1.  x and c 16-byte aligned, idx and dist 4-byte
 * aligned.  No workspace; deterministic.  Errors: ATTN_ERR_NULLPTR (x, c or
 * idx NULL), ATTN_ERR_SHAPE, ATTN_ERR_UNSUPPORTED_D, ATTN_ERR_ALIGNMENT,
 * ATTN_ERR_HIP.
 */
attn_status_t attn_kmeans_assign(const void *x, const void *c, int *idx, float *dist, int N, int K,
                                 int d, hipStream_t stream);

/*
 * attn_decode without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * layouts, split choice, result and errors as attn_decode, minus
 * workspace / workspace_bytes.  The split partials live in a fixed array of
 * ATTN_NOALLOC_SCRATCH_BYTES in device memory that the library holds on
 * every GPU it runs on until the process ends (its address is looked up
 * once per device, on the first call there).  Sizes whose partials need
 * more (attn_decode_workspace_bytes(...) > ATTN_NOALLOC_SCRATCH_BYTES) are
 * refused with ATTN_ERR_SCRATCH_LIMIT before any launch; with the split
 * count resolving to 1 no scratch is used at all.  Every call on one GPU
 * shares that GPU's array: calls that may overlap on one GPU (different
 * streams, other host threads) race on it and must be serialised by the
 * caller.  Nothing in the array needs clearing: every partial a call reads
 * is written by the same call.
 */
attn_status_t attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  void *o, float *lse, int B, int Hq, int Hkv, int Skv, int d,
                                  float scale, int num_splits, hipStream_t stream);

/* Bytes of decode workspace for these sizes (0 when num_splits resolves to
 * 1; num_splits <= 0 means the library's choice, as in attn_decode).  Returns
 * 0 for invalid sizes. */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Skv, int d, int num_splits);

/* Bytes of workspace for the split by the lengths of attn_decode_varlen,
 * attn_decode_paged and attn_decode_fp8 with seqlens_k (num_splits <= 0):
 * a header (16 bytes, then B + 1 ints, padded to 16 bytes: the run length
 * and each sequence's first tile, which the kernel writes), then fp32
 * partials with their log-sum-exp (d + 1 values each) in a row per
 * (sequence, query head) and min(Hq / Hkv, 32) rows per wave of the
 * 1024-wave grid.  Independent of Skv_max.  For sizes where that split is
 * not available (see attn_decode_varlen) this is
 * attn_decode_workspace_bytes(B, Hq, Hkv, Skv_max, d, 0), and the call
 * splits by the capacity.  Returns 0 for invalid sizes. */
size_t attn_decode_varlen_workspace_bytes(int B, int Hq, int Hkv, int Skv_max, int d);

/* The number of KV chunks attn_decode uses when passed num_splits <= 0:
 * about one work item per compute unit of an MI355X (256 items over the
 * (sequence, KV head, head block) groups), but chunks of at least 512 keys;
 * so 1 (whole sequences, no workspace) when the groups alone number 256 or
 * more.  Of that count s0 and up to max(2 s0, s0 + 3) chunks, the one whose
 * items fill the rounds of the workers best (256 workgroups, or 1024 waves
 * once there are at least 1024 split items) is taken when it fills them by
 * at least 0.15 more. */
int attn_decode_pick_splits(int B, int Hq, int Hkv, int Skv);

/* Static text for a status code (never NULL). */
const char *attn_status_string(attn_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
