// Fused tiled attention forward (prefill) for gfx950.
//
// Method (lecompute.fr, "FlashAttention-4 : limites du calcul matriciel"):
// scores Q*K^T, a softmax into weights that sum to one, and a second product
// with V (section "Entre deux multiplications il faut fabriquer les poids"),
// computed tile by tile so the score matrix never leaves the chip (same
// section), with a running maximum as the common scale of the old and new
// contributions (section "Déplacer une partie des exponentielles").  The
// page's point that the exponentials and sums, not the matrix units, become
// the limit (section "Blackwell déplace la limite vers les autres unités") is
// what the schedules below are built around: the softmax of one key tile runs
// on the vector ALUs while the matrix cores compute the scores of another
// (section "Faire avancer plusieurs tuiles sans écraser leurs données"
// describes the same overlap with thread-group roles on SM100).  Two kernels
// do it two ways:
//  * attn_fwd_pp_kernel (batches with at least one 256-row item per CU,
//    except fixed batches at d = 64): the two waves of each SIMD belong to
//    two wave groups that take turns, one running a tile's MFMAs while the
//    other runs a tile's softmax, a workgroup barrier after each phase;
//  * attn_fwd_kernel (smaller grids, the split-KV prefill, fixed batches at
//    d = 64): each wave interleaves both streams itself.
// Ragged batches on the persistent grid walk a cost-sorted list of their
// items that every workgroup builds in LDS from the offsets
// (fwd_sched_build).
//
// gfx950 mapping (shared by both kernels unless noted):
//  * one work item = 256 query rows of one (batch, head); a workgroup of 8
//    waves runs one item at a time, one workgroup per CU (two waves per
//    SIMD); each wave owns 32 rows and keeps its Q fragment, running max/sum
//    and fp32 output accumulator in registers.  A fixed batch with fewer
//    256-row items than CUs runs 128-row items on 4-wave workgroups instead
//    (one wave per SIMD, twice as many items, so more CUs work);
//  * K and V tiles of 64 keys move HBM -> LDS with buffer loads that write
//    straight to LDS (buffer_load_dwordx4 ... lds, no register staging) into
//    a 4-stage ring: while tile j is consumed, tile j+1 is ready and tiles
//    j+2, j+3 are in flight.  A stage is refilled only after the barrier that
//    follows its last read (the buffer-reuse rule of lecompute.fr, "Flapping
//    Airplanes, ThunderKittens and megakernels", section "Prepare the next
//    operation without overwriting the current one").  Rows are padded (K:
//    d+8, V: d+32 elements) so the MFMA operand reads are free of bank
//    conflicts; the padding slots are filled by harmless duplicate loads so
//    every load instruction covers a whole 1 KB run of LDS;
//  * persistent workgroups (fixed-size batches): the grid has one workgroup
//    per CU and each walks a static list of items.  The tile loads form one
//    stream across items, so the first tiles of the next item, and its query
//    rows, load while the current item finishes; the output of an item is
//    written while the scores of the next one are computed.  This is the
//    scheduling of the same page, section "Prepare the next operation
//    without overwriting the current one" (start the next piece of work
//    before the current one has fully drained), applied inside one kernel;
//  * S^T = K*Q^T and O^T += V^T*P^T on v_mfma_f32_32x32x16_bf16.  In the S^T
//    layout each lane owns one query row, so the row max/sum are in-lane plus
//    one v_permlane32_swap, the rescale factor is a per-lane scalar, and P goes
//    from the score accumulators straight into the B operand of the second
//    product (converted to bf16) without touching LDS.  V stays row-major in
//    LDS and is read as the A operand with ds_read_b64_tr_b16;
//  * attn_fwd_kernel's software pipeline inside each wave: iteration j
//    issues the MFMAs of S_{j+1} and of P_j * V_j, interleaved with the
//    softmax of S_j: group g
//    holds the score MFMAs of two d-slices, weight chunk g and the P * V
//    MFMAs of the key slices whose weights chunk g-1 made.  Groups are split
//    by scheduling barriers, and every LDS operand read is issued one group
//    ahead of its MFMAs;
//  * softmax in base 2: P = exp2(s*c - m) with c = scale*log2(e) folded into
//    one FMA; the reference max m moves only when a row max grows by more
//    than 2^8, so most tiles skip the output rescale; LSE = (m + log2 l)*ln 2;
//  * under the causal mask, key tiles above a query tile's diagonal are never
//    loaded, waves skip tiles above their own rows, and only tiles that cross
//    the diagonal or the sequence end evaluate the mask;
//  * item order: (tile rank, batch*head), so under the causal mask the
//    list runs from the longest items to the shortest.  A persistent
//    workgroup w takes position w in one row of the list and the mirror
//    position in the next (boustrophedon), which pairs long items with
//    short ones; the mirror is taken in steps of 8 so an item's head keeps
//    the XCD of workgroup w (workgroups go round-robin over the 8 XCDs) and
//    its K/V stays in one L2.  Each workgroup runs its rows from the last
//    (short items) to the first, so every workgroup ends on a long item: the
//    per-item overheads then fall where the next item's loads hide them
//    rather than in the kernel's tail (measured ~5 % faster on the causal
//    B4 H16 S2048 prefill than the reverse order, same HBM traffic).
//    Ragged batches on the persistent grid use a list of their own, sorted
//    by cost on the device (their item sizes are known only there); past
//    that list's bounds they keep this order, persistent when every
//    sequence is at most 512 tokens (items of one or two tiles keep a
//    static walk balanced), else one workgroup per item.
#include <type_traits>

#include "kernels.h"
#include "tile_common.h"
#include "exp2_poly.h"

namespace attn {

namespace {

constexpr int BC = kFwdBc;
constexpr int NS = 4;                 // LDS ring stages

// NW waves per workgroup (8, or 4 for grids with fewer 256-row items than
// CUs), 32 query rows each
template <int D, int NW>
struct FwdLay {
    static constexpr int KP = D + 8;                 // K row pitch (elements)
    // V rows are read with transposing reads: a half-wave reads 64 bytes of
    // each of 4 consecutive rows, and a pitch of 16 (mod 64) dwords puts
    // those rows on disjoint banks
    static constexpr int VP = D + 32;                // V row pitch (elements)
    static constexpr int KS = KP / 8, VS = VP / 8;   // 16-byte slots per row
    static constexpr int DS = D / 8;                 // slots holding data
    static constexpr int K_INSTR = BC * KS / 64;     // wave-wide loads per K tile
    static constexpr int V_INSTR = BC * VS / 64;     // ... per V tile
    // every wave issues KW K loads, VW V loads and one more: a K load (waves
    // below KR), a V load (the next VR waves) or a repeat of its own last V
    // load (same source, same destination, so harmless)
    static constexpr int KW = K_INSTR / NW, KR = K_INSTR % NW;
    static constexpr int VW = V_INSTR / NW, VR = V_INSTR % NW;
    static constexpr int PER_WAVE = KW + VW + 1;     // loads per wave per tile
    static constexpr int K_ELEMS = BC * KP;
    static constexpr int V_ELEMS = BC * VP;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static_assert(BC * KS % 64 == 0 && BC * VS % 64 == 0, "a tile must be whole wave loads");
    static_assert(KR + VR <= NW && KW >= 1 && VW >= 1, "load plan");
};

// One work item: query rows q0 .. q0+BR-1 (BR = 32 per wave) of one (batch or
// sequence, head).
struct FwdItem {
    int b, h;
    int Sq, Skv;            // query rows and keys of the sequence
    int q0;                 // first query row of the item
    int nt;                 // key tiles of the item (0: none)
    int t0;                 // first key tile of the item (split-KV: its share)
    int sp;                 // key split of the item (split-KV), else 0
    int64_t qrow0, krow0;   // first query / key row of the sequence
};

// (cu_l: for a ragged batch, an LDS copy of the offsets, 16 bytes per
// sequence b: cu_seqlens_q[b], cu_seqlens_q[b + 1], cu_seqlens_k[b],
// cu_seqlens_k[b + 1], so one read fetches them; else null)
template <bool CAUSAL, bool VARLEN, bool SPLIT, int BR>
__device__ __forceinline__ FwdItem fwd_item(const FwdParams &p, int it, const int *cu_l = nullptr) {
    FwdItem x;
    const int BH = p.nbatch * p.Hq;
    const int rs = (int)fdiv((uint32_t)it, p.fd_bh);
    const int bh = it - rs * BH;
    // split-KV items are (rank, split) pairs in rank-major order
    const int rank = SPLIT ? (int)fdiv((uint32_t)rs, p.fd_split) : rs;
    x.sp = SPLIT ? rs - rank * p.nsplit : 0;
    x.b = (int)fdiv((uint32_t)bh, p.fd_hq);
    x.h = bh - x.b * p.Hq;
    if constexpr (VARLEN) {
        // the offsets are never written by the kernel: read them through the
        // constant address space, so they are scalar loads into SGPRs (and
        // take no part in the vector-load counter the tile waits rely on)
        typedef const __attribute__((address_space(4))) int cint;
        int qs, qe, ks, ke;
        if (cu_l != nullptr) {
            typedef int i32x4 __attribute__((ext_vector_type(4)));
            const i32x4 r = *reinterpret_cast<const i32x4 *>(cu_l + 4 * x.b);
            qs = __builtin_amdgcn_readfirstlane(r[0]);
            qe = __builtin_amdgcn_readfirstlane(r[1]);
            ks = __builtin_amdgcn_readfirstlane(r[2]);
            ke = __builtin_amdgcn_readfirstlane(r[3]);
        } else {
            cint *cq = (cint *)p.cu_q, *ck = (cint *)p.cu_k;
            qs = cq[x.b];
            qe = cq[x.b + 1];
            ks = ck[x.b];
            ke = ck[x.b + 1];
        }
        const bool ok = qs >= 0 && qe >= qs && qe <= p.total_q && ks >= 0 && ke >= ks &&
                        ke <= p.total_k;
        x.Sq = ok ? qe - qs : 0;
        x.Skv = ok ? ke - ks : 0;
        x.qrow0 = qs;
        x.krow0 = ks;
    } else {
        x.Sq = p.Sq;
        x.Skv = p.Skv;
        x.qrow0 = (int64_t)x.b * p.Sq;
        x.krow0 = (int64_t)x.b * p.Skv;
    }
    const int tile = CAUSAL ? (p.ntiles - 1 - rank) : rank;
    x.q0 = tile * BR;
    int kend = x.Skv;
    // one past the last key any row of the item may see (bottom-right causal)
    if (CAUSAL) kend = min(x.Skv, x.q0 + BR + (x.Skv - x.Sq));
    x.nt = (x.q0 < x.Sq && kend > 0) ? (kend + BC - 1) / BC : 0;
    x.t0 = 0;
    if constexpr (SPLIT) {
        // the tile's own key tiles cut into nsplit shares of equal length
        const int ct = (int)fdiv((uint32_t)(x.nt + p.nsplit - 1), p.fd_split);
        x.t0 = min(x.sp * ct, x.nt);
        x.nt = min(ct, x.nt - x.t0);
    }
    return x;
}

// The r-th of this workgroup's positions in a sequence of N items, or -1:
// one per row of gridDim.x positions (boustrophedon: position w in even rows,
// the mirror position, in steps of 8 so the item's head stays on this XCD,
// in odd rows), taken from the last row to the first.  fwd_walk_len is the
// number of them.
__device__ __forceinline__ int fwd_walk_len(int N) {
    const int G = gridDim.x, w = blockIdx.x;
    const int mirror = (G % 8 == 0) ? (G / 8 - 1 - w / 8) * 8 + (w % 8) : G - 1 - w;
    const int R = (N + G - 1) / G;                        // rows of G positions
    const bool last_ok = (int64_t)(R - 1) * G + (((R - 1) & 1) ? mirror : w) < N;
    return last_ok ? R : R - 1;                           // rows holding a position of w
}
__device__ __forceinline__ int fwd_walk_pos(int N, int r) {
    const int G = gridDim.x, w = blockIdx.x;
    const int mirror = (G % 8 == 0) ? (G / 8 - 1 - w / 8) * 8 + (w % 8) : G - 1 - w;
    const int nv = fwd_walk_len(N);
    if (r >= nv) return -1;
    const int row = nv - 1 - r;                           // the rows in reverse order
    return row * G + ((row & 1) ? mirror : w);
}
// The r-th item of this workgroup in the launcher's item order, or -1.
__device__ __forceinline__ int fwd_item_at(const FwdParams &p, int r) {
    return fwd_walk_pos(p.nitems, r);
}

// Ragged batch: this workgroup's items, in the order of its walk, listed in
// LDS (sm: kSchedSeqs + kSchedSeqs + kSchedLevels + kSchedItems ints; on
// return the kSchedLevels ints at sm + 2 * kSchedSeqs hold the offsets as
// fwd_item's cu_l).  The
// items with rows, (sequence, head, query tile j), are put in one order of
// falling cost: by j from the highest down (the causal key range of a tile
// ends at its last row, and only long sequences have high tiles), within
// one j the sequences with more query tiles first (ties by index), then the
// heads.  The positions of that order are dealt out as by fwd_walk_pos, so
// the persistent workgroups get nearly equal work however the lengths mix
// (the launcher's own order holds a slot for every tile of the longest
// sequence in every sequence).  Returns the number of items listed, or -1
// when they do not fit (then the launcher's order applies).  Every thread
// of the workgroup takes part; the list is complete on return.
template <bool CAUSAL, int BR>
__device__ int fwd_sched_build(const FwdParams &p, int *sm) {
    int *s_t = sm, *s_perm = sm + kSchedSeqs, *s_lev = sm + 2 * kSchedSeqs;
    int *s_list = s_lev + kSchedLevels;
    const int tid = threadIdx.x, nth = blockDim.x;
    const int nseq = p.nbatch, nlev = p.ntiles, H = p.Hq;
    // query tiles of each sequence (bad offsets: none, as fwd_item has it)
    for (int b = tid; b < nseq; b += nth) {
        const int qs = p.cu_q[b], qe = p.cu_q[b + 1], ks = p.cu_k[b], ke = p.cu_k[b + 1];
        const bool ok = qs >= 0 && qe >= qs && qe <= p.total_q && ks >= 0 && ke >= ks &&
                        ke <= p.total_k;
        s_t[b] = ok ? min((qe - qs + BR - 1) / BR, nlev) : 0;
    }
    __syncthreads();
    // the sequences by falling tile count (a rank sort), and per level j the
    // items of the levels above it, H * sum_b max(0, T_b - j - 1)
    for (int b = tid; b < nseq; b += nth) {
        const int t = s_t[b];
        int rank = 0;
        for (int c = 0; c < nseq; ++c) rank += (s_t[c] > t || (s_t[c] == t && c < b)) ? 1 : 0;
        s_perm[rank] = b;
    }
    for (int j = tid; j < nlev; j += nth) {
        int above = 0;
        for (int c = 0; c < nseq; ++c) above += max(0, s_t[c] - j - 1);
        s_lev[j] = above * H;
    }
    // N = H * sum_b T_b, summed by every wave alike
    int tiles = 0;
    for (int b = (int)(threadIdx.x & 63); b < nseq; b += 64) tiles += s_t[b];
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) tiles += __shfl_xor(tiles, sh, 64);
    const int N = __builtin_amdgcn_readfirstlane(tiles) * H;
    const int cnt = fwd_walk_len(N);
    __syncthreads();
    // (one decision for every workgroup: the longest list, one per row)
    if ((N + (int)gridDim.x - 1) / (int)gridDim.x > kSchedItems) return -1;
    for (int r = tid; r < cnt; r += nth) {
        const int q = fwd_walk_pos(N, r);
        // level of position q: the lowest j with s_lev[j] <= q (s_lev falls
        // with j; s_lev[nlev - 1] = 0)
        int lo = 0, hi = nlev - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (s_lev[mid] <= q) hi = mid;
            else lo = mid + 1;
        }
        const int i = q - s_lev[lo];
        const int k = i / H, h = i - k * H;
        // the launcher's item id, as fwd_item decodes it: rank, then
        // (sequence, head), where the rank is the query tile (from the last,
        // under the causal mask)
        const int rank = CAUSAL ? nlev - 1 - lo : lo;
        s_list[r] = rank * (nseq * H) + s_perm[k] * H + h;
    }
    __syncthreads();
    // the level table is done with: it now keeps a copy of the offsets for
    // the walk's item lookups (one LDS read instead of chains of scalar loads
    // at every item change), in the layout fwd_item takes
    static_assert(kSchedLevels >= 4 * kSchedSeqs, "room for the offset records");
    for (int b = tid; b < nseq; b += nth) {
        s_lev[4 * b] = p.cu_q[b];
        s_lev[4 * b + 1] = p.cu_q[b + 1];
        s_lev[4 * b + 2] = p.cu_k[b];
        s_lev[4 * b + 3] = p.cu_k[b + 1];
    }
    __syncthreads();
    return cnt;
}

template <int D, bool CAUSAL, bool VARLEN, bool SPLIT, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void attn_fwd_kernel(FwdParams p) {
    static_assert(!(VARLEN && SPLIT), "split-KV is for fixed batches");
    static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");
    constexpr int BR = 32 * NW;
    using L = FwdLay<D, NW>;
    __shared__ __attribute__((aligned(16))) __bf16 lds[NS * L::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;            // which half of the wave
    const int col = lane & 31;          // query row within the wave
    const int64_t hd_q = (int64_t)p.Hq * D;
    const int64_t hd_k = (int64_t)p.Hkv * D;

    auto item = [&](int r) { return fwd_item<CAUSAL, VARLEN, SPLIT, BR>(p, fwd_item_at(p, r)); };
    // next item after position r that has key tiles, or -1
    auto next_tiled = [&](int r) -> int {
        for (int s = r + 1;; ++s) {
            const int it = fwd_item_at(p, s);
            if (it < 0) return -1;
            if (fwd_item<CAUSAL, VARLEN, SPLIT, BR>(p, it).nt > 0) return s;
        }
    };

    // Direct-load plan: a tile's K rows (KS 16-byte slots each, the last one
    // padding that re-reads the row's last chunk) and V rows (VS slots, the
    // last four padding) are cut into wave-wide loads of 64 slots; lane L of
    // load n of a tensor fills slot 64n + L.
    auto load_index = [&](int pp, bool &isv) -> int {   // wave-uniform
        if (pp < L::KW) { isv = false; return wave + NW * pp; }
        if (pp < L::KW + L::VW) { isv = true; return wave + NW * (pp - L::KW); }
        if (wave < L::KR) { isv = false; return NW * L::KW + wave; }
        isv = true;
        if (wave < L::KR + L::VR) return NW * L::VW + wave - L::KR;
        return wave + NW * (L::VW - 1);
    };
    uint32_t goff[L::PER_WAVE];      // byte offset of this lane's chunk within a tile
    int ldo[L::PER_WAVE];            // LDS element offset of the load within a stage
#pragma unroll
    for (int pp = 0; pp < L::PER_WAVE; ++pp) {
        bool isv;
        const int n = load_index(pp, isv);
        const int slot = 64 * n + lane;
        const int row = isv ? slot / L::VS : slot / L::KS;
        const int colx = min(slot - row * (isv ? L::VS : L::KS), L::DS - 1) * 8;
        goff[pp] = (uint32_t)(row * hd_k + colx) * 2u;
        ldo[pp] = (isv ? L::K_ELEMS : 0) + 512 * n;
    }
    const bool last_is_v = wave >= L::KR;

    // The load stream: every tile of every item of this workgroup, in order,
    // numbered 0, 1, 2, ...; tile n goes to stage n % NS.  Once the stream
    // is exhausted each issue is a load over an empty range (it only writes
    // zeros to a free stage), so every issue adds the same number of loads
    // to the wave's counter and the waits below are fixed counts.
    int l_r = -1;            // item of the next tile (-1: stream exhausted)
    int l_tiles = 0;         // tiles of that item still to issue
    int l_keys = 0;          // valid keys from the next tile on
    int64_t l_off = 0;       // element offset of the next tile (K and V alike)
    int l_stage = 0;         // LDS element offset of the next tile's stage
    auto load_item = [&](int r) {
        l_r = r;
        if (r >= 0) {
            const FwdItem x = item(r);
            l_tiles = x.nt;
            l_keys = x.Skv - x.t0 * BC;
            l_off = (x.krow0 + (int64_t)x.t0 * BC) * hd_k + (int64_t)fdiv((uint32_t)x.h, p.fd_group) * D;
        }
    };
    auto issue_next = [&]() {
        __bf16 *dst = lds + l_stage;
        const __bf16 *kb = p.k, *vb = p.v;
        int nbytes = 0;
        if (l_r >= 0) {
            // the descriptors end at the last valid key, so rows past the
            // sequence end read as zeros
            const int rows = min(BC, l_keys);
            nbytes = (int)(((int64_t)(rows - 1) * hd_k + D) * 2);
            kb = p.k + l_off;
            vb = p.v + l_off;
            l_off += BC * hd_k;
            l_keys -= BC;
            if (--l_tiles == 0) load_item(next_tiled(l_r));
        }
        const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kb, nbytes);
        const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vb, nbytes);
#pragma unroll
        for (int pp = 0; pp < L::PER_WAVE; ++pp) {
            const bool isv = pp == L::PER_WAVE - 1 ? last_is_v : pp >= L::KW;
            buffer_lds_dma16(isv ? vr : kr, goff[pp], dst + ldo[pp]);
        }
        l_stage = l_stage == (NS - 1) * L::STAGE ? 0 : l_stage + L::STAGE;
    };

    // Q fragments (B operand of S^T = K Q^T), resident while an item runs.
    // The buffer descriptor covers this wave's valid rows only, so rows past
    // the sequence end load as zeros.
    bf16x8 qf[D / 16];
    auto load_q = [&](const FwdItem &x) {
        const int wr0 = x.q0 + 32 * wave;
        const int rows = min(32, x.Sq - wr0);
        const __bf16 *qb = p.q + (x.qrow0 + wr0) * hd_q + (int64_t)x.h * D;
        const int nbytes = rows > 0 ? (int)(((int64_t)(rows - 1) * hd_q + D) * 2) : 0;
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(rows > 0 ? qb : p.q, nbytes);
        const uint32_t off0 = (uint32_t)((col * hd_q + 8 * g) * 2);
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
            qf[t] = __builtin_bit_cast(bf16x8,
                                       __builtin_amdgcn_raw_buffer_load_b128(rq, off0 + 32 * t, 0, 0));
    };

    // LDS element offset of this lane's first operand in the stage of tile n.
    // Kept opaque so that each read is one address register plus an
    // immediate offset (otherwise the optimizer keeps one register per read).
    auto lane_base = [&](int n, int lane_off) -> int {
        int o = (n % NS) * L::STAGE + lane_off;
        asm volatile("" : "+v"(o));
        return o;
    };
    const int k_lane = col * L::KP + 8 * g;

    // S^T = K Q^T for one tile: two 32-key blocks, chains interleaved.
    auto scores = [&](int n, f32x16 (&s)[BC / 32]) {
        const __bf16 *ks = lds + lane_base(n, k_lane);
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int tt = 0; tt < D / 16; ++tt)
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
                s[kb] = mfma32x32x16(ld_lds_bf16x8(ks + 32 * kb * L::KP + 16 * tt), qf[tt], s[kb]);
    };

    f32x16 oacc[D / 32];
    float m = -__builtin_inff();     // reference max, scaled base-2 units
    float lsum = 0.f;                // this lane's share of the running sum
    const float c = p.c;

    // geometry of the item being computed (wave-uniform, except qr); kt0 is
    // the key offset of its first tile (split-KV shares), else 0
    int Skv = 0, off = 0, wrow0 = 0, qr = 0, ntw = 0, kt0 = 0;

    // Mask keys past each row's causal limit or past the sequence end; only
    // tiles that cross the diagonal or the end need it.
    auto mask = [&](int t, f32x16 (&s)[BC / 32]) {
        const int key0 = kt0 + t * BC;
        if (key0 + BC > Skv || (CAUSAL && key0 + BC - 1 > wrow0 + off)) {
            int lim = Skv - 1;
            if (CAUSAL) lim = min(lim, qr + off);
            lim -= key0 + 4 * g;                  // this lane's keys: key0 + 4g + const
            // opaque to the optimizer: otherwise it folds 4g into the 32
            // constants below and keeps them live (32 registers) across the loop
            asm volatile("" : "+v"(lim));
            // each score: compare into VCC, then select -inf.  Written as one
            // asm pair per score so the masks never pile up: left to itself
            // the compiler hoists all 32 compares and holds 32 lane masks in
            // scalar registers, which pushes other scalars out to memory
            const float ninf = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = s[kb][r];
                    asm volatile("v_cmp_gt_i32_e32 vcc, %2, %1\n\tv_cndmask_b32_e32 %0, %0, %3, vcc"
                                 : "+v"(x)
                                 : "v"(lim), "i"(32 * kb + 8 * (r >> 2) + (r & 3)), "v"(ninf)
                                 : "vcc");
                    s[kb][r] = x;
                }
        }
    };

    // Row max of tile j and the lazy update of the reference max: m only
    // moves when a row's tile max exceeds it by more than kRescaleSlack, so
    // weights stay <= 2^kRescaleSlack and the (rare) output rescale is a
    // uniform branch taken before the fused region below.
    auto row_max = [&](f32x16 (&s)[BC / 32]) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        const float mt = half_swap_max(mx) * c;   // tile row max, scaled log2 units
        const bool raise = mt > m + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? mt : m;
            const float alpha = m_new == -__builtin_inff() ? 1.f : fast_exp2(m - m_new);
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m = m_new;
        }
    };

    // lane coordinates for the transpose reads of V
    const int tr_e = (lane & 15) >> 2;       // row (key) within a 4-key group
    const int tr_s = lane & 3;               // 4-column slice
    const int tr_dh = (lane >> 4) & 1;       // which 16 columns of a 32-column block

    const int v_lane = L::K_ELEMS + (4 * g + tr_e) * L::VP + 16 * tr_dh + 4 * tr_s;
    // The fused part of a step is cut into groups separated by full
    // scheduling barriers, so that every LDS read is issued one group ahead
    // of the MFMAs that consume it (in-order issue would otherwise stall each
    // MFMA on its own read).  Group g of the score product covers d-slices
    // 2g, 2g+1 (FPG fragments); weight chunk g makes the pk[] entries of key
    // slices KPG*g .. KPG*g + KPG-1.
    constexpr int NG = D / 32;                   // score groups per tile
    constexpr int FPG = 2 * (BC / 32);           // K fragments per group
    constexpr int VPL = (BC / 2) / NG;           // weights per lane per chunk
    constexpr int NV = 2 * (D / 32);             // V transpose reads per key slice
    constexpr int KPG = (BC / 16) / NG;          // key slices per weight chunk
    static_assert(KPG * NG == BC / 16, "weight chunks must cover whole key slices");
    static_assert(VPL % 8 == 0, "a weight chunk must fill whole pk entries");
    auto read_k = [&](int n, int grp, bf16x8 (&kf)[FPG]) {
        const __bf16 *ks = lds + lane_base(n, k_lane);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
                kf[u * (BC / 32) + kb] = ld_lds_bf16x8(ks + 32 * kb * L::KP + 16 * (2 * grp + u));
    };
    auto mfma_k = [&](int grp, const bf16x8 (&kf)[FPG], f32x16 (&s)[BC / 32]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
                s[kb] = mfma32x32x16(kf[u * (BC / 32) + kb], qf[2 * grp + u], s[kb]);
    };
    auto weight_chunk = [&](int grp, f32x16 (&s)[BC / 32], bf16x8 (&pk)[BC / 16], float m_use,
                            float &rs) {
#pragma unroll
        for (int f = grp * VPL; f < (grp + 1) * VPL; ++f) {
            const int kb = f / 16, r = f % 16;
            s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
            rs += s[kb][r];
        }
#pragma unroll
        for (int kk = grp * VPL / 8; kk < (grp + 1) * VPL / 8; ++kk)
            pk[kk] = pack_p8(s[kk >> 1], 8 * (kk & 1));
    };
    auto read_v = [&](int n, int kk, s16x4 (&vf)[NV]) {
        const __bf16 *vs = lds + lane_base(n, v_lane);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            vf[2 * db] = lds_read_tr(vs + 16 * kk * L::VP + 32 * db);
            vf[2 * db + 1] = lds_read_tr(vs + (16 * kk + 8) * L::VP + 32 * db);
        }
    };
    auto mfma_v = [&](int kk, const s16x4 (&vf)[NV], const bf16x8 (&pk)[BC / 16]) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            oacc[db] = mfma32x32x16(concat_tr(vf[2 * db], vf[2 * db + 1]), pk[kk], oacc[db]);
    };

    int cn = 0;              // stream number of the tile being computed
    bool stores = false;     // output stores issued since the last full wait
    bool q_pend = false;     // query rows loaded during the previous step
    int nt = 0;              // key tiles of the current item
    int rA = -1, rB = -1;    // current item and the next one with key tiles
    int ntB = 0, ntwB = 0;   // key tiles of item rB, and this wave's share

    // Query rows are loaded one step ahead: at the end of a step whose next
    // step is the last one of its item Y (that last step computes the first
    // scores of the item after Y; this step's score MFMAs are done with qf).
    auto prefetch_q = [&](int rY) {
        const int rn = next_tiled(rY);
        if (rn >= 0) {
            load_q(item(rn));
            q_pend = true;
        }
    };

    // One pipeline step of item-local tile j (stream tile cn): wait for tile
    // cn+1, refill the stage of tile cn-1 with the next tile of the stream,
    // then the scores of tile cn+1 and O += P_j V_j on the matrix cores,
    // interleaved with the softmax of S_j.  scur holds S_j, snext receives the
    // scores of tile cn+1, which on the item's last tile is the first tile of
    // the next item (computed with that item's query rows).  j >= nt is a
    // no-op (the loop below is unrolled by two).
    auto step = [&](int j, f32x16 (&scur)[BC / 32], f32x16 (&snext)[BC / 32]) {
        if (j >= nt) return;
        // tile cn+1 complete (the query rows and tile cn+2 issued after it
        // may still be in flight; loads complete in order); after output
        // stores wait for everything, since stores and loads share the counter
        if (stores) wait_vmcnt<0>();
        else if (q_pend) wait_vmcnt<L::PER_WAVE + D / 16>();
        else wait_vmcnt<L::PER_WAVE>();
        stores = false;
        q_pend = false;
        lds_barrier();
        const bool last = j == nt - 1;
        // the item whose last step comes next, if any (-2: none)
        const int r_last = j + 1 == nt - 1 ? rA : (last && ntB == 1 ? rB : -2);
        if (j < ntw) {
            // the first K group of tile cn+1 loads during the mask and row max
            // (scores nobody needs are computed anyway; the stage read is
            // always in bounds)
            bf16x8 kf[2][FPG];
            read_k(cn + 1, 0, kf[0]);
            mask(j, scur);
            row_max(scur);
            __builtin_amdgcn_s_setprio(1);
            const float m_use = m == -__builtin_inff() ? 0.f : m;
            float rs = 0.f;
            bf16x8 pk[BC / 16];
            s16x4 vf[2 * KPG][NV];
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) snext[kb] = f32x16{};
            // group gr: the scores of tile cn+1 for d-slices 2gr, 2gr+1,
            // weight chunk gr of tile cn, and O += P V for the key slices
            // whose weights the previous chunk made, so the matrix products
            // of both halves share the groups with the softmax arithmetic
#pragma unroll
            for (int gr = 0; gr < NG; ++gr) {
                __builtin_amdgcn_sched_barrier(0);
                if (gr + 1 < NG) read_k(cn + 1, gr + 1, kf[(gr + 1) & 1]);
#pragma unroll
                for (int u = 0; u < KPG; ++u) read_v(cn, gr * KPG + u, vf[(gr & 1) * KPG + u]);
                mfma_k(gr, kf[gr & 1], snext);
                weight_chunk(gr, scur, pk, m_use, rs);
                if (gr > 0) {
#pragma unroll
                    for (int u = 0; u < KPG; ++u)
                        mfma_v((gr - 1) * KPG + u, vf[((gr - 1) & 1) * KPG + u], pk);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < KPG; ++u)
                mfma_v((NG - 1) * KPG + u, vf[((NG - 1) & 1) * KPG + u], pk);
            __builtin_amdgcn_sched_barrier(0);
            lsum += rs;
            __builtin_amdgcn_s_setprio(0);
        } else {
            // no tile of this item for this wave; it may still owe the first
            // scores of the next item
            if (last && ntwB > 0) {
                scores(cn + 1, snext);
            } else {
                // a placeholder, so that no score buffer stays live across steps
#pragma unroll
                for (int kb = 0; kb < BC / 32; ++kb)
                    snext[kb] = __builtin_nondeterministic_value(snext[kb]);
            }
        }
        // one load point for both paths (a load in each branch would be
        // merged by register copies that wait for the load at once).  It
        // comes before the tile load below: the compiler's wait for qf in the
        // next step then counts the tile loads as younger and lets them fly
        // (issued after them, it made every step wait for the newest tile).
        if (r_last != -2) prefetch_q(r_last);
        // the next tile of the stream goes into the stage of tile cn-1 (every
        // wave is past its last read, at the barrier above); issued after
        // the compute so that the MFMAs start right after the barrier
        issue_next();
        ++cn;
    };

    // Output of an item: O = acc / l (bf16), LSE = (m + log2 l) * ln 2.  With
    // zero set, the item has no keys: O = 0 and LSE = -inf.  The stores go
    // through buffer descriptors that end at this wave's last valid row, so
    // rows past the sequence end are dropped by the range check instead of a
    // per-lane branch (a divergent branch here would make the compiler treat
    // the item loop's state as per-lane).
    auto write_out = [&](const FwdItem &x, bool zero) {
        const int wr0 = x.q0 + 32 * wave;
        if (wr0 >= x.Sq) return;
        const int rows = min(32, x.Sq - wr0);
        const float lt = zero ? 0.f : half_swap_sum(lsum);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if constexpr (SPLIT) {
            // this split's share: the normalised output (fp32) and its
            // natural-log LSE, merged with the other shares by a second kernel
            const int64_t row0 = (((int64_t)x.sp * p.nbatch + x.b) * p.Hq + x.h) * x.Sq + wr0;
            const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(p.ws_o + row0 * D, rows * D * 4);
            const uint32_t oo = (uint32_t)((col * D + 4 * g) * 4);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const f32x4 v4 = {oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv,
                                      oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, zero ? f32x4{} : v4), ro,
                                                           oo + (32 * db + 8 * rq) * 4, 0, 0);
                }
            const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(p.ws_lse + row0, rows * 4);
            const float v = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -__builtin_inff();
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rl,
                                                  g == 0 ? (uint32_t)(col * 4) : 0x80000000u, 0, 0);
            return;
        }
        const __bf16 *ob = p.o + (x.qrow0 + wr0) * hd_q + (int64_t)x.h * D;
        const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(ob, (int)(((int64_t)(rows - 1) * hd_q + D) * 2));
        // A lane holds four runs of 4 columns of its row per 32-column block
        // (at 8q + 4g); swapping one run of each pair with the other half of
        // the wave gives every lane 8 consecutive columns (lower half: 16k +
        // 0..7, upper half: 16k + 8..15), so each row is written in 32-byte
        // pieces by 16-byte stores instead of 16-byte pieces by 8-byte ones
        const uint32_t oo = (uint32_t)((col * hd_q + 8 * g) * 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const f32x16 &a = oacc[db];
                const int r = 8 * k;
                const bf16x4 lo = zero ? bf16x4{} :
                    to_bf16x4(a[r] * inv, a[r + 1] * inv, a[r + 2] * inv, a[r + 3] * inv);
                const bf16x4 hi = zero ? bf16x4{} :
                    to_bf16x4(a[r + 4] * inv, a[r + 5] * inv, a[r + 6] * inv, a[r + 7] * inv);
                const u32x2 ul = __builtin_bit_cast(u32x2, lo), uh = __builtin_bit_cast(u32x2, hi);
                const auto s0 = __builtin_amdgcn_permlane32_swap(ul[0], uh[0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(ul[1], uh[1], false, false);
                const u32x4 v = {(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
                __builtin_amdgcn_raw_buffer_store_b128(v, ro, oo + (32 * db + 16 * k) * 2, 0, 0);
            }
        if (p.lse != nullptr) {
            int64_t l0;
            if constexpr (VARLEN) l0 = (int64_t)x.h * p.total_q + x.qrow0 + wr0;
            else l0 = ((int64_t)x.b * p.Hq + x.h) * x.Sq + wr0;
            const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(p.lse + l0, rows * 4);
            const float v = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -__builtin_inff();
            // one lane per row stores; the other half's offset is out of range
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rl,
                                                  g == 0 ? (uint32_t)(col * 4) : 0x80000000u, 0, 0);
        }
    };

    // key tiles of item x that this wave computes (its rows' causal reach)
    auto wave_tiles = [&](const FwdItem &x) -> int {
        const int w0 = x.q0 + 32 * wave;
        if (w0 >= x.Sq || x.nt == 0) return 0;
        int wk = x.Skv;
        if (CAUSAL) wk = min(x.Skv, min(w0 + 32, x.Sq) + (x.Skv - x.Sq));
        return wk > 0 ? min(x.nt, max((wk + BC - 1) / BC - x.t0, 0)) : 0;
    };
    // items after position r0 and before r1 (-1: to the end) that have rows
    // but no keys: O = 0, LSE = -inf
    auto write_empty = [&](int r0, int r1) {
        for (int r = r0 + 1; r1 < 0 || r < r1; ++r) {
            const int it = fwd_item_at(p, r);
            if (it < 0) break;
            const FwdItem x = fwd_item<CAUSAL, VARLEN, SPLIT, BR>(p, it);
            if (x.q0 < x.Sq && x.nt == 0) {
                write_out(x, true);
                stores = true;
            }
        }
    };
    // make item r current: its geometry, and the next item with key tiles
    auto enter = [&](int r) {
        rA = r;
        const FwdItem x = item(r);
        nt = x.nt;
        Skv = x.Skv;
        off = x.Skv - x.Sq;                       // bottom-right causal offset
        wrow0 = x.q0 + 32 * wave;                 // first row of this wave
        qr = wrow0 + col;                         // this lane's query row
        kt0 = x.t0 * BC;
        ntw = wave_tiles(x);
        rB = next_tiled(r);
        ntB = 0;
        ntwB = 0;
        if (rB >= 0) {
            const FwdItem y = item(rB);
            ntB = y.nt;
            ntwB = wave_tiles(y);
        }
    };

    // score buffers: a step reads scur only for tiles whose scores it wrote
    f32x16 sa[BC / 32], sb[BC / 32];
    const int r0 = next_tiled(-1);
    write_empty(-1, r0);
    if (r0 >= 0) {
        enter(r0);
        load_q(item(r0));
        load_item(r0);
        issue_next();
        issue_next();
        issue_next();
        // the first item's query rows and first tile have landed (its next
        // tiles may be in flight), visible to all waves
        if (stores) wait_vmcnt<0>();
        else wait_vmcnt<2 * L::PER_WAVE>();
        stores = false;
        lds_barrier();
        if (ntw > 0) {
            scores(cn, sa);
        } else {
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) sa[kb] = __builtin_nondeterministic_value(sa[kb]);
        }
        if (nt == 1) {
            // the first step is already the item's last: it needs the next
            // item's rows.  Here no tile load follows them, so wait for them
            // at once (this path only; elsewhere tile loads follow the rows,
            // and the compiler's waits for qf then let those tiles fly)
            prefetch_q(rA);
            wait_vmcnt<0>();
        }
    }
    while (rA >= 0) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
        m = -__builtin_inff();
        lsum = 0.f;
        // unrolled by two so the score buffers alternate without copies
        for (int j = 0; j < nt; j += 2) {
            step(j, sa, sb);
            step(j + 1, sb, sa);
        }
        // the next item's first scores are in sb after an odd tile count
        if (nt & 1) {
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) sa[kb] = sb[kb];
        }
        write_out(item(rA), false);
        stores = true;
        write_empty(rA, rB);
        if (rB < 0) break;
        enter(rB);
    }
    wait_vmcnt<0>();                 // no load may outlive the workgroup
}

// Ping-pong prefill (8 waves, fixed or ragged batches, no key split).
//
// The waves form two groups of four, waves 0-3 and 4-7; a SIMD holds one
// wave of each.  Every key tile takes each wave through two phases, one
// workgroup barrier after each:
//  * an MFMA phase M(n): the scores of stream tile n+1 (S^T = K Q^T) and
//    O += P_n V_n, with the operand reads of each group of MFMAs issued one
//    group ahead;
//  * a softmax phase S(n+1): mask, row max, exponentials and the weights
//    P_{n+1} (bf16), on the vector ALUs only.
// Group B runs one phase behind group A, so on every SIMD one wave's
// exponentials run while the other wave's MFMAs run: the matrix products of
// one tile hide the softmax of another (lecompute.fr, "FlashAttention-4 :
// limites du calcul matriciel", section "Faire avancer plusieurs tuiles sans
// écraser leurs données", where two tiles alternate between the units).
//
// Tile loads go out spread over the MFMA phases, where the vector ALUs are
// idle, and are waited for a whole step later (details at the walk below).
//
// EMU > 0: of each lane's 32 exponentials per key tile, EMU (every 32/EMU-th)
// are computed by the polynomial of exp2_poly.h on the FMA path instead of
// the hardware exponential (the same page, section "Déplacer une partie des
// exponentielles").
template <int D, bool CAUSAL, bool VARLEN, int NS_, bool POISON, int EMU = 0>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_pp_kernel(FwdParams p) {
    static_assert(NS_ >= 3 && NS_ <= 4, "the schedule needs tiles n, n+1 and a free stage");
    static_assert(EMU >= 0 && EMU <= 32 && (EMU == 0 || 32 % EMU == 0), "a whole share of the 32");
    constexpr int NW = 8;
    constexpr int BR = 32 * NW;
    using L = FwdLay<D, NW>;
    // the K/V ring, then (ragged batches) the item list: one LDS object, so
    // the compiler keeps no alias scopes that would make it wait for every
    // tile load before the next LDS read (the walk orders those itself)
    constexpr int SCHED_INTS = VARLEN ? 2 * kSchedSeqs + kSchedLevels + kSchedItems : 0;
    __shared__ __attribute__((aligned(16))) __bf16 lds[NS_ * L::STAGE + 2 * SCHED_INTS];
    int *const sched = reinterpret_cast<int *>(lds + NS_ * L::STAGE);
    static_assert((NS_ * L::STAGE) % 8 == 0 && kSchedSeqs % 4 == 0, "16-byte offset records");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool grp_b = wave >= 4;
    // the r-th item of this workgroup: from its LDS list (a ragged batch on
    // a persistent grid), else in the launcher's order
    int n_listed = -1;
    if constexpr (VARLEN) {
        if (p.compact) n_listed = fwd_sched_build<CAUSAL, BR>(p, sched);
    }
    const int *const listed = sched + 2 * kSchedSeqs + kSchedLevels;
    const int *const cu_l = VARLEN && n_listed >= 0 ? sched + 2 * kSchedSeqs : nullptr;
    auto at = [&](int r) -> int {
        if constexpr (VARLEN) {
            if (n_listed >= 0) return r < n_listed ? listed[r] : -1;
        }
        return fwd_item_at(p, r);
    };
    auto item_of = [&](int it) { return fwd_item<CAUSAL, VARLEN, false, BR>(p, it, cu_l); };
    // the item's 32-row blocks alternate between the groups, so both groups
    // meet the causal diagonal alike
    const int rblk = grp_b ? 2 * (wave - 4) + 1 : 2 * wave;
    const int g = lane >> 5;
    const int col = lane & 31;
    const int64_t hd_q = (int64_t)p.Hq * D;
    const int64_t hd_k = (int64_t)p.Hkv * D;

    auto item = [&](int r) { return item_of(at(r)); };
    // the next position after r whose item has key tiles (-1: none), and
    // that item, decoded once for the caller
    auto next_tiled = [&](int r, FwdItem &x) -> int {
        for (int s = r + 1;; ++s) {
            const int it = at(s);
            if (it < 0) return -1;
            x = item_of(it);
            if (x.nt > 0) return s;
        }
    };

    // ---- the load stream (as in attn_fwd_kernel): every tile of every item
    // of this workgroup, tile n into stage n % NS_
    auto load_index = [&](int pp, bool &isv) -> int {
        if (pp < L::KW) { isv = false; return wave + NW * pp; }
        if (pp < L::KW + L::VW) { isv = true; return wave + NW * (pp - L::KW); }
        if (wave < L::KR) { isv = false; return NW * L::KW + wave; }
        isv = true;
        if (wave < L::KR + L::VR) return NW * L::VW + wave - L::KR;
        return wave + NW * (L::VW - 1);
    };
    uint32_t goff[L::PER_WAVE];
    int ldo[L::PER_WAVE];
#pragma unroll
    for (int pp = 0; pp < L::PER_WAVE; ++pp) {
        bool isv;
        const int n = load_index(pp, isv);
        const int slot = 64 * n + lane;
        const int row = isv ? slot / L::VS : slot / L::KS;
        const int colx = min(slot - row * (isv ? L::VS : L::KS), L::DS - 1) * 8;
        goff[pp] = (uint32_t)(row * hd_k + colx) * 2u;
        ldo[pp] = (isv ? L::K_ELEMS : 0) + 512 * n;
    }
    const bool last_is_v = wave >= L::KR;
    int l_r = -1, l_tiles = 0, l_keys = 0, l_stage = 0;
    int64_t l_off = 0;
    auto load_item = [&](int r, const FwdItem &x) {
        l_r = r;
        if (r >= 0) {
            l_tiles = x.nt;
            l_keys = x.Skv;
            l_off = x.krow0 * hd_k + (int64_t)fdiv((uint32_t)x.h, p.fd_group) * D;
        }
    };
    // The next tile of the stream: issue_begin() advances the stream and
    // makes the tile's descriptors, issue_part(pp) issues this wave's load
    // pp of it (PER_WAVE loads per tile); issue_next() does both at once.
    __amdgpu_buffer_rsrc_t t_kr, t_vr;
    __bf16 *t_dst = lds;
    // (issue_begin touches no memory, so it may run before the barrier
    // that frees the stage; issue_part only after it)
    auto issue_begin = [&]() {
        t_dst = lds + l_stage;
        const __bf16 *kb = p.k, *vb = p.v;
        int nbytes = 0;
        if (l_r >= 0) {
            const int rows = min(BC, l_keys);
            nbytes = (int)(((int64_t)(rows - 1) * hd_k + D) * 2);
            kb = p.k + l_off;
            vb = p.v + l_off;
            l_off += BC * hd_k;
            l_keys -= BC;
            if (--l_tiles == 0) {
                FwdItem x;
                const int r = next_tiled(l_r, x);
                load_item(r, x);
            }
        }
        t_kr = buffer_rsrc(kb, nbytes);
        t_vr = buffer_rsrc(vb, nbytes);
        l_stage = l_stage == (NS_ - 1) * L::STAGE ? 0 : l_stage + L::STAGE;
    };
    auto issue_part = [&](int pp) {
        if constexpr (POISON) {
            if (pp == 0) {
                // debug: fill what this wave's loads are about to overwrite
                // with NaN first, so a read of a stage before its loads land
                // (or after it was handed back to the loads) gives NaN
                // instead of old data
                const u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
#pragma unroll
                for (int q = 0; q < L::PER_WAVE; ++q) st_lds16(t_dst + ldo[q] + 8 * lane, nan4);
                wait_lgkmcnt0();
            }
        }
        const bool isv = pp == L::PER_WAVE - 1 ? last_is_v : pp >= L::KW;
        buffer_lds_dma16(isv ? t_vr : t_kr, goff[pp], t_dst + ldo[pp]);
    };
    auto issue_next = [&]() {
        issue_begin();
#pragma unroll
        for (int pp = 0; pp < L::PER_WAVE; ++pp) issue_part(pp);
    };

    // ---- query rows (B operand of S^T = K Q^T): qf for the item whose
    // scores the MFMA phases compute, qn loaded ahead for the next item.  qf
    // is only ever written by a register copy from qn, so no MFMA phase
    // waits for a load
    bf16x8 qf[D / 16], qn[D / 16];
    auto load_q = [&](const FwdItem &x, bf16x8 (&q)[D / 16]) {
        const int wr0 = x.q0 + 32 * rblk;
        const int rows = min(32, x.Sq - wr0);
        const __bf16 *qb = p.q + (x.qrow0 + wr0) * hd_q + (int64_t)x.h * D;
        const int nbytes = rows > 0 ? (int)(((int64_t)(rows - 1) * hd_q + D) * 2) : 0;
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(rows > 0 ? qb : p.q, nbytes);
        const uint32_t off0 = (uint32_t)((col * hd_q + 8 * g) * 2);
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
            q[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off0 + 32 * t, 0, 0));
    };

    auto lane_base = [&](int n, int lane_off) -> int {
        int o = (n % NS_) * L::STAGE + lane_off;
        asm volatile("" : "+v"(o));
        return o;
    };
    const int k_lane = col * L::KP + 8 * g;
    const int tr_e = (lane & 15) >> 2, tr_s = lane & 3, tr_dh = (lane >> 4) & 1;
    const int v_lane = L::K_ELEMS + (4 * g + tr_e) * L::VP + 16 * tr_dh + 4 * tr_s;

    f32x16 oacc[D / 32];
    f32x16 s[BC / 32];               // scores of the tile whose softmax comes next
    bf16x8 pk[BC / 16];              // weights of the tile whose P V comes next
    float m = -__builtin_inff(), lsum = 0.f;
    const float c = p.c;

    // ---- per-wave view of the item of tile n (the one being softmaxed and
    // then multiplied with V) and of the item of tile n+1
    struct View {
        int r;                // item position in this workgroup's walk (-1: none)
        int nt, ntw;          // its key tiles, and those this wave computes
        int Skv, off, wrow0, qr;
    };
    auto wave_tiles = [&](const FwdItem &x) -> int {
        const int w0 = x.q0 + 32 * rblk;
        if (w0 >= x.Sq || x.nt == 0) return 0;
        int wk = x.Skv;
        if (CAUSAL) wk = min(x.Skv, min(w0 + 32, x.Sq) + (x.Skv - x.Sq));
        return wk > 0 ? min(x.nt, (wk + BC - 1) / BC) : 0;
    };
    auto make_view = [&](int r, const FwdItem &x) {
        View v;
        v.r = r;
        v.nt = v.ntw = v.Skv = v.off = v.wrow0 = v.qr = 0;
        if (r >= 0) {
            v.nt = x.nt;
            v.ntw = wave_tiles(x);
            v.Skv = x.Skv;
            v.off = x.Skv - x.Sq;
            v.wrow0 = x.q0 + 32 * rblk;
            v.qr = v.wrow0 + col;
        }
        return v;
    };

    // items after position r0 and before r1 (-1: to the end) with rows but
    // no keys: O = 0, LSE = -inf
    auto write_rows = [&](const FwdItem &x, bool zero) {
        const int wr0 = x.q0 + 32 * rblk;
        if (wr0 >= x.Sq) return;
        const int rows = min(32, x.Sq - wr0);
        const float lt = zero ? 0.f : half_swap_sum(lsum);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const __bf16 *ob = p.o + (x.qrow0 + wr0) * hd_q + (int64_t)x.h * D;
        const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(ob, (int)(((int64_t)(rows - 1) * hd_q + D) * 2));
        const uint32_t oo = (uint32_t)((col * hd_q + 8 * g) * 2);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const f32x16 &a = oacc[db];
                const int r = 8 * k;
                const bf16x4 lo = zero ? bf16x4{} :
                    to_bf16x4(a[r] * inv, a[r + 1] * inv, a[r + 2] * inv, a[r + 3] * inv);
                const bf16x4 hi = zero ? bf16x4{} :
                    to_bf16x4(a[r + 4] * inv, a[r + 5] * inv, a[r + 6] * inv, a[r + 7] * inv);
                const u32x2 ul = __builtin_bit_cast(u32x2, lo), uh = __builtin_bit_cast(u32x2, hi);
                const auto s0 = __builtin_amdgcn_permlane32_swap(ul[0], uh[0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(ul[1], uh[1], false, false);
                const u32x4 v = {(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
                __builtin_amdgcn_raw_buffer_store_b128(v, ro, oo + (32 * db + 16 * k) * 2, 0, 0);
            }
        if (p.lse != nullptr) {
            int64_t l0;
            if constexpr (VARLEN) l0 = (int64_t)x.h * p.total_q + x.qrow0 + wr0;
            else l0 = ((int64_t)x.b * p.Hq + x.h) * x.Sq + wr0;
            const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(p.lse + l0, rows * 4);
            const float v = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -__builtin_inff();
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rl,
                                                  g == 0 ? (uint32_t)(col * 4) : 0x80000000u, 0, 0);
        }
    };
    auto write_empty = [&](int r0, int r1) {
        for (int r = r0 + 1; r1 < 0 || r < r1; ++r) {
            const int it = at(r);
            if (it < 0) break;
            const FwdItem x = item_of(it);
            if (x.q0 < x.Sq && x.nt == 0) write_rows(x, true);
        }
    };

    // The MFMA phase as one fixed sequence of 2*NOPS operations, score and
    // P V MFMAs alternating; every operand fragment is read RING operations
    // ahead into a ring of fragment registers, so each read has RING-1 MFMAs
    // of time to land.  Score op i: key block i % 2, d-slice i / 2 (the same
    // accumulation order as a plain loop over d); P V op i: key slice
    // i / (D / 32), output block i % (D / 32).
    constexpr int NSOP = 2 * (D / 16);           // score MFMAs (two key blocks)
    constexpr int NPOP = (BC / 16) * (D / 32);   // P V MFMAs
    static_assert(NSOP == NPOP, "score and P V MFMAs alternate one for one");
    constexpr int NOPS = NSOP;
    constexpr int RING = 8;
    // the tile loads of an MFMA phase (ld = PER_WAVE, or 0 for none): one
    // every LD_EVERY operations
    constexpr int LD_EVERY = (2 * NOPS) / L::PER_WAVE;
    static_assert(LD_EVERY >= 1, "every load finds its operation");
    auto mphase_t = [&](auto ds, auto dpv, int n, auto ld) {
        constexpr bool DS = decltype(ds)::value, DPV = decltype(dpv)::value;
        constexpr int NLD = decltype(ld)::value;
        __builtin_amdgcn_s_setprio(1);
        const __bf16 *ks = lds + lane_base(n + 1, k_lane);
        const __bf16 *vs = lds + lane_base(n, v_lane);
        // operation o of the sequence: o even -> score op o/2, odd -> P V op o/2
        auto valid = [&](int o) { return (o & 1) ? DPV : DS; };
        bf16x8 fr[RING];
        auto read = [&](int o) {
            const int i = o >> 1;
            if (o & 1) {
                const int kk = i / (D / 32), db = i % (D / 32);
                fr[o % RING] = concat_tr(lds_read_tr(vs + 16 * kk * L::VP + 32 * db),
                                         lds_read_tr(vs + (16 * kk + 8) * L::VP + 32 * db));
            } else {
                const int kb = i & 1, t = i >> 1;
                fr[o % RING] = ld_lds_bf16x8(ks + 32 * kb * L::KP + 16 * t);
            }
        };
        if constexpr (DS) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) s[kb] = f32x16{};
        }
#pragma unroll
        for (int o = 0; o < RING; ++o)
            if (valid(o)) read(o);
#pragma unroll
        for (int o = 0; o < 2 * NOPS; ++o) {
            __builtin_amdgcn_sched_barrier(0);
            const int i = o >> 1;
            if (valid(o)) {
                if (o & 1) {
                    const int kk = i / (D / 32), db = i % (D / 32);
                    oacc[db] = mfma32x32x16(fr[o % RING], pk[kk], oacc[db]);
                } else {
                    const int kb = i & 1, t = i >> 1;
                    s[kb] = mfma32x32x16(fr[o % RING], qf[t], s[kb]);
                }
            }
            if (NLD > 0 && o % LD_EVERY == 0 && o / LD_EVERY < NLD) issue_part(o / LD_EVERY);
            if (o + RING < 2 * NOPS && valid(o + RING)) read(o + RING);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
    };
    typedef std::integral_constant<bool, true> T_;
    typedef std::integral_constant<bool, false> F_;
    typedef std::integral_constant<int, 0> LD0_;
    typedef std::integral_constant<int, L::PER_WAVE> LDW_;

    // ---- the softmax phase of tile n (item-local index j of view v)
    auto sphase = [&](const View &v, int j) {
        const int key0 = j * BC;
        if (key0 + BC > v.Skv || (CAUSAL && key0 + BC - 1 > v.wrow0 + v.off)) {
            int lim = v.Skv - 1;
            if (CAUSAL) lim = min(lim, v.qr + v.off);
            lim -= key0 + 4 * g;
            asm volatile("" : "+v"(lim));
            const float ninf = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = s[kb][r];
                    asm volatile("v_cmp_gt_i32_e32 vcc, %2, %1\n\tv_cndmask_b32_e32 %0, %0, %3, vcc"
                                 : "+v"(x)
                                 : "v"(lim), "i"(32 * kb + 8 * (r >> 2) + (r & 3)), "v"(ninf)
                                 : "vcc");
                    s[kb][r] = x;
                }
        }
        float mx = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        const float mt = half_swap_max(mx) * c;
        const bool raise = mt > m + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? mt : m;
            const float alpha = m_new == -__builtin_inff() ? 1.f : fast_exp2(m - m_new);
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m = m_new;
        }
        const float m_use = m == -__builtin_inff() ? 0.f : m;
        float rs = 0.f;
#pragma unroll
        for (int f = 0; f < 32; ++f) {
            const int kb = f >> 4, r = f & 15;
            const float x = __builtin_fmaf(s[kb][r], c, -m_use);
            if constexpr (EMU > 0) {
                s[kb][r] = f % (32 / EMU) == 32 / EMU - 1 ? exp2_poly(x) : fast_exp2(x);
            } else {
                s[kb][r] = fast_exp2(x);
            }
            rs += s[kb][r];
        }
#pragma unroll
        for (int kk = 0; kk < BC / 16; ++kk) pk[kk] = pack_p8(s[kk >> 1], 8 * (kk & 1));
        lsum += rs;
    };

    // ---- walk.  Every wave runs the same sequence S(n), M(n) over the
    // stream's tiles n, with a barrier after each; group B starts one
    // barrier late (it idles through A's first MFMA phase) and group A ends
    // one barrier late.  cur is the item of tile n, nx the next one with key
    // tiles.
    //
    // Phases: group A runs S(n) in phase 2n+1 and M(n) in phase 2n+2, group
    // B one phase later.  Tile t is read by the MFMA phases M(t-1) (its keys)
    // and M(t) (its values): first in phase 2t (A's M(t-1)), last in phase
    // 2t+3 (B's M(t)).
    // Tile loads: the first NS_-1 tiles go out before the first barrier; then
    // every wave issues its share of tile n+NS_-1 during its M(n), spread
    // over the MFMAs, into the stage of tile n-1, whose last reader, B's
    // M(n-1), ran in phase 2n+1, before A's M(n) (phase 2n+2) and B's (2n+3).
    // The descriptors are made at the end of the softmax phase before (the
    // scalar unit is idle there).  At the end of M(n) a wave waits for all
    // its loads but tile n+NS_-1's, i.e. for tile n+NS_-2 (issued in
    // M(n-1)), which is first read in phase 2n+2*NS_-4: after the barrier
    // that ends B's M(n) (phase 2n+3) when NS_ = 4.  With NS_ = 3 it is tile
    // n+2 itself, first read in phase 2n+4, so there the wait takes every
    // load.
    // Rows: qf holds those of the item whose tiles the MFMA phases score,
    // qn those of sq1, the next item with key tiles.  Once the scores of the
    // former's last tile are issued, qf takes qn's rows and qn is refilled.
    int sq1 = -1;
    auto rows_advance = [&]() {
#pragma unroll
        for (int t = 0; t < D / 16; ++t) qf[t] = qn[t];
        FwdItem x;
        sq1 = sq1 >= 0 ? next_tiled(sq1, x) : -1;
        if (sq1 >= 0) load_q(x, qn);
    };

    FwdItem x0, x1;
    const int r0 = next_tiled(-1, x0);
    write_empty(-1, r0);
    if (r0 < 0) {
        wait_vmcnt<0>();
        return;
    }
    View cur = make_view(r0, x0);
    const int r1 = next_tiled(r0, x1);
    View nx = make_view(r1, x1);
    sq1 = nx.r;
    // At the start every workgroup loads at once: only r0's rows and tiles
    // 0 .. NS_-2 go out before the first barrier (tile 0 is waited for
    // there); the next item's rows follow after it, under the first MFMA
    // phase, and tile 1 is waited for after that phase, ahead of the
    // barrier before the first M(0)
    load_q(x0, qf);
    load_item(r0, x0);
    for (int i = 0; i < NS_ - 1; ++i) issue_next();
    wait_vmcnt<(NS_ - 2) * L::PER_WAVE>();
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    lds_barrier();
    if (grp_b) lds_barrier();            // B idles through A's M(-1)
    if (sq1 >= 0) load_q(x1, qn);
    // M(-1): the scores of tile 0
    mphase_t(T_{}, F_{}, -1, LD0_{});
    if (sq1 >= 0) wait_vmcnt<D / 16 + (NS_ - 3) * L::PER_WAVE>();
    else wait_vmcnt<(NS_ - 3) * L::PER_WAVE>();
    if (cur.nt == 1) rows_advance();     // tile 0 was r0's last
    lds_barrier();

    int jn = 0;                          // index of tile n in cur
    for (int n = 0;; ++n) {
        // S(n): the weights of tile n (zero weights for a tile past this
        // wave's rows, so the P V below adds exactly nothing); then the
        // descriptors of tile n+NS_-1
        const bool same = jn + 1 < cur.nt;
        if (jn < cur.ntw) {
            sphase(cur, jn);
        } else {
#pragma unroll
            for (int kk = 0; kk < BC / 16; ++kk) pk[kk] = bf16x8{};
        }
        issue_begin();
        lds_barrier();
        // M(n): the scores of tile n+1 and O += P_n V_n (one branch-free
        // body: scores nobody needs are computed anyway, and a P V of zero
        // weights adds nothing), with the loads of tile n+NS_-1; then tile
        // n+NS_-2 completes.  Loads complete in the order they were issued,
        // so at most PER_WAVE outstanding operations means every load but
        // the last PER_WAVE done; output stores in between share the
        // counter, but only ever add to it.
        mphase_t(T_{}, T_{}, n, LDW_{});
        if (NS_ == 3) wait_vmcnt<0>();
        else wait_vmcnt<L::PER_WAVE>();
        // tile n+1, just scored, the last of its item: the next MFMA phase
        // scores the next item's first tile
        if (same ? jn + 2 == cur.nt : nx.nt == 1) rows_advance();
        lds_barrier();
        // on to tile n+1: past the end of cur, write its output (its last
        // P V was this wave's M(n)) and enter the next item
        if (same) {
            ++jn;
        } else {
            write_rows(item(cur.r), false);
            write_empty(cur.r, nx.r);
            if (nx.r < 0) break;
            cur = nx;
            jn = 0;
            m = -__builtin_inff();
            lsum = 0.f;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
            FwdItem xn;
            const int rn = next_tiled(cur.r, xn);
            nx = make_view(rn, xn);
        }
    }
    if (!grp_b) lds_barrier();           // A's barrier for B's last phase
    wait_vmcnt<0>();                     // no load may outlive the workgroup
}


// Merge of the split-KV shares, one wave per query row: LSE = M + log(sum_s
// exp(lse_s - M)), O = sum_s exp(lse_s - LSE) O_s (the decode merge, per row).
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_merge_kernel(FwdParams p) {
    constexpr int PER = D / 64;
    const int64_t rows = (int64_t)p.nbatch * p.Hq * p.Sq;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (b, h, i)
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const float *lse_p = p.ws_lse + row;
    float M = -__builtin_inff();
    for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, lse_p[s * rows]);
    const float Mu = M == -__builtin_inff() ? 0.f : M;
    float tot = 0.f;
    for (int s = 0; s < p.nsplit; ++s) tot += fast_exp2((lse_p[s * rows] - Mu) * kLog2e);
    const float lse = tot > 0.f ? Mu + fast_log2(tot) * kLn2 : -__builtin_inff();
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    if (tot > 0.f) {
        const float *o_p = p.ws_o + row * D + PER * lane;
        for (int s = 0; s < p.nsplit; ++s) {
            const float w = fast_exp2((lse_p[s * rows] - lse) * kLog2e);
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += w * o_p[s * rows * D + e];
        }
    }
    // row = (b * Hq + h) * Sq + i; O is [B, Sq, Hq, d], LSE [B, Hq, Sq]
    const int64_t i = row % p.Sq, bh = row / p.Sq;
    const int64_t b = bh / p.Hq, h = bh % p.Hq;
    __bf16 *op = p.o + ((b * p.Sq + i) * p.Hq + h) * D + PER * lane;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[e] = (__bf16)acc[e];
    if (p.lse != nullptr && lane == 0) p.lse[row] = lse;
}

// The fixed-batch ping-pong kernel with `share` of each lane's 32
// exponentials per tile on the polynomial (4, 8 or 16), on `grid` workgroups.
template <int D, bool CAUSAL>
hipError_t launch_poly(const FwdParams &p, int share, int grid, hipStream_t s) {
    const dim3 g((unsigned)grid), b(512);
    switch (share) {
    case 4:
        hipLaunchKernelGGL((attn_fwd_pp_kernel<D, CAUSAL, false, NS, false, 4>), g, b, 0, s, p);
        break;
    case 8:
        hipLaunchKernelGGL((attn_fwd_pp_kernel<D, CAUSAL, false, NS, false, 8>), g, b, 0, s, p);
        break;
    case 16:
        hipLaunchKernelGGL((attn_fwd_pp_kernel<D, CAUSAL, false, NS, false, 16>), g, b, 0, s, p);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN, bool SPLIT, int NW = 8>
hipError_t launch_t(const FwdParams &p_in, hipStream_t s, int exp2_poly = 0) {
    FwdParams p = p_in;
    // the host counts 256-row tiles; the 4-wave variant has 128-row ones (a
    // ragged batch: twice the count, an upper bound for every sequence; the
    // items past a sequence's end have no rows and end at once)
    if constexpr (NW == 4) p.ntiles = VARLEN ? 2 * p_in.ntiles : (p.Sq + 127) / 128;
    const int64_t items = (int64_t)p.ntiles * p.nbatch * p.Hq * (SPLIT ? p.nsplit : 1);
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffff) return hipErrorInvalidConfiguration;
    p.nitems = (int)items;
    p.fd_bh = make_fastdiv((uint32_t)(p.nbatch * p.Hq));
    p.fd_hq = make_fastdiv((uint32_t)p.Hq);
    p.fd_group = make_fastdiv((uint32_t)p.group);
    p.fd_split = make_fastdiv((uint32_t)(SPLIT ? p.nsplit : 1));
    int grid = p.nitems;
    if constexpr (VARLEN && NW == 8) {
        // fewer 256-row items than CUs: 128-row items on 4-wave workgroups
        int cus = 0;
        const hipError_t e = current_cu_count(&cus);
        if (e != hipSuccess) return e;
        if (cus > 0 && items < cus) return launch_t<D, CAUSAL, VARLEN, SPLIT, 4>(p_in, s);
        // a persistent grid, one workgroup per CU, whose load stream runs
        // across items instead of a workgroup per item: over a cost-sorted
        // list of the items with rows where it fits the LDS bounds, else for
        // short sequences only (at most two tiles per item, so a static walk
        // over the launcher's order stays balanced)
        if (cus > 0 && p.nbatch <= kSchedSeqs && p.ntiles <= kSchedLevels &&
            items <= (int64_t)kSchedItems * cus) {
            grid = cus;
            p.compact = 1;
        } else if (cus > 0 && p.max_len <= 512) {
            grid = cus;
        }
    }
    if constexpr (!VARLEN) {
        // one workgroup per CU (the LDS ring allows no more), each walking
        // its share of the items
        int cus = 0;
        const hipError_t e = current_cu_count(&cus);
        if (e != hipSuccess) return e;
        if constexpr (NW == 8 && !SPLIT) {
            // the polynomial share of the exponentials: the ping-pong kernel
            // at every grid size (it walks any number of items per workgroup)
            if (exp2_poly > 0) return launch_poly<D, CAUSAL>(p, exp2_poly, cus > 0 && grid > cus ? cus : grid, s);
            // fewer 256-row items than CUs: 128-row items on 4-wave
            // workgroups occupy more CUs (one wave per SIMD instead of two)
            if (cus > 0 && items < cus && p.Sq > 128)
                return launch_t<D, CAUSAL, VARLEN, SPLIT, 4>(p_in, s);
        }
        if (cus > 0 && grid > cus) grid = cus;
    }
    // the ping-pong kernel, except for fixed batches at d = 64, where a phase
    // has half the MFMAs to hide the same barrier and descriptor work and the
    // single-group kernel measured faster on short causal shapes (3-10 %,
    // within 1.5 % the other way on long or non-causal ones; the same bits)
    if constexpr (NW == 8 && !SPLIT && (D == 128 || VARLEN)) {
        // debug builds of the fixed-batch path (see the C ABI's ATTN_DEBUG):
        // NaN-poisoned stages, the shallowest ring the pipeline allows, or
        // both
        if (!VARLEN && (p.debug & 6) == 6)
            hipLaunchKernelGGL((attn_fwd_pp_kernel<D, CAUSAL, false, 3, true>),
                               dim3((unsigned)grid), dim3(64 * NW), 0, s, p);
        else if (!VARLEN && (p.debug & 4))
            hipLaunchKernelGGL((attn_fwd_pp_kernel<D, CAUSAL, false, 3, false>),
                               dim3((unsigned)grid), dim3(64 * NW), 0, s, p);
        else if (!VARLEN && (p.debug & 2))
            hipLaunchKernelGGL((attn_fwd_pp_kernel<D, CAUSAL, false, NS, true>),
                               dim3((unsigned)grid), dim3(64 * NW), 0, s, p);
        else
            hipLaunchKernelGGL((attn_fwd_pp_kernel<D, CAUSAL, VARLEN, NS, false>),
                               dim3((unsigned)grid), dim3(64 * NW), 0, s, p);
    } else
        hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, VARLEN, SPLIT, NW>), dim3((unsigned)grid),
                           dim3(64 * NW), 0, s, p);
    hipError_t e = hipGetLastError();
    if (!SPLIT || e != hipSuccess) return e;
    const int64_t rows = (int64_t)p.nbatch * p.Hq * p.Sq;
    hipLaunchKernelGGL(attn_fwd_merge_kernel<D>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams &p, int d, bool causal, bool varlen, hipStream_t s,
                      int exp2_poly) {
    if (varlen && exp2_poly != 0) return hipErrorInvalidValue;
    if (d == 128) {
        if (varlen)
            return causal ? launch_t<128, true, true, false>(p, s) : launch_t<128, false, true, false>(p, s);
        return causal ? launch_t<128, true, false, false>(p, s, exp2_poly)
                      : launch_t<128, false, false, false>(p, s, exp2_poly);
    }
    if (d == 64) {
        if (varlen)
            return causal ? launch_t<64, true, true, false>(p, s) : launch_t<64, false, true, false>(p, s);
        return causal ? launch_t<64, true, false, false>(p, s, exp2_poly)
                      : launch_t<64, false, false, false>(p, s, exp2_poly);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_split(const FwdParams &p, int d, bool causal, hipStream_t s) {
    if (d == 128) return causal ? launch_t<128, true, false, true>(p, s) : launch_t<128, false, false, true>(p, s);
    if (d == 64) return causal ? launch_t<64, true, false, true>(p, s) : launch_t<64, false, false, true>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
