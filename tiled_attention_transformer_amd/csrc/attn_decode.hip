// Split-KV decode for gfx950: one new query token per sequence against a KV
// cache, with a log-sum-exp merge of the key ranges.
//
// The per-range work is the attention of the FlashAttention-4 page
// (lecompute.fr, "FlashAttention-4 : limites du calcul matriciel", section
// "Entre deux multiplications il faut fabriquer les poids"); the merges use
// the same common-scale bookkeeping as the tiled softmax (section "Déplacer
// une partie des exponentielles"), applied across key ranges.  Decode rereads
// the whole context state for every generated token, so it is bound by
// memory bandwidth (lecompute.fr, "Flapping Airplanes, ThunderKittens and
// megakernels", section "Follow the request instead of one utilization
// number", and the KV-cache note in "A benchmark that could test the broader
// promise").
//
// gfx950 mapping (the split kernel streams; it is bound by HBM bandwidth):
//  * a persistent grid, one 4-wave workgroup per CU: workgroup w takes the
//    work items w, w + grid, ...; an item is (sequence, KV head, block of
//    <= 32 query heads, key range), and all query heads of a GQA group share
//    one pass over that range of K and V;
//  * the four waves split an item's keys: wave v takes 32-key tiles v, v+4,
//    v+8, ... (so together they read 128 consecutive keys at a time) and
//    streams them through a private LDS ring (2 stages of bf16 tiles, or 4
//    of fp8 tiles: the same 32 KB) with buffer loads that write straight to
//    LDS.  The loads are non-temporal: each cache byte is read once per call,
//    and streaming it past L2 and the infinity cache instead of through them
//    measured 5.5 % faster for a bf16 cache and 20 % for an fp8 one.  No wave
//    waits for another while streaming:
//    a ring shared by the workgroup needs a barrier per tile, and that
//    barrier alone held a plain load stream of this shape to ~5.35 TB/s
//    where private rings reach ~5.9 TB/s;
//  * each wave keeps its own online softmax (running max, sum, fp32
//    output) for its keys: S^T = K Q^T and O^T += V^T P^T on
//    v_mfma_f32_32x32x16_bf16, V read with ds_read_b64_tr_b16; rows are
//    unpadded and their 16-byte chunks XOR-swizzled by row so both operand
//    reads are free of bank conflicts.  An fp8 (e4m3fn) cache stays fp8 in
//    LDS and is widened to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8,
//    exact) right before the MFMAs; V then comes through ds_read_b64_tr_b8;
//  * when the split items number at least four per CU, every wave is a
//    worker of its own instead (template parameter WI): it takes whole items
//    and writes each one's partial itself, with no merge of the waves and
//    no barrier;
//  * with per-sequence key counts the split can follow the counts instead of
//    the capacity (template parameter LISTED, with WI): every workgroup
//    builds the same list of sequence offsets in LDS from the counts, the
//    32-key tiles of all groups lie end to end, and wave w of the fixed
//    1024-wave grid takes the run of tiles [w Ct, (w+1) Ct) with
//    Ct = ceil(tiles / 1024), meeting one or more groups.  Every wave reads
//    the same number of bytes whatever the mix of lengths; a group's first
//    run writes its partial to the group's own row, a run that continues a
//    group begun by an earlier wave to that wave's one continuation row, and
//    a group inside one run writes its result directly;
//  * at the end of an item the four waves merge their states through LDS
//    (log-sum-exp weights, then a fixed-order sum, so results are
//    deterministic) and the result goes out: bf16 O and LSE when the item is
//    the whole sequence, else a normalised fp32 partial with its natural-log
//    LSE for a second small kernel that merges the key ranges;
//  * the next item's query rows are loaded into spare registers at the end
//    of each wave's last tile, ahead of that wave's next tile load, so the
//    stream does not drain between items.
#include "kernels.h"
#include "tile_common.h"

namespace attn {

namespace {

constexpr int NT = kDecThreads;          // 4 waves
constexpr int NWV = NT / 64;
constexpr int NCOL = kDecCols;           // query heads per block (MFMA columns)

// LDS plan of the split kernel for one cached element type: bf16, or fp8
// (OCP e4m3fn codes).  Tiles are 32 keys either way; an fp8 tile is half the
// bytes, so the same ring holds four stages instead of two and each wave
// keeps three tiles in flight instead of one.  The stream is bound by how
// many bytes are in flight, not by the compute per tile.
template <int D, bool F8>
struct DecLay {
    static constexpr int EB = F8 ? 1 : 2;              // bytes per cached element
    static constexpr int TK = 32;                      // keys per wave tile
    static constexpr int STAGES = F8 ? 4 : 2;          // ring stages per wave
    static constexpr int NB = TK / 32;                 // 32-key MFMA blocks per tile
    static constexpr int NP = TK / 16;                 // 16-key parts per tile (own descriptors)
    static constexpr int RB = D * EB;                  // bytes per cached row
    static constexpr int CPR = RB / 16;                // 16-byte chunks per row
    static constexpr int T_BYTES = TK * RB;            // one K or V tile
    static constexpr int STAGE = 2 * T_BYTES;          // K, then V
    static constexpr int LOADS = T_BYTES / 1024;       // wave-wide loads per K (or V) tile
    static constexpr int RING = STAGES * STAGE;        // the wave's ring
    static constexpr int MERGE = NCOL * D;             // fp32 output block for the merge
    static constexpr int LSE = NWV * NCOL;             // per-wave LSEs (fp32)
    // LDS bytes: the rings, then the fp32 merge areas, then the item list of
    // a batch split by its key counts (one LDS object, so the compiler
    // keeps no alias scopes that would make it wait for every tile load
    // before the next LDS read)
    static constexpr int TOTAL = NWV * RING + 4 * (MERGE + LSE);
    static constexpr int LIST = 4 * (kDecListSeqs + 1 + NWV);
    static_assert((CPR & (CPR - 1)) == 0 && 32 % CPR == 0, "chunk swizzle needs a power of two");
    static_assert(T_BYTES % 1024 == 0, "a tile must be whole wave loads");
    static_assert(16 % (1024 / RB) == 0, "a load must stay within a 16-key part");
    static_assert((STAGES & (STAGES - 1)) == 0 && STAGES <= 4, "stage count");
};

// Chunk swizzles (physical chunk = logical chunk ^ f(row)); LDS serves 256
// bytes (64 banks) per cycle, so the 16-byte chunks one cycle reads must
// cover distinct 16-byte bank groups.
//  * bf16: K is read by rows (lane = key row, 16 bytes), so 16 consecutive
//    rows must hit distinct chunks; V is read by 4 consecutive rows at a time
//    (ds_read_b64_tr_b16), so those 4 rows must hit distinct 64-byte groups.
//  * fp8: rows are 128 (d = 128) or 64 (d = 64) bytes, so 2 or 4 rows share a
//    256-byte bank line.  K reads 16 consecutive rows per chunk; V's
//    ds_read_b64_tr_b8 has each 16-lane group read 8 rows x 16 bytes, and the
//    swizzle keeps any two groups of one read apart.  (Checked exhaustively
//    on the CPU for both head sizes.)
template <int D, bool F8>
__device__ __forceinline__ int swz_k(int row) {
    if constexpr (F8) return D == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
    else return row & (D / 8 - 1);
}
template <int D, bool F8>
__device__ __forceinline__ int swz_v(int row) {
    if constexpr (F8) return D == 128 ? ((row & 2) | ((row >> 1) & 4) | ((row >> 2) & 1)) : (row >> 2) & 3;
    else return (4 * (row & 3)) & (D / 8 - 1);
}

// Eight fp8 (e4m3fn) codes -> bf16x8, exactly (every e4m3fn value is a bf16
// value); v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two codes.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Decode split by the per-sequence key counts.  The 32-key tiles of every
// group (sequence b, KV head, query-head block) are laid end to end, the
// groups in (b, KV head, block) order, sequence b's `per` groups holding
// ceil(len_b / 32) tiles each; list[b] = the position of sequence b's first
// tile, list[B] = the tile count Wt.  Every wave w of the `workers` takes the
// run of tiles [w Ct, (w+1) Ct) (clipped to Wt), with Ct = ceil(Wt /
// workers), at least kDecListMinTiles; returns Ct.  list holds
// kDecListSeqs + 1 + NWV ints in LDS, the last NWV scratch.  Every thread of
// the workgroup takes part; the list is complete on return, and every
// workgroup computes the same one.
__device__ int decode_list_build(const DecParams &p, int *list, int workers) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nt = (int)blockDim.x;
    int *const wave_tot = list + kDecListSeqs + 1;
    typedef const __attribute__((address_space(1))) int gint;
    const int per = p.Hkv * p.ncb;                   // groups per sequence
    // the tiles of one group of each sequence (lengths clamped to
    // [0, capacity]) into list[]
    for (int b = tid; b < p.B; b += nt)
        list[b] = (min(max(((gint *)p.seqlens)[b], 0), p.Skv) + 31) / 32;
    __syncthreads();
    // sequence tiles, an exclusive scan over the workgroup: thread t owns
    // the sequences t*K .. t*K+K-1 (K = ceil(B / threads)), in order
    const int K = (p.B + nt - 1) / nt;
    int mine = 0;
    for (int i = 0; i < K; ++i) {
        const int b = tid * K + i;
        if (b < p.B) mine += list[b] * per;
    }
    int inc = mine;                                   // inclusive scan in the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int up = __shfl_up(inc, o, 64);
        if (lane >= o) inc += up;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    int base = inc - mine;
    for (int w = 0; w < wave; ++w) base += wave_tot[w];
    // each thread replaces its own tile counts by its sequences' offsets
    for (int i = 0; i < K; ++i) {
        const int b = tid * K + i;
        if (b < p.B) {
            const int n = list[b] * per;
            list[b] = base;
            base += n;
        }
    }
    if (tid == nt - 1) list[p.B] = base;
    __syncthreads();
    const int Wt = list[p.B];
    return max(kDecListMinTiles, (Wt + workers - 1) / workers);
}

// WI (wave items): every wave is a worker of its own that takes whole items
// (each one key chunk of one group) and writes their partials itself: no
// merge of the waves, no barrier.  Used for split counts that give every
// wave of the grid work; otherwise (WI = false) the four waves of a
// workgroup share each item's keys and merge their states through LDS.
// LISTED (with WI): the split by the key counts, each wave's items being the
// groups its run of tiles meets (decode_list_build).
template <int D, bool F8, bool WI, bool LISTED>
__global__ __launch_bounds__(NT)
void attn_decode_split_kernel(DecParams p) {
    using L = DecLay<D, F8>;
    constexpr int TK = L::TK;
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::TOTAL + (LISTED ? L::LIST : 0)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int col = lane & 31;
    const int64_t hd_k = (int64_t)p.Hkv * D;     // elements between consecutive keys
    unsigned char *ring = lds + wave * L::RING;
    float *merge_o = reinterpret_cast<float *>(lds + NWV * L::RING);
    float *merge_l = merge_o + L::MERGE;
    typedef const __attribute__((address_space(4))) int cint;
    // the sequence's key count (per sequence when given), read through the
    // constant address space: a scalar load, outside the vector-load
    // counter the tile waits rely on
    auto seq_len = [&](int b) {
        return p.seqlens ? min(max(((cint *)p.seqlens)[b], 0), p.Skv) : p.Skv;
    };

    // Work items are (group, key range), range fastest, with group =
    // (sequence, KV head, block of query heads); worker w takes items
    // w, w + workers, ...  A worker is a workgroup, or with WI a wave.
    const int G = WI ? (int)gridDim.x * NWV : (int)gridDim.x;
    const int worker = WI ? (int)blockIdx.x * NWV + wave : (int)blockIdx.x;
    // Split by the key counts: this wave's run of tiles [s_lo, s_hi) of the
    // groups laid end to end (see decode_list_build), whose items are the
    // groups it meets, from g_first on (empty sequences' groups among them
    // are items without keys)
    int *const list = reinterpret_cast<int *>(lds + L::TOTAL);
    const int per = p.Hkv * p.ncb;                   // groups per sequence
    int my_items = 0, Ct = 1, s_lo = 0, s_hi = 0, g_first = 0;
    // (lo, n) of sequence b: its first tile and the tiles of each group
    auto seq_tiles = [&](int b, int &lo) {
        lo = __builtin_amdgcn_readfirstlane(list[b]);
        return (__builtin_amdgcn_readfirstlane(list[b + 1]) - lo) / per;
    };
    if constexpr (LISTED) {
        // (the same in every lane: say so, so the item arithmetic stays scalar)
        Ct = __builtin_amdgcn_readfirstlane(decode_list_build(p, list, G));
        if (blockIdx.x == 0) {
            // the run length and the offsets, for the merge
            if (tid == 0) p.ws_hdr[0] = Ct;
            for (int b = tid; b <= p.B; b += NT) p.ws_hdr[4 + b] = list[b];
        }
        const int Wt = __builtin_amdgcn_readfirstlane(list[p.B]);
        const int64_t lo = (int64_t)worker * Ct;
        if (lo < Wt) {
            s_lo = (int)lo;
            s_hi = (int)min(lo + Ct, (int64_t)Wt);
            // the group holding tile t: sequence = the last b with
            // list[b] <= t (it has tiles, as t < list[b + 1])
            auto group_at = [&](int t) {
                int a = 0, z = p.B - 1;
                while (a < z) {
                    const int mid = (a + z + 1) >> 1;
                    if (__builtin_amdgcn_readfirstlane(list[mid]) <= t) a = mid;
                    else z = mid - 1;
                }
                int l0;
                const int n = seq_tiles(a, l0);
                return a * per + (t - l0) / n;
            };
            g_first = group_at(s_lo);
            my_items = group_at(s_hi - 1) - g_first + 1;
        }
    } else {
        const int nitems = p.B * p.Hkv * p.ncb * p.nsplit;
        my_items = (worker < nitems) ? (nitems - worker + G - 1) / G : 0;
    }

    struct Item {
        int b, hk, h0, ncols, sp, nsp, k_lo, nkeys, ntiles;
    };
    auto get_item = [&](int it) {
        Item r;
        int id, cb;
        if constexpr (LISTED) {
            // group g_first + it (g_first = 0 for a wave without items):
            // its tiles [sg, sg + n) meet this wave's run in [a, e); sp = 0
            // for the group's first run, else the run continues a group an
            // earlier wave began; nsp = the runs of the group
            id = min(g_first + it, p.B * per - 1);
            r.b = id / per;
            const int i = id - r.b * per;
            r.hk = i / p.ncb;
            cb = i - r.hk * p.ncb;
            int l0;
            const int n = seq_tiles(r.b, l0);
            const int sg = l0 + i * n;
            r.sp = n > 0 ? worker - sg / Ct : 0;
            r.nsp = n > 0 ? (sg + n - 1) / Ct - sg / Ct + 1 : 0;
            const int a = max(s_lo, sg), e = min(s_hi, sg + n);
            r.k_lo = n > 0 ? (a - sg) * 32 : 0;
            r.nkeys = n > 0 ? max(0, min(seq_len(r.b), (e - sg) * 32) - r.k_lo) : 0;
        } else {
            const int item = worker + G * it;
            r.sp = item % p.nsplit;
            r.nsp = p.nsplit;
            id = item / p.nsplit;
            cb = id % p.ncb;
            id /= p.ncb;
            r.hk = id % p.Hkv;
            r.b = id / p.Hkv;
            r.k_lo = r.sp * p.chunk;
            r.nkeys = max(0, min(seq_len(r.b), r.k_lo + p.chunk) - r.k_lo);
        }
        r.ntiles = (r.nkeys + TK - 1) / TK;
        r.ncols = min(NCOL, p.group - NCOL * cb);
        r.h0 = r.hk * p.group + NCOL * cb;
        return r;
    };
    // this wave's tiles of an item: w, w + NWV, ... (with WI: all of them)
    auto wave_tiles = [&](const Item &it) {
        if constexpr (WI) return it.ntiles;
        return wave < it.ntiles ? (it.ntiles - wave + NWV - 1) / NWV : 0;
    };
    // the position of this wave's tile t within its item, in tiles
    auto tile_pos = [&](int t) { return WI ? t : wave + NWV * t; };

    // Load plan: load m of a tensor (m < LOADS) fills bytes 1024m ..
    // 1024m+1023 of the tile; lane L's 16-byte slot is (row, physical
    // chunk).  A tile is read as parts of 16 keys, each through its own
    // buffer descriptor (in a paged cache the parts may sit in different
    // pages); a load never straddles two parts, and its offset is relative
    // to its part.
    uint32_t goff[2 * L::LOADS];
#pragma unroll
    for (int pp = 0; pp < 2 * L::LOADS; ++pp) {
        const bool isv = pp >= L::LOADS;
        const int m = isv ? pp - L::LOADS : pp;
        const int slot = 64 * m + lane;
        const int row = slot / L::CPR;
        const int lc = (slot % L::CPR) ^ (isv ? swz_v<D, F8>(row) : swz_k<D, F8>(row));
        goff[pp] = (uint32_t)((row % 16) * hd_k * L::EB + 16 * lc);
    }

    // This wave's load stream: its tiles of every item, in order.  `li` is
    // the item of the next tile, `lt` the wave's tile index within it.
    int li = 0, lt = 0, lstage = 0;
    int lcnt = 0;                                // tiles issued so far
    Item litem = get_item(0);
    int lcount = my_items > 0 ? wave_tiles(litem) : 0;
    // skip items where this wave has no tile
    auto lskip = [&]() {
        while (li < my_items && lt >= lcount) {
            lt = 0;
            if (++li < my_items) {
                litem = get_item(li);
                lcount = wave_tiles(litem);
            }
        }
    };
    lskip();
    const unsigned char *kbase = static_cast<const unsigned char *>(p.k);
    const unsigned char *vbase = static_cast<const unsigned char *>(p.v);
    auto issue_next = [&]() {
        if (li >= my_items) return;
        const int key0 = litem.k_lo + TK * tile_pos(lt);
        const int rows = min(TK, litem.k_lo + litem.nkeys - key0);
        __amdgpu_buffer_rsrc_t kr[L::NP], vr[L::NP];
#pragma unroll
        for (int h = 0; h < L::NP; ++h) {
            const int rh = min(max(rows - 16 * h, 0), 16);   // valid rows of the part
            const int kh = key0 + 16 * h;
            int64_t row0 = 0;
            bool ok = rh > 0;
            if (p.block_table != nullptr) {
                // the page holding these 16 keys (16 divides the page size);
                // a page id outside the pool reads as zeros, no memory access
                typedef const __attribute__((address_space(4))) int cint;
                const int pid = ok ? ((cint *)p.block_table)[(int64_t)litem.b * p.max_pages + kh / p.page_size] : 0;
                ok = ok && pid >= 0 && pid < p.num_pages;
                row0 = ((int64_t)(ok ? pid : 0) * p.page_size + kh % p.page_size) * hd_k;
            } else {
                row0 = ((int64_t)litem.b * p.Skv + kh) * hd_k;
            }
            row0 = (row0 + (int64_t)litem.hk * D) * L::EB;   // bytes
            // the descriptors end at the last valid key: rows past it read zeros
            const int nbytes = ok ? (int)(((int64_t)(rh - 1) * hd_k + D) * L::EB) : 0;
            kr[h] = buffer_rsrc(ok ? kbase + row0 : kbase, nbytes);
            vr[h] = buffer_rsrc(ok ? vbase + row0 : vbase, nbytes);
        }
        unsigned char *dst = ring + lstage * L::STAGE;
#pragma unroll
        for (int pp = 0; pp < 2 * L::LOADS; ++pp) {
            const int m = pp % L::LOADS;
            const int h = (m * (1024 / L::RB)) / 16;          // rows of load m: m * 1024/RB ..
            // the cache is read once per call: non-temporal, so it streams
            // past L2 and the infinity cache instead of thrashing them
            buffer_lds_dma16<kNonTemporal>(pp >= L::LOADS ? vr[h] : kr[h], goff[pp],
                                           dst + (pp >= L::LOADS ? L::T_BYTES : 0) + 1024 * m);
        }
        lstage = (lstage + 1) & (L::STAGES - 1);
        ++lt;
        ++lcnt;
        lskip();
    };

    // Query rows of an item (heads h0 .. h0+ncols-1, contiguous in memory),
    // as the B operand of S^T = K Q^T: column `col` is query head h0 + col.
    // The descriptor covers the item's heads only, so other columns are 0.
    // bf16 caches: MFMA t contracts d = 16t .. 16t+15, lane half g holding
    // 16t + 8g ..  fp8 caches: a lane reads 16 fp8 codes (two MFMAs' worth)
    // of a key row at once, so MFMA u = 2t + j contracts d = 32t + 16g + 8j
    // .. +7 in lane half g; the query takes the same order.
    auto load_q = [&](const Item &it, bf16x8 (&q)[D / 16]) {
        const __amdgpu_buffer_rsrc_t qr =
            buffer_rsrc(p.q + ((int64_t)it.b * p.Hq + it.h0) * D, it.ncols * D * 2);
        const uint32_t o0 = (uint32_t)((col * D + (F8 ? 16 : 8) * g) * 2);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            const uint32_t ot = F8 ? 64 * (t >> 1) + 16 * (t & 1) : 32 * t;
            q[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, o0 + ot, 0, 0));
        }
    };

    // Per-lane operand offsets (bytes, within a stage).
    //  K (bf16): row col, logical chunk 2t + g.  K (fp8): row col, logical
    //  chunk 2t + g for MFMAs 2t and 2t+1 (low and high 8 bytes).
    //  V (bf16): the transposing read of keys 4g + e (+16kk, +8) and columns
    //  32*db + 16*dh + 4*s.  V (fp8): 16-lane group G reads keys
    //  8(b/4) + 4g + b%4 (b = 0..7, two lanes per key, 8 bytes each) of the
    //  16 columns 32*db + 16*(G%2) ..; lane i of the group receives column i,
    //  in the key order of the P^T operand.
    constexpr int NKO = F8 ? D / 32 : D / 16;
    int kof[NKO];
#pragma unroll
    for (int t = 0; t < NKO; ++t) kof[t] = col * L::RB + 16 * ((2 * t + g) ^ swz_k<D, F8>(col));
    int vof[D / 32];
    if constexpr (F8) {
        const int grp = lane >> 4, bi = (lane & 15) >> 1, hh = lane & 1;
        const int vkey = 8 * (bi >> 2) + 4 * (grp >> 1) + (bi & 3);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            vof[db] = L::T_BYTES + vkey * L::RB + 16 * ((2 * db + (grp & 1)) ^ swz_v<D, F8>(vkey)) + 8 * hh;
    } else {
        const int tr_e = (lane & 15) >> 2, tr_s = lane & 3, tr_dh = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int vlc = 4 * db + 2 * tr_dh + (tr_s >> 1);
            vof[db] = L::T_BYTES + (4 * g + tr_e) * L::RB + 16 * (vlc ^ swz_v<D, F8>(tr_e)) + 8 * (tr_s & 1);
        }
    }

    f32x16 oacc[D / 32];
    float m = -__builtin_inff();
    float lsum = 0.f;
    const float c = p.c;
    bf16x8 qf[D / 16], qn[D / 16];

    // The first item's query rows, then the first tiles of the stream (one
    // per stage): the rows are older than every tile, so the first tile wait
    // covers them.
    if (my_items > 0) load_q(get_item(0), qf);
#pragma unroll
    for (int i = 0; i < L::STAGES; ++i) issue_next();

    int cstage = 0;                              // stage of the tile being computed
    int ccnt = 0;                                // tiles computed so far
    bool stores = false;                         // output stores since the last full wait
    for (int ci = 0; ci < my_items; ++ci) {
        const Item it = get_item(ci);
        const int nmine = wave_tiles(it);
        if (ci > 0) {
#pragma unroll
            for (int t = 0; t < D / 16; ++t) qf[t] = qn[t];
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
        m = -__builtin_inff();
        lsum = 0.f;

        for (int tw = 0; tw < nmine; ++tw) {
            // this tile complete.  Loads complete in order, so everything but
            // the loads of the tiles issued after this one must be done;
            // after output stores (which share the counter), wait for all.
            const int ahead = stores ? 0 : min(lcnt - ccnt - 1, L::STAGES - 1);
            if (ahead >= 3) wait_vmcnt<3 * 2 * L::LOADS>();
            else if (ahead == 2) wait_vmcnt<2 * 2 * L::LOADS>();
            else if (ahead == 1) wait_vmcnt<2 * L::LOADS>();
            else wait_vmcnt<0>();
            stores = false;
            const unsigned char *st = ring + cstage * L::STAGE;

            // S^T for the tile's keys, 32 at a time
            f32x16 s[L::NB];
#pragma unroll
            for (int kb = 0; kb < L::NB; ++kb) {
                s[kb] = f32x16{};
                const unsigned char *sk = st + kb * 32 * L::RB;
                if constexpr (F8) {
#pragma unroll
                    for (int t = 0; t < D / 32; ++t) {
                        const u32x4 raw = *reinterpret_cast<const u32x4 *>(sk + kof[t]);
                        s[kb] = mfma32x32x16(fp8x8_to_bf16(raw[0], raw[1]), qf[2 * t], s[kb]);
                        s[kb] = mfma32x32x16(fp8x8_to_bf16(raw[2], raw[3]), qf[2 * t + 1], s[kb]);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < D / 16; ++t)
                        s[kb] = mfma32x32x16(ld_lds_bf16x8((const __bf16 *)(sk + kof[t])), qf[t], s[kb]);
                }
            }
            const int kt = TK * tile_pos(tw);       // first key of the tile, within the item
            if (kt + TK > it.nkeys) {
#pragma unroll
                for (int kb = 0; kb < L::NB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kt + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3) >= it.nkeys) s[kb][r] = -__builtin_inff();
            }
            // online softmax, lazy rescale (reference max moves by > kRescaleSlack)
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < L::NB; ++kb)
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
            for (int kb = 0; kb < L::NB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
                    rs += s[kb][r];
                }
            lsum += rs;
            // O^T += V^T P^T, 16 keys at a time, all D columns
#pragma unroll
            for (int kk = 0; kk < TK / 16; ++kk) {
                const bf16x8 pk = pack_p8(s[kk >> 1], 8 * (kk & 1));
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    bf16x8 va;
                    if constexpr (F8) {
                        const u32x2 raw = lds_read_tr8(st + vof[db] + 16 * kk * L::RB);
                        va = fp8x8_to_bf16(raw[0], raw[1]);
                    } else {
                        const s16x4 lo = lds_read_tr((const __bf16 *)(st + vof[db] + 16 * kk * L::RB));
                        const s16x4 hi = lds_read_tr((const __bf16 *)(st + vof[db] + (16 * kk + 8) * L::RB));
                        va = concat_tr(lo, hi);
                    }
                    oacc[db] = mfma32x32x16(va, pk, oacc[db]);
                }
            }
            // the next item's query rows, ahead of this wave's next tile load
            if (tw == nmine - 1 && ci + 1 < my_items) load_q(get_item(ci + 1), qn);
            // this stage is consumed: refill it with the tile after next
            issue_next();
            cstage = (cstage + 1) & (L::STAGES - 1);
            ++ccnt;
        }
        if (nmine == 0 && ci + 1 < my_items) load_q(get_item(ci + 1), qn);

        if constexpr (WI) {
            // this wave's own item: its normalised partial and natural-log
            // LSE go straight to the workspace (an empty chunk: O = 0,
            // LSE = -inf, weight 0 in the merge)
            const float lt2 = half_swap_sum(lsum);
            // 1 / l, times the value scale of an fp8 cache
            const float inv = lt2 > 0.f ? (F8 ? p.v_scale : 1.f) / lt2 : 0.f;
            stores = true;
            if (LISTED && it.nkeys == 0) {
                // a group of an empty sequence: the merge writes its result
            } else if (LISTED && it.nsp == 1) {
                // the sequence's only chunk (split by the key counts): the
                // result itself, which the merge then leaves alone
                if (col < it.ncols) {
                    const int h = it.h0 + col;
                    __bf16 *op = p.o + ((int64_t)it.b * p.Hq + h) * D + 4 * g;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
#pragma unroll
                        for (int rq = 0; rq < 4; ++rq)
                            *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * rq) =
                                to_bf16x4(oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv,
                                          oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv);
                    if (g == 0 && p.lse != nullptr)
                        p.lse[(int64_t)it.b * p.Hq + h] =
                            lt2 > 0.f ? (m + fast_log2(lt2)) * kLn2 : -__builtin_inff();
                }
            } else if (col < it.ncols) {
                const int h = it.h0 + col;
                // the partial's row: split by the capacity, (sp, b, h); split
                // by the key counts, (b, h) for a group's first run, else the
                // wave's own continuation row
                const int64_t row = !LISTED ? ((int64_t)it.sp * p.B + it.b) * p.Hq + h
                                    : it.sp == 0 ? (int64_t)it.b * p.Hq + h
                                                 : (int64_t)p.B * p.Hq + (int64_t)worker * p.ncm + col;
                float *op = p.ws_o + row * D + 4 * g;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const f32x4 v4 = {oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv,
                                          oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv};
                        *reinterpret_cast<f32x4 *>(op + 32 * db + 8 * rq) = v4;
                    }
                if (g == 0) p.ws_lse[row] = lt2 > 0.f ? (m + fast_log2(lt2)) * kLn2 : -__builtin_inff();
            }
            continue;
        }

        // Merge of the four waves' states: per query column, the waves'
        // log-sum-exp values give each wave's weight; the weighted outputs
        // are then summed in a fixed wave order through LDS.
        const float lt2 = half_swap_sum(lsum);
        const float lse2 = lt2 > 0.f ? m + fast_log2(lt2) : -__builtin_inff();   // log2 units
        if (g == 0) merge_l[wave * NCOL + col] = lse2;
        wait_lgkmcnt0();
        lds_barrier();
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < NWV; ++w) M = fmaxf(M, merge_l[w * NCOL + col]);
        float wsum = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
            const float lw = merge_l[w * NCOL + col];
            wsum += lw == -__builtin_inff() ? 0.f : fast_exp2(lw - M);
        }
        // weight of this wave's normalised output, times 1 / l for the
        // normalisation: exp2(lse2 - M) / wsum / l = exp2(m - M) / wsum
        // (times the value scale of an fp8 cache)
        float f = lt2 > 0.f ? fast_exp2(m - M) / wsum : 0.f;
        if constexpr (F8) f *= p.v_scale;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= f;
        // merge_o holds O^T in the accumulator layout: element (db, r) of
        // lane L at index ((db * 16 + r) * 64 + L), so reads and writes are
        // contiguous per register
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
            if (wave == w) {
                if (w > 0) {
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[db][r] += merge_o[(db * 16 + r) * 64 + lane];
                }
                if (w < NWV - 1) {
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) merge_o[(db * 16 + r) * 64 + lane] = oacc[db][r];
                }
            }
            if (w < NWV - 1) {
                wait_lgkmcnt0();
                lds_barrier();
            }
        }
        if (wave == NWV - 1) stores = true;
        if (wave == NWV - 1 && col < it.ncols) {
            const int h = it.h0 + col;
            const float lse_nat = M == -__builtin_inff() ? -__builtin_inff() : (M + fast_log2(wsum)) * kLn2;
            if (p.nsplit == 1) {
                __bf16 *op = p.o + ((int64_t)it.b * p.Hq + h) * D + 4 * g;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq)
                        *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * rq) =
                            to_bf16x4(oacc[db][4 * rq], oacc[db][4 * rq + 1], oacc[db][4 * rq + 2],
                                      oacc[db][4 * rq + 3]);
                if (g == 0 && p.lse != nullptr) p.lse[(int64_t)it.b * p.Hq + h] = lse_nat;
            } else {
                float *op = p.ws_o + (((int64_t)it.sp * p.B + it.b) * p.Hq + h) * D + 4 * g;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const f32x4 v4 = {oacc[db][4 * rq], oacc[db][4 * rq + 1], oacc[db][4 * rq + 2],
                                          oacc[db][4 * rq + 3]};
                        *reinterpret_cast<f32x4 *>(op + 32 * db + 8 * rq) = v4;
                    }
                if (g == 0) p.ws_lse[((int64_t)it.sp * p.B + it.b) * p.Hq + h] = lse_nat;
            }
        }
    }
    wait_vmcnt<0>();                 // no load may outlive the workgroup
}

// Merge of the key-range partials: one 4-wave workgroup per (sequence,
// query head); LSE = M + log(sum_s exp(lse_s - M)), O = sum_s exp(lse_s - LSE) O_s.
// The partials' LSE values are spread over the threads (read once, kept in
// registers for M and the sum); the O rows over the waves, each wave taking
// partials w, w+4, ... with eight loads in flight; the waves' sums are then
// combined in a fixed order, so the result is deterministic.  A row may have
// many partials (a long sequence split into many short runs): the loads, not
// the arithmetic, set the time.
constexpr int CW = 4;                        // waves of the merge kernel
constexpr int CU_ = 8;                       // O loads in flight per wave

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D, bool LISTED>
// (at most 64 VGPRs: eight waves per SIMD, every CU holding eight rows at once)
__global__ __launch_bounds__(64 * CW, 8) void attn_decode_combine_kernel(DecParams p) {
    constexpr int PER = D / 64;                     // output elements per lane
    __shared__ float red[CW];
    __shared__ float part[CW - 1][D];
    const int bh = blockIdx.x;                      // b * Hq + h
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t stride = (int64_t)p.B * p.Hq;
    // the partials of this row: one per chunk (split by the capacity), or
    // (split by the key counts) one per run of the head's group -- the
    // first in row bh, the others in the continuation rows of the waves
    // w0 + 1, w0 + 2, ..; a group of one run has its result written already
    int ns = p.nsplit, w0 = 0, ccol = 0;
    if constexpr (LISTED) {
        typedef const __attribute__((address_space(4))) int cint;
        const cint *hdr = (const cint *)p.ws_hdr;
        const int b = bh / p.Hq, h = bh - b * p.Hq;
        const int hk = h / p.group, hc = h - hk * p.group;
        const int i = hk * p.ncb + hc / NCOL;          // the head's group in its sequence
        ccol = hc % NCOL;
        const int per = p.Hkv * p.ncb, Ct = hdr[0], l0 = hdr[4 + b];
        const int n = (hdr[5 + b] - l0) / per;          // tiles of the group
        const int sg = l0 + i * n;
        w0 = sg / Ct;
        ns = n > 0 ? (sg + n - 1) / Ct - w0 + 1 : 0;
        if (ns == 1) return;
    }
    auto row = [&](int s) -> int64_t {
        if constexpr (!LISTED) return (int64_t)s * stride + bh;
        return s == 0 ? bh : stride + (int64_t)(w0 + s) * p.ncm + ccol;
    };

    // M = max_s lse_s; thread t holds lse_t (and loops past 64 * CW partials)
    const float lse_t = t < ns ? p.ws_lse[row(t)] : -__builtin_inff();
    float mx = lse_t;
    for (int s = t + 64 * CW; s < ns; s += 64 * CW) mx = fmaxf(mx, p.ws_lse[row(s)]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < CW; ++w) M = fmaxf(M, red[w]);
    const float Mu = M == -__builtin_inff() ? 0.f : M;
    __syncthreads();
    // tot = sum_s exp(lse_s - M)
    float tt = t < ns ? fast_exp2((lse_t - Mu) * kLog2e) : 0.f;
    for (int s = t + 64 * CW; s < ns; s += 64 * CW) tt += fast_exp2((p.ws_lse[row(s)] - Mu) * kLog2e);
    tt = wave_sum(tt);
    if (lane == 0) red[wave] = tt;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < CW; ++w) tot += red[w];
    const float lse = tot > 0.f ? Mu + fast_log2(tot) * kLn2 : -__builtin_inff();

    // O: wave w sums partials w, w+CW, ..., CU_ of them per round; lane L
    // holds elements PER*L ..
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    if (tot > 0.f) {
        const float *o_p = p.ws_o + PER * lane;
#pragma unroll 1
        for (int s = wave; s < ns; s += CU_ * CW) {
            float wu[CU_], vu[CU_][PER];
#pragma unroll
            for (int u = 0; u < CU_; ++u) {
                const int su = s + u * CW;
                wu[u] = -__builtin_inff();
#pragma unroll
                for (int e = 0; e < PER; ++e) vu[u][e] = 0.f;
                if (su < ns) {
                    const int64_t ru = row(su);
                    wu[u] = p.ws_lse[ru];
#pragma unroll
                    for (int e = 0; e < PER; ++e) vu[u][e] = o_p[ru * D + e];
                }
            }
#pragma unroll
            for (int u = 0; u < CU_; ++u) {
                const float w = wu[u] == -__builtin_inff() ? 0.f : fast_exp2((wu[u] - lse) * kLog2e);
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] += w * vu[u][e];
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int e = 0; e < PER; ++e) part[wave - 1][PER * lane + e] = acc[e];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 1; w < CW; ++w)
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += part[w - 1][PER * lane + e];
        __bf16 *op = p.o + (int64_t)bh * D + PER * lane;
#pragma unroll
        for (int e = 0; e < PER; ++e) op[e] = (__bf16)acc[e];
        if (p.lse != nullptr && lane == 0) p.lse[bh] = lse;
    }
}

template <int D, bool F8>
hipError_t launch_t(DecParams p, hipStream_t s) {
    static_assert(NWV == 4, "a workgroup is four waves");
    int cus = 0;
    hipError_t e = current_cu_count(&cus);
    if (e != hipSuccess) return e;
    // The split count is the caller's (or the host-side choice): one key
    // range per item means whole sequences per workgroup, whose four waves
    // split the keys and merge them, and the result goes out directly;
    // otherwise the key ranges of a sequence spread over the workgroups and
    // a second kernel merges their partials.
    if (p.listed) {
        // split by the key counts: a fixed grid (the workspace holds a row
        // per wave of it), every wave a worker with its own run; the merge
        // follows
        hipLaunchKernelGGL((attn_decode_split_kernel<D, F8, true, true>), dim3(kDecListWGs), dim3(NT), 0,
                           s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((attn_decode_combine_kernel<D, true>), dim3((unsigned)(p.B * p.Hq)),
                           dim3(64 * CW), 0, s, p);
        return hipGetLastError();
    }
    const int64_t groups = (int64_t)p.B * p.Hkv * p.ncb;
    const int64_t items = groups * p.nsplit;
    if (items > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int blocks = (int)(items < cus ? items : cus);
    if (blocks <= 0) return hipSuccess;
    // split items for every wave of the grid: waves take whole items
    if (p.nsplit > 1 && items >= (int64_t)NWV * cus)
        hipLaunchKernelGGL((attn_decode_split_kernel<D, F8, true, false>), dim3((unsigned)blocks), dim3(NT), 0,
                           s, p);
    else
        hipLaunchKernelGGL((attn_decode_split_kernel<D, F8, false, false>), dim3((unsigned)blocks), dim3(NT),
                           0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    hipLaunchKernelGGL((attn_decode_combine_kernel<D, false>), dim3((unsigned)(p.B * p.Hq)), dim3(64 * CW), 0,
                       s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecParams &p, int d, bool fp8, hipStream_t s) {
    if (fp8) {
        if (d == 128) return launch_t<128, true>(p, s);
        if (d == 64) return launch_t<64, true>(p, s);
    } else {
        if (d == 128) return launch_t<128, false>(p, s);
        if (d == 64) return launch_t<64, false>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
