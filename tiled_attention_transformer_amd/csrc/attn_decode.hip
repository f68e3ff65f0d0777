// Split-KV decode for gfx950: one new query token per sequence against a KV
// cache, followed by a log-sum-exp merge of the key chunks.
//
// The per-chunk work is the attention of the FlashAttention-4 page
// (lecompute.fr, "FlashAttention-4 : limites du calcul matriciel", section
// "Entre deux multiplications il faut fabriquer les poids"); the merge uses
// the same common-scale bookkeeping as the tiled softmax (section "Déplacer
// une partie des exponentielles"), applied across chunks.  Decode rereads the
// whole context state for every generated token, so it is bound by memory
// bandwidth (lecompute.fr, "Flapping Airplanes, ThunderKittens and
// megakernels", section "Follow the request instead of one utilization
// number", and the KV-cache note in "A benchmark that could test the broader
// promise").
//
// gfx950 mapping (the split kernel streams; it is bound by HBM bandwidth):
//  * a persistent grid, one 4-wave workgroup per CU: workgroup w takes the
//    work items (sequence, KV head, block of <= 32 query heads, key chunk)
//    w, w + grid, ... and streams their 64-key K/V tiles back to back, so the
//    load pipeline never drains between items;
//  * tiles move HBM -> LDS with buffer loads that write straight to LDS into
//    a 4-stage ring (3 tiles, 96 KB, in flight per CU); rows are unpadded
//    and their 16-byte chunks are XOR-swizzled by row so that both operand
//    reads below are free of bank conflicts;
//  * every wave computes the scores of all 64 keys against all query heads
//    of the block (S^T = K Q^T, v_mfma_f32_32x32x16_bf16; cheap next to the
//    memory time) and keeps identical softmax state; wave w then owns output
//    columns 32w .. 32w+31 of O^T += V^T P^T (V read with ds_read_b64_tr_b16),
//    so no cross-wave merge is needed;
//  * the next item's query rows load into LDS the same way while the
//    current item streams (a load into registers would make every wait on
//    the in-order load counter also wait for all older tile loads);
//  * each item's result is written normalised, in fp32, with its natural-log
//    LSE, and a second small kernel merges the chunks; with a single chunk
//    the result goes out directly as bf16.
#include "kernels.h"
#include "tile_common.h"

namespace attn {

namespace {

constexpr int NT = kDecThreads;          // 4 waves
constexpr int NWV = NT / 64;
constexpr int NCOL = kDecCols;           // query heads per block (MFMA columns)

template <int D, int BC, int NSD>
struct DecLay {
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int T_ELEMS = BC * D;             // one K or V tile
    static constexpr int STAGE = 2 * T_ELEMS;          // K, then V
    static constexpr int LOADS = 2 * BC * CPR / 64;    // wave-wide loads per tile
    static constexpr int PER_WAVE = LOADS / NWV;
    static constexpr int Q_ELEMS = NCOL * D;           // query rows of one item
    static constexpr int Q_LOADS = Q_ELEMS / 512;      // wave-wide loads for them
    static constexpr int Q_PER_WAVE = (Q_LOADS + NWV - 1) / NWV;
    static constexpr int Q_BASE = NSD * STAGE;
    static constexpr int TOTAL = Q_BASE + Q_ELEMS;
    static_assert(LOADS % (2 * NWV) == 0, "K and V loads must split evenly over the waves");
    static_assert((CPR & (CPR - 1)) == 0 && 32 % CPR == 0, "chunk swizzle needs a power of two");
};

// Chunk swizzles (physical chunk = logical chunk ^ f(row)).  K is read by
// rows (lane = key row, 16 bytes), so 16 consecutive rows must hit distinct
// chunks; V is read by 4 consecutive rows at a time (transposing reads), so
// those 4 rows must hit distinct 64-byte column groups.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return row & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int row) { return (4 * (row & 3)) & (D / 8 - 1); }

// BC keys per tile, NSD ring stages
template <int D, int BC, int NSD>
__global__ __launch_bounds__(NT)
void attn_decode_split_kernel(DecParams p) {
    using L = DecLay<D, BC, NSD>;
    __shared__ __attribute__((aligned(16))) __bf16 lds[L::TOTAL];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int col = lane & 31;
    const int64_t hd_k = (int64_t)p.Hkv * D;

    // Work items are (group, chunk) with group = (sequence, KV head, block of
    // query heads).  Without own_groups, workgroup w takes items w, w + grid,
    // ... (chunks of one group spread over workgroups; a second kernel merges
    // them).  With own_groups, it takes whole groups w, w + grid, ..., their
    // chunks in order, and merges the chunks itself.
    const int G = gridDim.x;
    const int ngroups = p.B * p.Hkv * p.ncb;
    const int my_items = p.own_groups
                             ? (ngroups - (int)blockIdx.x + G - 1) / G * p.nsplit
                             : (ngroups * p.nsplit - (int)blockIdx.x + G - 1) / G;
    const int ntot = my_items * p.nti;           // tiles this workgroup streams

    struct Item {
        int b, hk, h0, ncols, sp, k_lo, nkeys;
    };
    // work item `it` of this workgroup (it < my_items)
    auto get_item = [&](int it) {
        Item r;
        int id;                                  // group index
        if (p.own_groups) {
            r.sp = it % p.nsplit;
            id = (int)blockIdx.x + G * (it / p.nsplit);
        } else {
            const int item = (int)blockIdx.x + G * it;   // (group, chunk), chunk fastest
            r.sp = item % p.nsplit;
            id = item / p.nsplit;
        }
        const int cb = id % p.ncb;
        id /= p.ncb;
        r.hk = id % p.Hkv;
        r.b = id / p.Hkv;
        r.k_lo = r.sp * p.chunk;
        // the sequence's cache length (per sequence when given; tiles past it
        // get empty load ranges, so they read no memory, and are masked)
        const int len = p.seqlens ? min(max(p.seqlens[r.b], 0), p.Skv) : p.Skv;
        r.nkeys = max(0, min(len, r.k_lo + p.chunk) - r.k_lo);
        r.ncols = min(NCOL, p.group - NCOL * cb);
        r.h0 = r.hk * p.group + NCOL * cb;
        return r;
    };

    // Load plan: wave w issues loads w, w+4, ... of a tile (K loads first);
    // lane L of load m of a tensor fills slot 64m + L = (row, physical chunk).
    uint32_t goff[L::PER_WAVE];
    int ldo[L::PER_WAVE];
#pragma unroll
    for (int pp = 0; pp < L::PER_WAVE; ++pp) {
        const int n = wave + NWV * pp;
        const bool isv = pp >= L::PER_WAVE / 2;
        const int m = isv ? n - L::LOADS / 2 : n;
        const int slot = 64 * m + lane;
        const int row = slot / L::CPR;
        const int lc = (slot % L::CPR) ^ (isv ? swz_v<D>(row) : swz_k<D>(row));
        goff[pp] = (uint32_t)(row * hd_k + 8 * lc) * 2u;
        ldo[pp] = (isv ? L::T_ELEMS : 0) + 512 * m;
    }

    // Load stream: tile `lt` of item `li`; `lbase` is that item's first key row.
    int li = 0, lt = 0, lstage = 0;
    Item litem = get_item(0);
    auto issue_next = [&]() {
        int rows = 0;
        int64_t row0 = 0;
        if (li < my_items) {
            rows = min(BC, litem.nkeys - BC * lt);
            row0 = ((int64_t)litem.b * p.Skv + litem.k_lo + BC * lt) * hd_k + (int64_t)litem.hk * D;
        }
        const int nbytes = rows > 0 ? (int)(((int64_t)(rows - 1) * hd_k + D) * 2) : 0;
        const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.k + (rows > 0 ? row0 : 0), nbytes);
        const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(p.v + (rows > 0 ? row0 : 0), nbytes);
        __bf16 *dst = lds + lstage * L::STAGE;
#pragma unroll
        for (int pp = 0; pp < L::PER_WAVE; ++pp)
            buffer_lds_dma16(pp >= L::PER_WAVE / 2 ? vr : kr, goff[pp], dst + ldo[pp]);
        lstage = lstage == NSD - 1 ? 0 : lstage + 1;
        if (++lt == p.nti) {
            lt = 0;
            if (++li < my_items) litem = get_item(li);
        }
    };

    // Query rows of an item (heads h0 .. h0+ncols-1, contiguous in memory)
    // into the LDS query buffer; rows past ncols read as zeros.
    auto issue_q = [&](const Item &it) {
        const int nbytes = it.ncols * D * 2;
        const __amdgpu_buffer_rsrc_t qr =
            buffer_rsrc(p.q + ((int64_t)it.b * p.Hq + it.h0) * D, nbytes);
#pragma unroll
        for (int pp = 0; pp < L::Q_PER_WAVE; ++pp) {
            const int n = min(wave + NWV * pp, L::Q_LOADS - 1);
            buffer_lds_dma16(qr, (uint32_t)(1024 * n + 16 * lane), lds + L::Q_BASE + 512 * n);
        }
    };
    // Query fragments (B operand of S^T = K Q^T) from the LDS buffer: column
    // `col` is query head h0 + col.
    auto read_q = [&](bf16x8 (&qf)[D / 16]) {
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
            qf[t] = ld_lds_bf16x8(lds + L::Q_BASE + col * D + 8 * g + 16 * t);
    };

    // Per-lane operand offsets (elements, within a stage).  K: row col (+32kb),
    // logical chunk 2t + g.  V: the transposing read of keys 4g + e (+16kk,
    // +8) and columns 32*wave + 16*dh + 4*s.
    int kof[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) kof[t] = col * D + 8 * ((2 * t + g) ^ swz_k<D>(col));
    const int tr_e = (lane & 15) >> 2, tr_s = lane & 3, tr_dh = (lane >> 4) & 1;
    const bool pv_wave = wave < D / 32;
    const int vlc = 4 * (pv_wave ? wave : 0) + 2 * tr_dh + (tr_s >> 1);
    const int vof = L::T_ELEMS + (4 * g + tr_e) * D + 8 * (vlc ^ swz_v<D>(tr_e)) + 4 * (tr_s & 1);

    f32x16 oacc = f32x16{};
    float m = -__builtin_inff();
    float lsum = 0.f;
    const float c = p.c;
    // running merge of a group's chunks (own_groups): the log-sum-exp
    // combine, in log2 units, on normalised chunk outputs
    f32x16 macc = f32x16{};
    float mm = -__builtin_inff(), ml = 0.f;

    int ci = 0, ct = 0, cstage = 0;              // compute stream: item, tile, stage
    Item citem = get_item(0);
    bf16x8 qf[D / 16];
    issue_q(citem);
#pragma unroll
    for (int i = 0; i < NSD - 1; ++i) issue_next();
    // The next item's query rows are loaded at its predecessor's second tile
    // (after the barrier that follows every wave's read of the buffer), so
    // nti - 2 tile batches follow that load before the item starts; with
    // fewer than NSD - 2 of them the per-step wait does not cover it, and
    // item starts wait for every load.
    const bool short_items = p.nti < NSD;

    for (int tau = 0; tau < ntot; ++tau) {
        // tile tau complete (the next NSD-2 may still be in flight), visible
        // to every wave; its stage's previous tile has been consumed
        if (ct == 0 && short_items) wait_vmcnt<0>();
        else wait_vmcnt<(NSD - 2) * L::PER_WAVE>();
        lds_barrier();
        issue_next();
        if (ct == 0) {
            read_q(qf);
            if (p.nti == 1 && ci + 1 < my_items) {
                wait_lgkmcnt0();                 // this wave's copy has landed ...
                lds_barrier();                   // ... and every other wave's
                issue_q(get_item(ci + 1));
            }
        } else if (ct == 1 && ci + 1 < my_items) {
            issue_q(get_item(ci + 1));
        }
        const __bf16 *st = lds + cstage * L::STAGE;

        // S^T for the tile's two 32-key blocks
        f32x16 s[BC / 32];
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
                s[kb] = mfma32x32x16(ld_lds_bf16x8(st + kof[t] + 32 * kb * D), qf[t], s[kb]);
        const int key0 = BC * ct;
        if (key0 + BC > citem.nkeys) {
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (key0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3) >= citem.nkeys)
                        s[kb][r] = -__builtin_inff();
        }
        // online softmax, lazy rescale (reference max moves by > kRescaleSlack)
        float mx = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        const float mt = half_swap_max(mx) * c;
        const bool raise = mt > m + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float m_new = raise ? mt : m;
            const float alpha = m_new == -__builtin_inff() ? 1.f : fast_exp2(m - m_new);
            lsum *= alpha;
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[r] *= alpha;
            m = m_new;
        }
        const float m_use = m == -__builtin_inff() ? 0.f : m;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
                rs += s[kb][r];
            }
        lsum += rs;
        if (pv_wave) {
#pragma unroll
            for (int kk = 0; kk < BC / 16; ++kk) {
                const bf16x8 pk = pack_p8(s[kk >> 1], 8 * (kk & 1));
                const s16x4 lo = lds_read_tr(st + vof + 16 * kk * D);
                const s16x4 hi = lds_read_tr(st + vof + (16 * kk + 8) * D);
                oacc = mfma32x32x16(concat_tr(lo, hi), pk, oacc);
            }
        }

        if (ct == p.nti - 1 && p.own_groups) {
            // chunk done: fold (O_s = acc / l, lse_s = m + log2 l) into the
            // group's merge; the last chunk writes the result
            const float lt2 = half_swap_sum(lsum);
            const float inv = lt2 > 0.f ? 1.f / lt2 : 0.f;
            const float ls2 = lt2 > 0.f ? m + fast_log2(lt2) : -__builtin_inff();
            if (ls2 != -__builtin_inff()) {
                const float mn = fmaxf(mm, ls2);
                const float a = mm == -__builtin_inff() ? 0.f : fast_exp2(mm - mn);
                const float w = fast_exp2(ls2 - mn) * inv;
#pragma unroll
                for (int r = 0; r < 16; ++r) macc[r] = macc[r] * a + oacc[r] * w;
                ml = ml * a + fast_exp2(ls2 - mn);
                mm = mn;
            }
            if (citem.sp == p.nsplit - 1) {
                const float inv2 = ml > 0.f ? 1.f / ml : 0.f;
                const int h = citem.h0 + col;
                if (col < citem.ncols) {
                    if (pv_wave) {
                        __bf16 *op = p.o + ((int64_t)citem.b * p.Hq + h) * D + 32 * wave + 4 * g;
#pragma unroll
                        for (int rq = 0; rq < 4; ++rq)
                            *reinterpret_cast<bf16x4 *>(op + 8 * rq) =
                                to_bf16x4(macc[4 * rq] * inv2, macc[4 * rq + 1] * inv2,
                                          macc[4 * rq + 2] * inv2, macc[4 * rq + 3] * inv2);
                    }
                    if (wave == 0 && g == 0 && p.lse != nullptr)
                        p.lse[(int64_t)citem.b * p.Hq + h] =
                            ml > 0.f ? (mm + fast_log2(ml)) * kLn2 : -__builtin_inff();
                }
                macc = f32x16{};
                mm = -__builtin_inff();
                ml = 0.f;
            }
            oacc = f32x16{};
            m = -__builtin_inff();
            lsum = 0.f;
            ct = 0;
            if (++ci < my_items) citem = get_item(ci);
        } else if (ct == p.nti - 1) {
            // item done: O = acc / l, LSE = (m + log2 l) ln 2
            const float lt2 = half_swap_sum(lsum);
            const float inv = lt2 > 0.f ? 1.f / lt2 : 0.f;
            const float lse_nat = lt2 > 0.f ? (m + fast_log2(lt2)) * kLn2 : -__builtin_inff();
            const int h = citem.h0 + col;
            if (col < citem.ncols) {
                if (pv_wave) {
                    const int dbase = 32 * wave + 4 * g;
                    if (p.nsplit == 1) {
                        __bf16 *op = p.o + ((int64_t)citem.b * p.Hq + h) * D + dbase;
#pragma unroll
                        for (int rq = 0; rq < 4; ++rq)
                            *reinterpret_cast<bf16x4 *>(op + 8 * rq) =
                                to_bf16x4(oacc[4 * rq] * inv, oacc[4 * rq + 1] * inv,
                                          oacc[4 * rq + 2] * inv, oacc[4 * rq + 3] * inv);
                    } else {
                        float *op = p.ws_o + (((int64_t)citem.sp * p.B + citem.b) * p.Hq + h) * D + dbase;
#pragma unroll
                        for (int rq = 0; rq < 4; ++rq) {
                            f32x4 v4 = {oacc[4 * rq] * inv, oacc[4 * rq + 1] * inv,
                                        oacc[4 * rq + 2] * inv, oacc[4 * rq + 3] * inv};
                            *reinterpret_cast<f32x4 *>(op + 8 * rq) = v4;
                        }
                    }
                }
                if (wave == 0 && g == 0) {
                    if (p.nsplit == 1) {
                        if (p.lse != nullptr) p.lse[(int64_t)citem.b * p.Hq + h] = lse_nat;
                    } else {
                        p.ws_lse[((int64_t)citem.sp * p.B + citem.b) * p.Hq + h] = lse_nat;
                    }
                }
            }
            oacc = f32x16{};
            m = -__builtin_inff();
            lsum = 0.f;
            ct = 0;
            if (++ci < my_items) citem = get_item(ci);
        } else {
            ++ct;
        }
        cstage = cstage == NSD - 1 ? 0 : cstage + 1;
    }
    wait_vmcnt<0>();                 // no load may outlive the workgroup
}

// Merge of the chunk partials: one 64-thread workgroup per (sequence, query
// head); LSE = M + log(sum_s exp(lse_s - M)), O = sum_s exp(lse_s - LSE) O_s.
template <int D>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(DecParams p) {
    const int bh = blockIdx.x;                      // b * Hq + h
    const int t = threadIdx.x;
    const int64_t stride = (int64_t)p.B * p.Hq;
    float M = -__builtin_inff();
    for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, p.ws_lse[s * stride + bh]);
    const float Mu = M == -__builtin_inff() ? 0.f : M;
    float tot = 0.f;
    for (int s = 0; s < p.nsplit; ++s) tot += fast_exp2((p.ws_lse[s * stride + bh] - Mu) * kLog2e);
    const float lse = tot > 0.f ? Mu + fast_log2(tot) * kLn2 : -__builtin_inff();
    constexpr int PER = D / 64;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int s = 0; s < p.nsplit; ++s) {
        const float ls = p.ws_lse[s * stride + bh];
        const float w = tot > 0.f ? fast_exp2((ls - lse) * kLog2e) : 0.f;
        const float *os = p.ws_o + (s * stride + bh) * D + PER * t;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += w * os[e];
    }
    __bf16 *op = p.o + (int64_t)bh * D + PER * t;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[e] = (__bf16)acc[e];
    if (p.lse != nullptr && t == 0) p.lse[bh] = lse;
}

// Tile size, ring depth and workgroups per CU of the split kernel.
#ifndef DEC_BC
#define DEC_BC 64
#endif
#ifndef DEC_NS
#define DEC_NS 4
#endif
#ifndef DEC_WPC
#define DEC_WPC 1
#endif

template <int D>
hipError_t launch_t(DecParams p, hipStream_t s) {
    constexpr int BC = DEC_BC;
    const int64_t items = (int64_t)p.B * p.Hkv * p.ncb * p.nsplit;
    if (items > 0x7fffffff) return hipErrorInvalidConfiguration;
    int cus = 0;
    hipError_t e = current_cu_count(&cus);
    if (e != hipSuccess) return e;
    p.nti = (p.chunk + BC - 1) / BC;
    const int64_t want = (int64_t)cus * DEC_WPC;
    // whole groups per workgroup when they spread evenly (at most 10 % idle)
    const int64_t groups = (int64_t)p.B * p.Hkv * p.ncb;
    const int64_t rounds = (groups + want - 1) / want;
    p.own_groups = p.nsplit > 1 && groups >= want && rounds * want * 10 <= groups * 11;
    const int64_t units = p.own_groups ? groups : items;
    const int blocks = (int)(units < want ? units : want);
    hipLaunchKernelGGL((attn_decode_split_kernel<D, BC, DEC_NS>), dim3((unsigned)blocks), dim3(NT), 0,
                       s, p);
    e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1 || p.own_groups) return e;
    hipLaunchKernelGGL(attn_decode_combine_kernel<D>, dim3((unsigned)(p.B * p.Hq)), dim3(64), 0,
                       s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecParams &p, int d, hipStream_t s) {
    if (d == 128) return launch_t<128>(p, s);
    if (d == 64) return launch_t<64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace attn
