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
// what the schedule below is built around: the softmax of one key tile runs
// on the vector ALUs while the matrix cores already compute the scores of the
// next tile (section "Faire avancer plusieurs tuiles sans écraser leurs
// données" describes the same overlap with thread-group roles on SM100; here
// one wave interleaves both streams).
//
// gfx950 mapping:
//  * one workgroup = 8 waves = 256 query rows of one (batch, head), one
//    workgroup per CU (two waves per SIMD); each wave owns 32 rows and keeps
//    its Q fragment, running max/sum and fp32 output accumulator in registers;
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
//  * S^T = K*Q^T and O^T += V^T*P^T on v_mfma_f32_32x32x16_bf16.  In the S^T
//    layout each lane owns one query row, so the row max/sum are in-lane plus
//    one v_permlane32_swap, the rescale factor is a per-lane scalar, and P goes
//    from the score accumulators straight into the B operand of the second
//    product (converted to bf16) without touching LDS.  V stays row-major in
//    LDS and is read as the A operand with ds_read_b64_tr_b16;
//  * software pipeline inside each wave: iteration j issues the MFMAs of
//    S_{j+1} and, interleaved with them, the softmax of S_j; then P_j * V_j.
//    Both parts run as groups of four MFMAs split by scheduling barriers, and
//    every LDS operand read is issued one group ahead of its MFMAs;
//  * softmax in base 2: P = exp2(s*c - m) with c = scale*log2(e) folded into
//    one FMA; the reference max m moves only when a row max grows by more
//    than 2^8, so most tiles skip the output rescale; LSE = (m + log2 l)*ln 2;
//  * under the causal mask, key tiles above a query tile's diagonal are never
//    loaded, waves skip tiles above their own rows, and only tiles that cross
//    the diagonal or the sequence end evaluate the mask;
//  * the grid is 1-D, ordered (tile rank, batch*head) so that every head's
//    longest tile is dispatched first under the causal mask, and all tiles of
//    one head land on the same XCD (workgroups go round-robin over the 8 XCDs)
//    when batch*heads is a multiple of 8, so they share that XCD's L2 for K/V.
#include "kernels.h"
#include "tile_common.h"

namespace attn {

namespace {

constexpr int NW = kFwdWaves;
constexpr int NT = kFwdThreads;
constexpr int BR = kFwdBr;
constexpr int BC = kFwdBc;
constexpr int NS = 4;                 // LDS ring stages

template <int D>
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

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p) {
    using L = FwdLay<D>;
    __shared__ __attribute__((aligned(16))) __bf16 lds[NS * L::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;            // which half of the wave
    const int col = lane & 31;          // query row within the wave

    const int BH = p.nbatch * p.Hq;
    const int id = blockIdx.x;
    const int tile_rank = id / BH;
    const int bh = id - tile_rank * BH;
    const int b = bh / p.Hq;
    const int h = bh - b * p.Hq;
    const int hk = h / p.group;

    int64_t qrow0, krow0;
    int Sq, Skv;
    int64_t lse_base, lse_hstride;
    if constexpr (VARLEN) {
        const int qs = p.cu_q[b], qe = p.cu_q[b + 1];
        const int ks = p.cu_k[b], ke = p.cu_k[b + 1];
        const bool ok = qs >= 0 && qe >= qs && qe <= p.total_q && ks >= 0 && ke >= ks &&
                        ke <= p.total_k;
        Sq = ok ? qe - qs : 0;
        Skv = ok ? ke - ks : 0;
        qrow0 = qs;
        krow0 = ks;
        lse_base = qs;
        lse_hstride = p.total_q;
    } else {
        Sq = p.Sq;
        Skv = p.Skv;
        qrow0 = (int64_t)b * Sq;
        krow0 = (int64_t)b * Skv;
        lse_base = (int64_t)b * p.Hq * Sq;
        lse_hstride = Sq;
    }
    const int tile = CAUSAL ? (p.ntiles - 1 - tile_rank) : tile_rank;
    const int q0 = tile * BR;
    if (q0 >= Sq) return;                        // whole workgroup: uniform exit

    const int off = Skv - Sq;                    // bottom-right causal offset
    int kend = Skv;
    if (CAUSAL) kend = min(Skv, q0 + BR + off);  // one past the last key any row may see
    const int nt = kend > 0 ? (kend + BC - 1) / BC : 0;

    const int wrow0 = q0 + 32 * wave;            // first row of this wave
    const int qr = wrow0 + col;                  // this lane's query row
    // key tiles this wave computes (its rows' causal reach; none past Sq)
    int ntw = 0;
    if (wrow0 < Sq) {
        int wk = Skv;
        if (CAUSAL) wk = min(Skv, min(wrow0 + 32, Sq) + off);
        ntw = wk > 0 ? min(nt, (wk + BC - 1) / BC) : 0;
    }
    const int64_t hd_q = (int64_t)p.Hq * D;
    const int64_t hd_k = (int64_t)p.Hkv * D;

    // Q fragments (B operand of S^T = K Q^T), resident for the whole loop.
    bf16x8 qf[D / 16];
    {
        const __bf16 *qp = p.q + (qrow0 + qr) * hd_q + (int64_t)h * D + 8 * g;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            if (qr < Sq) qf[t] = ld_global_bf16x8(qp + 16 * t);
            else qf[t] = bf16x8{};
        }
    }

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
    const __bf16 *kbase = p.k + krow0 * hd_k + (int64_t)hk * D;
    const __bf16 *vbase = p.v + krow0 * hd_k + (int64_t)hk * D;
    auto issue = [&](int t) {
        const int key0 = t * BC;
        __bf16 *dst = lds + (t % NS) * L::STAGE;
        // the descriptors end at the last valid key, so rows past the sequence
        // end read as zeros
        const int rows = min(BC, Skv - key0);
        const int nbytes = (int)(((int64_t)(rows - 1) * hd_k + D) * 2);
        const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(kbase + (int64_t)key0 * hd_k, nbytes);
        const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(vbase + (int64_t)key0 * hd_k, nbytes);
#pragma unroll
        for (int pp = 0; pp < L::PER_WAVE; ++pp) {
            const bool isv = pp == L::PER_WAVE - 1 ? last_is_v : pp >= L::KW;
            buffer_lds_dma16(isv ? vr : kr, goff[pp], dst + ldo[pp]);
        }
    };

    // LDS element offset of this lane's first operand in stage t.  Kept
    // opaque so that each read is one address register plus an immediate
    // offset (otherwise the optimizer keeps one register per read).
    auto lane_base = [&](int t, int lane_off) -> int {
        int o = (t % NS) * L::STAGE + lane_off;
        asm volatile("" : "+v"(o));
        return o;
    };
    const int k_lane = col * L::KP + 8 * g;

    // S^T = K Q^T for one tile: two 32-key blocks, chains interleaved.
    auto scores = [&](int t, f32x16 (&s)[BC / 32]) {
        const __bf16 *ks = lds + lane_base(t, k_lane);
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int tt = 0; tt < D / 16; ++tt)
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
                s[kb] = mfma32x32x16(ld_lds_bf16x8(ks + 32 * kb * L::KP + 16 * tt), qf[tt], s[kb]);
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m = -__builtin_inff();     // reference max, scaled base-2 units
    float lsum = 0.f;                // this lane's share of the running sum
    const float c = p.c;

    // Mask keys past each row's causal limit or past the sequence end; only
    // tiles that cross the diagonal or the end need it.
    auto mask = [&](int t, f32x16 (&s)[BC / 32]) {
        const int key0 = t * BC;
        if (key0 + BC > Skv || (CAUSAL && key0 + BC - 1 > wrow0 + off)) {
            int lim = Skv - 1;
            if (CAUSAL) lim = min(lim, qr + off);
            lim -= key0 + 4 * g;                  // this lane's keys: key0 + 4g + const
            // opaque to the optimizer: otherwise it folds 4g into the 32
            // constants below and keeps them live (32 registers) across the loop
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -__builtin_inff();
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
    // 2g, 2g+1 (FPG fragments); weight chunk g makes pk[] entries of the same
    // rank.
    constexpr int NG = D / 32;                   // score groups per tile
    constexpr int FPG = 2 * (BC / 32);           // K fragments per group
    constexpr int VPL = (BC / 2) / NG;           // weights per lane per chunk
    constexpr int NV = 2 * (D / 32);             // V transpose reads per key slice
    static_assert(VPL % 8 == 0, "a weight chunk must fill whole pk entries");
    auto read_k = [&](int t, int grp, bf16x8 (&kf)[FPG]) {
        const __bf16 *ks = lds + lane_base(t, k_lane);
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
    auto read_v = [&](int t, int kk, s16x4 (&vf)[NV]) {
        const __bf16 *vs = lds + lane_base(t, v_lane);
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

    // One pipeline step: wait for tile j+1, refill the stage of tile j-1 with
    // tile j+3, then S_{j+1} on the matrix cores interleaved with the softmax
    // of S_j, then O += P_j V_j.  scur holds S_j, snext receives S_{j+1}.
    auto step = [&](int j, f32x16 (&scur)[BC / 32], f32x16 (&snext)[BC / 32]) {
        // tile j+1 complete (tiles j+2, j+3 may still be in flight)
        if (j + 2 < nt) wait_vmcnt<L::PER_WAVE>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (j + 3 < nt) issue(j + 3);
        if (j >= ntw) {
            // no tile for this wave: snext gets a placeholder, so that no score
            // buffer has to stay live across steps
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
                snext[kb] = __builtin_nondeterministic_value(snext[kb]);
        }
        if (j < ntw) {
            // the first K group of tile j+1 loads during the mask and row max
            // (on a wave's last tile those scores are not used; the stage
            // read is always in bounds)
            bf16x8 kf[2][FPG];
            read_k(j + 1, 0, kf[0]);
            mask(j, scur);
            row_max(scur);
            __builtin_amdgcn_s_setprio(1);
            const float m_use = m == -__builtin_inff() ? 0.f : m;
            float rs = 0.f;
            bf16x8 pk[BC / 16];
            s16x4 vf[2][NV];
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) snext[kb] = f32x16{};
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                __builtin_amdgcn_sched_barrier(0);
                if (g + 1 < NG) read_k(j + 1, g + 1, kf[(g + 1) & 1]);
                else read_v(j, 0, vf[0]);
                mfma_k(g, kf[g & 1], snext);
                weight_chunk(g, scur, pk, m_use, rs);
            }
            lsum += rs;
#pragma unroll
            for (int kk = 0; kk < BC / 16; ++kk) {
                __builtin_amdgcn_sched_barrier(0);
                if (kk + 1 < BC / 16) read_v(j, kk + 1, vf[(kk + 1) & 1]);
                mfma_v(kk, vf[kk & 1], pk);
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        }
    };

    // score buffers: a step reads scur only for tiles whose scores it wrote
    f32x16 sa[BC / 32], sb[BC / 32];
    if (nt > 0) {
        issue(0);
        if (nt > 1) issue(1);
        if (nt > 2) issue(2);
        // tile 0 complete (tiles 1, 2 may still be in flight), visible to all waves
        if (nt > 2) wait_vmcnt<2 * L::PER_WAVE>();
        else if (nt > 1) wait_vmcnt<L::PER_WAVE>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (ntw > 0) scores(0, sa);
    }
    // unrolled by two so the score buffers alternate without copies; the
    // second step always runs (past the end it only waits at the barrier)
    for (int j = 0; j < nt; j += 2) {
        step(j, sa, sb);
        step(j + 1, sb, sa);
    }

    // Epilogue: O = acc / l (bf16), LSE = (m + log2 l) * ln 2.
    if (wrow0 >= Sq) return;
    const float lt = half_swap_sum(lsum);
    if (qr >= Sq) return;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    __bf16 *op = p.o + (qrow0 + qr) * hd_q + (int64_t)h * D + 4 * g;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const bf16x4 v4 = to_bf16x4(oacc[db][4 * rq] * inv, oacc[db][4 * rq + 1] * inv,
                                        oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv);
            *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * rq) = v4;
        }
    if (p.lse != nullptr && g == 0)
        p.lse[lse_base + (int64_t)h * lse_hstride + qr] =
            lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -__builtin_inff();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_t(const FwdParams &p, hipStream_t s) {
    const int64_t blocks = (int64_t)p.ntiles * p.nbatch * p.Hq;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)blocks), dim3(NT), 0,
                       s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams &p, int d, bool causal, bool varlen, hipStream_t s) {
    if (d == 128) {
        if (varlen) return causal ? launch_t<128, true, true>(p, s) : launch_t<128, false, true>(p, s);
        return causal ? launch_t<128, true, false>(p, s) : launch_t<128, false, false>(p, s);
    }
    if (d == 64) {
        if (varlen) return causal ? launch_t<64, true, true>(p, s) : launch_t<64, false, true>(p, s);
        return causal ? launch_t<64, true, false>(p, s) : launch_t<64, false, false>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
