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
//  * K and V tiles of 64 keys move HBM -> LDS with direct loads
//    (global_load_lds_dwordx4, no register staging) into a 3-stage ring:
//    while tile j is consumed, tile j+1 is ready and tile j+2 is in flight.
//    A stage is refilled only after the barrier that follows its last read
//    (the buffer-reuse rule of lecompute.fr, "Flapping Airplanes,
//    ThunderKittens and megakernels", section "Prepare the next operation
//    without overwriting the current one").  Rows are padded (K: d+8, V: d+16
//    elements) so the MFMA operand reads are free of bank conflicts; the
//    padding slots are filled by harmless duplicate loads so every load
//    instruction covers whole 1 KB runs of LDS;
//  * S^T = K*Q^T and O^T += V^T*P^T on v_mfma_f32_32x32x16_bf16.  In the S^T
//    layout each lane owns one query row, so the row max/sum are in-lane plus
//    one v_permlane32_swap, the rescale factor is a per-lane scalar, and P goes
//    from the score accumulators straight into the B operand of the second
//    product (converted to bf16) without touching LDS.  V stays row-major in
//    LDS and is read as the A operand with ds_read_b64_tr_b16;
//  * software pipeline inside each wave: iteration j issues the MFMAs of
//    S_{j+1} and, interleaved with them, the softmax of S_j; then P_j * V_j;
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
    static constexpr int VP = D + 16;                // V row pitch (elements)
    static constexpr int KS = KP / 8, VS = VP / 8;   // 16-byte slots per row
    static constexpr int DS = D / 8;                 // slots holding data
    static constexpr int K_INSTR = BC * KS / 64;     // wave-wide loads per tile
    static constexpr int V_INSTR = BC * VS / 64;
    static constexpr int N_INSTR = K_INSTR + V_INSTR;
    static constexpr int PER_WAVE = (N_INSTR + NW - 1) / NW;   // loads per wave per tile
    static constexpr int K_ELEMS = BC * KP;
    static constexpr int V_ELEMS = BC * VP;
    // loads n >= N_INSTR (rounding up to a whole number per wave) repeat a
    // real load into a 1 KB spare area at the end of the stage
    static constexpr int SPARE = K_ELEMS + V_ELEMS;
    static constexpr int STAGE = SPARE + 512;
    static_assert(BC * KS % 64 == 0 && BC * VS % 64 == 0, "a tile must be whole wave loads");
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

    // Direct-load plan: the tile's K rows (KS slots each, the last one padding)
    // then V rows (VS slots) are cut into wave-wide loads of 64 slots; wave w
    // issues loads w, w+8, ...  Lane L of load n fills slot 64*m + L of its
    // tensor; a padding slot re-reads the row's last data chunk.
    // Load n of a tile (n < N_INSTR): tensor (K, then V), slot 64*m + lane of
    // that tensor -> (row, column); a padding slot re-reads the row's last
    // chunk.  A wave's loads n >= N_INSTR repeat its load n - NW into the
    // spare area, so that every wave issues exactly PER_WAVE loads per tile.
    // Load pp of this wave: tensor (K or V), destination in the stage and
    // this lane's byte offset within the tile.  Loads past N_INSTR repeat the
    // wave's load n - NW into the spare area.
    auto plan_load = [&](int pp, bool &isv, int &ld) -> int {   // returns the slot
        const int n0 = wave + NW * pp;
        const bool spare = n0 >= L::N_INSTR;
        const int n = spare ? n0 - NW : n0;
        isv = n >= L::K_INSTR;
        ld = spare ? L::SPARE : (isv ? L::K_ELEMS + 512 * (n - L::K_INSTR) : 512 * n);
        return 64 * (isv ? n - L::K_INSTR : n) + lane;
    };
    uint32_t goff[L::PER_WAVE];      // byte offset of this lane's chunk within a tile
#pragma unroll
    for (int pp = 0; pp < L::PER_WAVE; ++pp) {
        bool isv;
        int ld;
        const int slot = plan_load(pp, isv, ld);
        const int row = isv ? slot / L::VS : slot / L::KS;
        const int colx = min(slot - row * (isv ? L::VS : L::KS), L::DS - 1) * 8;
        goff[pp] = (uint32_t)(row * hd_k + colx) * 2u;
    }
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
            bool isv;
            int ld;
            plan_load(pp, isv, ld);
            buffer_lds_dma16(isv ? vr : kr, goff[pp], dst + ld);
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

    // Weights of one tile (branch-free, so it interleaves with the next
    // tile's MFMAs): the row sum adds the fp32 weights (the LSE needs them
    // unrounded); the second product takes them rounded to bf16.
    auto weights = [&](f32x16 (&s)[BC / 32], bf16x8 (&pk)[BC / 16]) {
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
#pragma unroll
        for (int kk = 0; kk < BC / 16; ++kk) pk[kk] = pack_p8(s[kk >> 1], 8 * (kk & 1));
    };

    // lane coordinates for the transpose reads of V
    const int tr_e = (lane & 15) >> 2;       // row (key) within a 4-key group
    const int tr_s = lane & 3;               // 4-column slice
    const int tr_dh = (lane >> 4) & 1;       // which 16 columns of a 32-column block

    const int v_lane = L::K_ELEMS + (4 * g + tr_e) * L::VP + 16 * tr_dh + 4 * tr_s;
    auto pv = [&](int t, const bf16x8 (&pk)[BC / 16]) {
        const __bf16 *vs = lds + lane_base(t, v_lane);
#pragma unroll
        for (int kk = 0; kk < BC / 16; ++kk) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const s16x4 lo = lds_read_tr(vs + 16 * kk * L::VP + 32 * db);
                const s16x4 hi = lds_read_tr(vs + (16 * kk + 8) * L::VP + 32 * db);
                oacc[db] = mfma32x32x16(concat_tr(lo, hi), pk[kk], oacc[db]);
            }
        }
    };

    // One pipeline step: wait for tile j+1, refill the stage of tile j-1 with
    // tile j+2, then S_{j+1} on the matrix cores interleaved with the softmax
    // of S_j, then O += P_j V_j.  scur holds S_j, snext receives S_{j+1}.
    auto step = [&](int j, f32x16 (&scur)[BC / 32], f32x16 (&snext)[BC / 32]) {
        // tile j+1 complete (tile j+2 may still be in flight)
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
            mask(j, scur);
            row_max(scur);
            bf16x8 pk[BC / 16];
            // One basic block: the vector ALUs make this tile's weights while
            // the matrix cores compute the next tile's scores (on a wave's
            // last tile those scores are not used; the stage read is always in
            // bounds), then the second product.
            __builtin_amdgcn_s_setprio(1);
            weights(scur, pk);
            scores(j + 1, snext);
            __builtin_amdgcn_sched_barrier(0);   // keep the V reads out of the fused region
            pv(j, pk);
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
