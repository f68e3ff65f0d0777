// Fused tiled attention forward (prefill) for gfx950.
//
// Method (lecompute.fr, "FlashAttention-4 : limites du calcul matriciel"):
// scores Q*K^T, a softmax into weights that sum to one, and a second product
// with V (section "Entre deux multiplications il faut fabriquer les poids"),
// computed tile by tile so the score matrix never leaves the chip (same
// section), with a running maximum as the common scale of the old and new
// contributions (section "Déplacer une partie des exponentielles").
//
// gfx950 mapping:
//  * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//    owns 32 rows and keeps its Q fragment, running max/sum and the fp32
//    output accumulator in registers for the whole key loop;
//  * K and V tiles of 64 keys are staged HBM -> registers -> LDS with 16-byte
//    coalesced loads and two LDS stages: the next tile's global loads are in
//    flight while the current tile is computed, and one barrier per tile
//    guards stage reuse (a stage is rewritten only after every wave has
//    finished reading it);
//  * S^T = K*Q^T and O^T += V^T*P^T run on v_mfma_f32_32x32x16_bf16.  In the
//    S^T layout each lane owns one query row, so the row max/sum are in-lane
//    plus one v_permlane32_swap, the rescale factor is a per-lane scalar, and
//    P goes from the score accumulators straight into the B operand of the
//    second product (converted to bf16) without touching LDS;
//  * V stays row-major in LDS and is read as the A operand with
//    ds_read_b64_tr_b16 (4 keys of one column per read);
//  * softmax in base 2: P = exp2(s*c - m) with c = scale*log2(e) folded into
//    one FMA; LSE = (m + log2 l) * ln 2;
//  * under the causal mask, tiles above a query tile's diagonal are never
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

constexpr int BR = kFwdBr, BC = kFwdBc, NT = kFwdThreads;

template <int D>
struct FwdLds {
    static constexpr int KP = D + 8;    // K row pitch (elements): conflict-free b128 reads
    static constexpr int VP = D + 16;   // V row pitch: spreads the 4 rows of a transpose read
    static constexpr int K_ELEMS = BC * KP;
    static constexpr int V_ELEMS = BC * VP;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int CHUNKS = BC * D / 8 / NT;   // 16-byte chunks per thread per tensor
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(FwdParams p) {
    using L = FwdLds<D>;
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * L::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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

    // Global -> register staging of one K/V tile.  Thread tid moves the
    // 16-byte chunks tid + 256*i of the tile (row = key, 16 chunks per row for
    // d = 128), so each wave instruction reads whole 256-byte key rows.
    const __bf16 *kbase = p.k + krow0 * hd_k + (int64_t)hk * D;
    const __bf16 *vbase = p.v + krow0 * hd_k + (int64_t)hk * D;
    const int64_t tile_step = (int64_t)BC * hd_k;
    int64_t goff[L::CHUNKS];     // element offset of chunk i within a tile
    int lrow[L::CHUNKS];         // key row of chunk i within a tile
#pragma unroll
    for (int i = 0; i < L::CHUNKS; ++i) {
        const int cidx = tid + NT * i;
        lrow[i] = cidx / (D / 8);
        goff[i] = (int64_t)lrow[i] * hd_k + (cidx % (D / 8)) * 8;
    }
    u32x4 kreg[L::CHUNKS], vreg[L::CHUNKS];
    auto load_tile = [&](int j) {
        const __bf16 *kt = kbase + j * tile_step;
        const __bf16 *vt = vbase + j * tile_step;
        if ((j + 1) * BC <= Skv) {                 // whole tile in range (uniform)
#pragma unroll
            for (int i = 0; i < L::CHUNKS; ++i) {
                kreg[i] = ld_global16(kt + goff[i]);
                vreg[i] = ld_global16(vt + goff[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < L::CHUNKS; ++i) {
                const bool in = j * BC + lrow[i] < Skv;
                kreg[i] = in ? ld_global16(kt + goff[i]) : u32x4{0, 0, 0, 0};
                vreg[i] = in ? ld_global16(vt + goff[i]) : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&](int st) {
        __bf16 *ks = lds + st * L::STAGE;
        __bf16 *vs = ks + L::K_ELEMS;
#pragma unroll
        for (int i = 0; i < L::CHUNKS; ++i) {
            const int cidx = tid + NT * i;
            const int cc = (cidx % (D / 8)) * 8;
            st_lds16(ks + lrow[i] * L::KP + cc, kreg[i]);
            st_lds16(vs + lrow[i] * L::VP + cc, vreg[i]);
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m = -__builtin_inff();     // running max, scaled base-2 units
    float lsum = 0.f;                // this lane's share of the running sum
    const float c = p.c;

    // lane coordinates for the transpose reads of V
    const int tr_e = (lane & 15) >> 2;       // row (key) within a 4-key group
    const int tr_s = lane & 3;               // 4-column slice
    const int tr_dh = (lane >> 4) & 1;       // which 16 columns of a 32-column block

    if (nt > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
    }
    for (int j = 0; j < nt; ++j) {
        const int st = j & 1;
        if (j + 1 < nt) load_tile(j + 1);
        const int key0 = j * BC;
        const bool wave_live = wrow0 < Sq && (!CAUSAL || key0 <= wrow0 + 31 + off);
        if (wave_live) {
            const __bf16 *ks = lds + st * L::STAGE;
            const __bf16 *vs = ks + L::K_ELEMS;
            // S^T = K Q^T for the BC/32 key blocks; the independent chains are
            // interleaved and each K fragment is read from LDS one step ahead.
            f32x16 s[BC / 32];
            {
                bf16x8 kf[2][BC / 32];
#pragma unroll
                for (int kb = 0; kb < BC / 32; ++kb) {
                    s[kb] = f32x16{};
                    kf[0][kb] = ld_lds_bf16x8(ks + (32 * kb + col) * L::KP + 8 * g);
                }
#pragma unroll
                for (int t = 0; t < D / 16; ++t) {
                    if (t + 1 < D / 16) {
#pragma unroll
                        for (int kb = 0; kb < BC / 32; ++kb)
                            kf[(t + 1) & 1][kb] =
                                ld_lds_bf16x8(ks + (32 * kb + col) * L::KP + 8 * g + 16 * (t + 1));
                    }
#pragma unroll
                    for (int kb = 0; kb < BC / 32; ++kb)
                        s[kb] = mfma32x32x16(kf[t & 1][kb], qf[t], s[kb]);
                }
            }
            // Mask keys past the row's causal limit or past the sequence end
            // (only tiles that cross the diagonal or the end need it).
            const bool need_mask = key0 + BC > Skv || (CAUSAL && key0 + BC - 1 > wrow0 + off);
            if (need_mask) {
                int lim = Skv - 1;
                if (CAUSAL) lim = min(lim, qr + off);
                lim -= key0 + 4 * g;                  // this lane's keys: key0 + 4g + const
#pragma unroll
                for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -__builtin_inff();
            }
            float mx = -__builtin_inff();
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            const float mt = half_swap_max(mx) * c;   // tile row max, scaled log2 units
            // Lazy rescaling: the reference max m only moves when a row's tile
            // max exceeds it by more than kRescaleSlack, so exp2(s*c - m) stays
            // <= 2^kRescaleSlack and most tiles skip the O rescale entirely.
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
            // P = exp2(s*c - m); the row sum adds the fp32 values (the LSE
            // needs them unrounded) and P enters the second product as bf16.
            bf16x8 pk[BC / 16];
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_use));
                    lsum += s[kb][r];
                }
#pragma unroll
            for (int kk = 0; kk < BC / 16; ++kk) pk[kk] = pack_p8(s[kk >> 1], 8 * (kk & 1));
#pragma unroll
            for (int kk = 0; kk < BC / 16; ++kk) {
                const __bf16 *v0 = vs + (16 * kk + 4 * g + tr_e) * L::VP + 16 * tr_dh + 4 * tr_s;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const s16x4 lo = lds_read_tr(v0 + 32 * db);
                    const s16x4 hi = lds_read_tr(v0 + 8 * L::VP + 32 * db);
                    oacc[db] = mfma32x32x16(concat_tr(lo, hi), pk[kk], oacc[db]);
                }
            }
        }
        if (j + 1 < nt) store_tile(st ^ 1);
        __syncthreads();
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
