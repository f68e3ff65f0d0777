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
// gfx950 mapping:
//  * one workgroup per (sequence, KV head, block of <= 32 query heads, chunk):
//    all query heads of a GQA group share ONE pass over the chunk's K and V,
//    so every cache byte is read from HBM once;
//  * K/V tiles of 128 keys stream HBM -> registers -> LDS with 16-byte
//    coalesced loads; the next tile's loads are issued before the current
//    tile is computed;
//  * each wave takes 32 keys of a tile and runs the same MFMA micro-kernel as
//    the prefill (S^T = K Q^T, then O^T += V^T P^T) with the query heads as the
//    32 columns; the four waves' partial (max, sum, output) states are merged
//    through LDS at the end;
//  * the chunk result is written normalised, in fp32, with its natural-log
//    LSE, and a second small kernel merges the chunks; with a single chunk
//    the first kernel writes the final bf16 output directly.
#include "kernels.h"
#include "tile_common.h"

namespace attn {

namespace {

constexpr int BC = kDecBc, NT = kDecThreads, NCOL = kDecCols;

template <int D>
struct DecLds {
    static constexpr int KP = D + 8;
    static constexpr int VP = D + 16;
    static constexpr int K_ELEMS = BC * KP;
    static constexpr int V_ELEMS = BC * VP;
    static constexpr int ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int CHUNKS = BC * D / 8 / NT;
    // merge area (reuses the tile area): per wave m[32], l[32], O[32][D+1]
    // fp32; the odd column pitch keeps the 32 lanes of a write on 32 banks
    static constexpr int OP = D + 1;
    static constexpr int MERGE_FLOATS = 4 * (2 * NCOL + NCOL * OP);
    static_assert(MERGE_FLOATS * 4 <= ELEMS * 2, "merge area must fit in the tile area");
};

template <int D>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_decode_split_kernel(DecParams p) {
    using L = DecLds<D>;
    __shared__ __attribute__((aligned(16))) __bf16 lds[L::ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 5;
    const int col = lane & 31;

    // blockIdx.x -> (b, hk, cb, split), split fastest
    int id = blockIdx.x;
    const int sp = id % p.nsplit;
    id /= p.nsplit;
    const int cb = id % p.ncb;
    id /= p.ncb;
    const int hk = id % p.Hkv;
    const int b = id / p.Hkv;

    const int k_lo = sp * p.chunk;
    const int k_hi = min(p.Skv, k_lo + p.chunk);
    const int nkeys = k_hi > k_lo ? k_hi - k_lo : 0;
    const int nt = (nkeys + BC - 1) / BC;

    const int ncols = min(NCOL, p.group - NCOL * cb);   // valid query heads here
    const int h0 = hk * p.group + NCOL * cb;             // first query head of the block

    // Q fragments: column `col` is query head h0 + col.
    bf16x8 qf[D / 16];
    {
        const __bf16 *qp = p.q + ((int64_t)b * p.Hq + h0 + col) * D + 8 * g;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
            if (col < ncols) qf[t] = ld_global_bf16x8(qp + 16 * t);
            else qf[t] = bf16x8{};
        }
    }

    const int64_t hd_k = (int64_t)p.Hkv * D;
    const __bf16 *kbase = p.k + ((int64_t)b * p.Skv + k_lo) * hd_k + (int64_t)hk * D;
    const __bf16 *vbase = p.v + ((int64_t)b * p.Skv + k_lo) * hd_k + (int64_t)hk * D;
    u32x4 kreg[L::CHUNKS], vreg[L::CHUNKS];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int i = 0; i < L::CHUNKS; ++i) {
            const int c = tid + NT * i;
            const int row = c / (D / 8);
            const int cc = (c % (D / 8)) * 8;
            const int key = j * BC + row;        // relative to k_lo
            if (key < nkeys) {
                kreg[i] = ld_global16(kbase + (int64_t)key * hd_k + cc);
                vreg[i] = ld_global16(vbase + (int64_t)key * hd_k + cc);
            } else {
                kreg[i] = u32x4{0, 0, 0, 0};
                vreg[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&]() {
        __bf16 *ks = lds;
        __bf16 *vs = lds + L::K_ELEMS;
#pragma unroll
        for (int i = 0; i < L::CHUNKS; ++i) {
            const int c = tid + NT * i;
            const int row = c / (D / 8);
            const int cc = (c % (D / 8)) * 8;
            st_lds16(ks + row * L::KP + cc, kreg[i]);
            st_lds16(vs + row * L::VP + cc, vreg[i]);
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m = -__builtin_inff();
    float lsum = 0.f;
    const float c = p.c;
    const int tr_e = (lane & 15) >> 2;
    const int tr_s = lane & 3;
    const int tr_dh = (lane >> 4) & 1;

    if (nt > 0) load_tile(0);
    for (int j = 0; j < nt; ++j) {
        store_tile();
        __syncthreads();
        if (j + 1 < nt) load_tile(j + 1);
        const int kw0 = j * BC + 32 * wave;     // first key of this wave (relative)
        if (kw0 < nkeys) {
            const __bf16 *kr = lds + (32 * wave + col) * L::KP + 8 * g;
            f32x16 s = f32x16{};
#pragma unroll
            for (int t = 0; t < D / 16; ++t) s = mfma32x32x16(ld_lds_bf16x8(kr + 16 * t), qf[t], s);
            if (kw0 + 32 > nkeys) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kw0 + 8 * (r >> 2) + 4 * g + (r & 3) >= nkeys) s[r] = -__builtin_inff();
            }
            float mx = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = half_swap_max(mx);
            const float m_new = fmaxf(m, mx * c);
            const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
            const float alpha = fast_exp2(m - m_use);
            float rs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = fast_exp2(__builtin_fmaf(s[r], c, -m_use));
                rs += s[r];
            }
            const bf16x8 pk0 = pack_p8(s, 0), pk1 = pack_p8(s, 8);
            lsum = lsum * alpha + rs;
            m = m_new;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            const __bf16 *vs = lds + L::K_ELEMS;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 pb = kk ? pk1 : pk0;
                const __bf16 *v0 =
                    vs + (32 * wave + 16 * kk + 4 * g + tr_e) * L::VP + 16 * tr_dh + 4 * tr_s;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const s16x4 lo = lds_read_tr(v0 + 32 * db);
                    const s16x4 hi = lds_read_tr(v0 + 8 * L::VP + 32 * db);
                    oacc[db] = mfma32x32x16(concat_tr(lo, hi), pb, oacc[db]);
                }
            }
        }
        __syncthreads();
    }

    // Merge the four waves' states through LDS (the tile area is free now:
    // the last barrier above follows every read of it).
    float *mw = reinterpret_cast<float *>(lds);     // [4][32]
    float *lw = mw + 4 * NCOL;                      // [4][32]
    float *ow = lw + 4 * NCOL;                      // [4][32][D]
    const float lt = half_swap_sum(lsum);
    if (g == 0) {
        mw[wave * NCOL + col] = m;
        lw[wave * NCOL + col] = lt;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dcol = 32 * db + 8 * (r >> 2) + 4 * g + (r & 3);
            ow[(wave * NCOL + col) * L::OP + dcol] = oacc[db][r];
        }
    __syncthreads();

    // 32 columns x D values over 256 threads: thread t takes column t % 32
    // and PER consecutive values (lanes of a wave walk the columns).
    constexpr int PER = NCOL * D / NT;
    const int mc = tid % NCOL;                      // column
    const int d0 = (tid / NCOL) * PER;
    if (mc >= ncols) return;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mw[w * NCOL + mc]);
    const float Mu = M == -__builtin_inff() ? 0.f : M;
    float wgt[4];
    float Ltot = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        wgt[w] = fast_exp2(mw[w * NCOL + mc] - Mu);
        Ltot += wgt[w] * lw[w * NCOL + mc];
    }
    const float inv = Ltot > 0.f ? 1.f / Ltot : 0.f;
    const int h = h0 + mc;
    const float lse_nat = Ltot > 0.f ? (M + fast_log2(Ltot)) * kLn2 : -__builtin_inff();
    if (p.nsplit == 1) {
        __bf16 *op = p.o + ((int64_t)b * p.Hq + h) * D + d0;
#pragma unroll
        for (int e = 0; e < PER; e += 4) {
            float v4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) acc += wgt[w] * ow[(w * NCOL + mc) * L::OP + d0 + e + u];
                v4[u] = acc * inv;
            }
            *reinterpret_cast<bf16x4 *>(op + e) = to_bf16x4(v4[0], v4[1], v4[2], v4[3]);
        }
        if (p.lse != nullptr && d0 == 0) p.lse[(int64_t)b * p.Hq + h] = lse_nat;
    } else {
        float *op = p.ws_o + (((int64_t)sp * p.B + b) * p.Hq + h) * D + d0;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) acc += wgt[w] * ow[(w * NCOL + mc) * L::OP + d0 + e];
            op[e] = acc * inv;
        }
        if (d0 == 0) p.ws_lse[((int64_t)sp * p.B + b) * p.Hq + h] = lse_nat;
    }
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

template <int D>
hipError_t launch_t(const DecParams &p, hipStream_t s) {
    const int64_t blocks = (int64_t)p.B * p.Hkv * p.ncb * p.nsplit;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(attn_decode_split_kernel<D>, dim3((unsigned)blocks), dim3(NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
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
