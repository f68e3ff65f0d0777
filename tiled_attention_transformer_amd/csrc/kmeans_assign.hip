// Fused k-means assignment for gfx950: for every point, the nearest centroid
// (squared Euclidean distance, lowest index on ties) and that distance,
// without ever writing the N x K distance matrix.
//
// This is the FlashAssign step of Flash-KMeans (lefilia.fr, "Flash-KMeans :
// un K-Means exact et optimisé pour les E/S, plus de 200 fois plus rapide que
// FAISS sur GPU", the paragraph on the assignment phase): distances and the
// running minimum are computed tile by tile in on-chip memory, the way the
// attention kernels never write their score matrix.
//
//   argmin_k |x - c_k|^2 = argmax_k (x.c_k - |c_k|^2 / 2)   (|x|^2 is common)
//
// gfx950 mapping (MFMA-bound: 2*d flops per (point, centroid) pair, while
// the points are read once and the centroids stay in L2):
//  * a workgroup of 8 waves owns 256 points; wave w keeps points
//    32w .. 32w+31 in registers as the B operand of S^T = C X^T
//    (v_mfma_f32_32x32x16_bf16, fp32 accumulation), so every lane owns one
//    point and half of each tile's centroid rows;
//  * 64-centroid tiles (128 from K = 1024 on) stream through a 4-stage LDS
//    ring filled by buffer loads written straight to LDS (every wave issues
//    1/8 of each tile), one
//    workgroup barrier per tile; rows are unpadded with XOR-swizzled 16-byte
//    chunks, so the A-operand reads are free of bank conflicts;
//  * -|c|^2 / 2 of the tile after the current one is computed by all 512
//    threads with v_dot2_f32_bf16 right after the barrier that makes that
//    tile visible, into a small per-stage LDS array (the next barrier
//    publishes it); rows past K get -inf, so they never win and the last
//    tile needs no mask;
//  * the MFMA accumulators start from those values (read from LDS straight
//    into the accumulator registers), so the products come out as
//    x.c - |c|^2/2 with no further arithmetic; each lane then keeps, per
//    accumulator register, the largest value seen so far and the 32-centroid
//    block it came from (3 VALU operations per (point, centroid) pair);
//    scanning blocks in increasing order with a strict ">" keeps the lowest
//    index among equal values.  At the end the lane's 16 candidates and its
//    partner lane's (the other half of the centroid rows) are reduced with
//    the rule (value, then index), and the distance is
//    |x|^2 - 2 (x.c - |c|^2/2).
#include "kernels.h"
#include "tile_common.h"

namespace attn {

namespace {

constexpr int KW = 8;                    // waves per workgroup
constexpr int KT = 64 * KW;              // threads
constexpr int KP = 32 * KW;              // points per workgroup
constexpr int KSTG = 4;                  // ring stages

template <int D, int CT>          // CT centroids per tile
struct AsgLay {
    static constexpr int RB = D * 2;                   // bytes per centroid row
    static constexpr int CPR = RB / 16;                // 16-byte chunks per row
    static constexpr int T_BYTES = CT * RB;            // one tile
    static constexpr int LOADS = T_BYTES / 1024;       // wave-wide loads per tile
    static constexpr int LPW = LOADS / KW;             // of them per wave
    static constexpr int RING = KSTG * T_BYTES;
    static constexpr int TOTAL = RING + KSTG * CT * 4;  // + per-stage -|c|^2/2
    static_assert(LOADS % KW == 0, "tile loads must split evenly over the waves");
};

// physical chunk = logical chunk ^ swz(row): the 16 rows one ds_read_b128
// cycle touches (lanes = rows) land in distinct 16-byte bank groups
template <int D>
__device__ __forceinline__ int asg_swz(int row) {
    return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

// (value, index) order: larger x.c - |c|^2/2, then smaller index
__device__ __forceinline__ bool asg_better(float s1, int k1, float s2, int k2) {
    return s1 > s2 || (s1 == s2 && k1 < k2);
}

template <int D, int CT>
__global__ __launch_bounds__(KT)
void kmeans_assign_kernel(AssignParams p) {
    using L = AsgLay<D, CT>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::TOTAL];
    float *cnorm = reinterpret_cast<float *>(lds + L::RING);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int col = lane & 31;
    const int ntiles = (p.K + CT - 1) / CT;

    // this wave's 32 points, as B operand fragments: MFMA t contracts
    // d = 16t .. 16t+15, lane half g holding 16t + 8g ..; points past N read 0
    const int p0 = (int)blockIdx.x * KP + 32 * wave;
    // (readfirstlane keeps the clamp scalar: a vector clamp would put the
    // load descriptor in vector registers and force a loop over lanes)
    const int npts = __builtin_amdgcn_readfirstlane(min(max(p.N - p0, 0), 32));
    bf16x8 xf[D / 16];
    {
        const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(p.x + (int64_t)p0 * D, npts * D * 2);
        const uint32_t o0 = (uint32_t)((col * D + 8 * g) * 2);
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
            xf[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xr, o0 + 32 * t, 0, 0));
    }

    // tile loads: this wave fills bytes 1024m .. 1024m+1023 of each tile for
    // m = LPW*wave .. LPW*wave + LPW-1; lane L's 16 bytes are (row, physical
    // chunk) of slot 64m + L
    uint32_t goff[L::LPW];
    int dst_off[L::LPW];
#pragma unroll
    for (int i = 0; i < L::LPW; ++i) {
        const int m = L::LPW * wave + i;
        const int slot = 64 * m + lane;
        const int row = slot / L::CPR;
        const int lc = (slot % L::CPR) ^ asg_swz<D>(row);
        goff[i] = (uint32_t)(row * L::RB + 16 * lc);
        dst_off[i] = 1024 * m;
    }
    auto issue_tile = [&](int j) {
        const int r0 = j * CT;
        const int rows = min(CT, p.K - r0);
        // the descriptor ends at the last centroid: rows past it read zeros
        const __amdgpu_buffer_rsrc_t cr = buffer_rsrc(p.c + (int64_t)r0 * D, rows * L::RB);
        unsigned char *dst = lds + (j % KSTG) * L::T_BYTES;
#pragma unroll
        for (int i = 0; i < L::LPW; ++i) buffer_lds_dma16(cr, goff[i], dst + dst_off[i]);
    };

    // -|c|^2/2 of tile j (-inf past the last centroid): NPR threads per
    // centroid, D/NPR elements each, summed by v_dot2_f32_bf16 and then across
    // the NPR threads
    constexpr int NPR = KT / CT;
    constexpr int CPT = D / (8 * NPR);         // 16-byte chunks per thread
    const int nr_row = tid / NPR, nr_part = tid % NPR;
    auto tile_norms = [&](int j) {
        const unsigned char *t = lds + (j % KSTG) * L::T_BYTES + nr_row * L::RB;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int lc = CPT * nr_part + i;
            const bf16x8 v = ld_lds_bf16x8((const __bf16 *)(t + 16 * (lc ^ asg_swz<D>(nr_row))));
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const bf16x2 w = {v[e], v[e + 1]};
                acc = __builtin_amdgcn_fdot2_f32_bf16(w, w, acc, false);
            }
        }
#pragma unroll
        for (int m = 1; m < NPR; m <<= 1) acc += __shfl_xor(acc, m);
        if (nr_part == 0)
            cnorm[(j % KSTG) * CT + nr_row] = j * CT + nr_row < p.K ? -0.5f * acc : -__builtin_inff();
    };

    // A-operand offsets (bytes within a tile): row col (+32 per block),
    // logical chunk 2t + g
    int aof[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) aof[t] = col * L::RB + 16 * ((2 * t + g) ^ asg_swz<D>(col));

    float best[16];
    int bblk[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        best[r] = -__builtin_inff();
        bblk[r] = 0;
    }

    // prologue: tiles 0 .. KSTG-2 in flight, tile 0 landed and its norms made
    for (int j = 0; j < KSTG - 1; ++j)
        if (j < ntiles) issue_tile(j);
    if (ntiles > 2) wait_vmcnt<2 * L::LPW>();
    else if (ntiles == 2) wait_vmcnt<L::LPW>();
    else wait_vmcnt<0>();
    lds_barrier();
    tile_norms(0);

    for (int j = 0; j < ntiles; ++j) {
        // tile j+1 landed (own loads; tiles issued after it may be pending)
        const int after = min(j + KSTG - 2, ntiles - 1) - (j + 1);
        if (after >= 1) wait_vmcnt<L::LPW>();
        else wait_vmcnt<0>();
        // every wave's part of tile j+1 and the norms of tile j are visible,
        // and every wave is done with tile j-1, whose stage is refilled now
        wait_lgkmcnt0();
        lds_barrier();
        if (j + KSTG - 1 < ntiles) issue_tile(j + KSTG - 1);
        if (j + 1 < ntiles) tile_norms(j + 1);

        const unsigned char *st = lds + (j % KSTG) * L::T_BYTES;
        const float *nrm = cnorm + (j % KSTG) * CT;
#pragma unroll
        for (int kb = 0; kb < CT / 32; ++kb) {
            // accumulators start at -|c|^2/2 of this lane's rows 8q + 4g .. +3
            f32x16 s;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(nrm + 32 * kb + 8 * q + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * q + e] = v[e];
            }
#pragma unroll
            for (int t = 0; t < D / 16; ++t)
                s = mfma32x32x16(ld_lds_bf16x8((const __bf16 *)(st + kb * 32 * L::RB + aof[t])), xf[t], s);
            const int blk = (CT / 32) * j + kb;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool gt = s[r] > best[r];
                best[r] = gt ? s[r] : best[r];
                bblk[r] = gt ? blk : bblk[r];
            }
        }
    }

    // the lane's best over its rows, then over the partner lane's rows
    float bd = best[0];
    int bk = 32 * bblk[0] + 4 * g;
#pragma unroll
    for (int r = 1; r < 16; ++r) {
        const int k = 32 * bblk[r] + 8 * (r >> 2) + 4 * g + (r & 3);
        if (asg_better(best[r], k, bd, bk)) {
            bd = best[r];
            bk = k;
        }
    }
    {
        const auto sd = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, bd),
                                                         __builtin_bit_cast(uint32_t, bd), false, false);
        const auto sk = __builtin_amdgcn_permlane32_swap((uint32_t)bk, (uint32_t)bk, false, false);
        // lane l < 32 receives lane l + 32's values in the second word, and
        // lane l >= 32 lane l - 32's in the first
        const float od = __builtin_bit_cast(float, (uint32_t)(g ? sd[0] : sd[1]));
        const int ok = (int)(g ? sk[0] : sk[1]);
        if (asg_better(od, ok, bd, bk)) {
            bd = od;
            bk = ok;
        }
    }
    // |x|^2 of the lane's point: its half of the coordinates, plus the partner's
    float xx = 0.f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 w = {xf[t][e], xf[t][e + 1]};
            xx = __builtin_amdgcn_fdot2_f32_bf16(w, w, xx, false);
        }
    xx = half_swap_sum(xx);
    if (g == 0 && col < npts) {
        p.idx[p0 + col] = bk;
        if (p.dist != nullptr) p.dist[p0 + col] = fmaxf(__builtin_fmaf(-2.f, bd, xx), 0.f);
    }
}

}  // namespace

hipError_t launch_kmeans_assign(const AssignParams &p, int d, hipStream_t s) {
    const int64_t blocks = ((int64_t)p.N + KP - 1) / KP;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    // 128-centroid tiles halve the per-tile barrier, wait and norm work; with
    // few centroids the half-empty last tile and the deeper prologue cost more
    const bool wide = p.K >= 1024;
    if (d == 128) {
        if (wide) hipLaunchKernelGGL((kmeans_assign_kernel<128, 128>), dim3((unsigned)blocks), dim3(KT), 0, s, p);
        else hipLaunchKernelGGL((kmeans_assign_kernel<128, 64>), dim3((unsigned)blocks), dim3(KT), 0, s, p);
    } else if (d == 64) {
        if (wide) hipLaunchKernelGGL((kmeans_assign_kernel<64, 128>), dim3((unsigned)blocks), dim3(KT), 0, s, p);
        else hipLaunchKernelGGL((kmeans_assign_kernel<64, 64>), dim3((unsigned)blocks), dim3(KT), 0, s, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace attn
