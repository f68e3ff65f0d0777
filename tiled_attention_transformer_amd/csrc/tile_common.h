// Device helpers shared by the gfx950 attention kernels: vector types, the
// bf16 MFMA, LDS transpose reads, the cross-half lane swap and tile loads.
//
// Lane layouts used throughout (wave64, v_mfma_f32_32x32x16_bf16):
//   A operand (32 x 16):  lane l holds A[l % 32][8*(l/32) .. +7]
//   B operand (16 x 32):  lane l holds B[8*(l/32) .. +7][l % 32]
//   C/D       (32 x 32):  lane l, register r holds
//                         C[8*(r/4) + 4*(l/32) + (r%4)][l % 32]
// The kernels compute S^T = K * Q^T (keys as rows, query rows as columns), so
// every lane owns ONE query row (l % 32) and the softmax over keys is mostly
// in-lane; the partner lane l ^ 32 holds the other keys of the same row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Combine a value with the one held by lane l ^ 32 (the other half of the
// wave).  v_permlane32_swap returns {x[l], x[l+32]} in the low half and
// {x[l-32], x[l]} in the high half, so a commutative op of the pair gives the
// same bits in both lanes of a row.
__device__ __forceinline__ float half_swap_max(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Four consecutive fp32 values -> four bf16 (round to nearest even).
__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
    f32x2 lo = {a, b}, hi = {c, d};
    bf16x2 l2 = __builtin_convertvector(lo, bf16x2);
    bf16x2 h2 = __builtin_convertvector(hi, bf16x2);
    return __builtin_shufflevector(l2, h2, 0, 1, 2, 3);
}

// Eight fp32 values (registers r0..r0+7 of an accumulator) -> bf16x8.
__device__ __forceinline__ bf16x8 pack_p8(const f32x16 &s, int r0) {
    bf16x4 a = to_bf16x4(s[r0 + 0], s[r0 + 1], s[r0 + 2], s[r0 + 3]);
    bf16x4 b = to_bf16x4(s[r0 + 4], s[r0 + 5], s[r0 + 6], s[r0 + 7]);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lanes 4e..4e+3 each point at 4 consecutive bf16 of "row" e; lane i of the
// group then receives element i of rows 0..3.  Used to fetch 4 keys of one
// value column from a row-major V tile.  The restrict qualifier gives the
// access alias information; without it the compiler must assume the read may
// alias any buffer load still writing LDS and waits for all of them first.
__device__ __forceinline__ s16x4 lds_read_tr(const __bf16 *__restrict__ p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}

// LDS transpose read of bytes (ds_read_b64_tr_b8).  Within each group of 16
// lanes, lanes 2b and 2b+1 point at bytes 0..7 and 8..15 of "row" b
// (b = 0..7); lane i of the group then receives byte i of rows 0..7, row b in
// byte b.  Used to fetch 8 keys of one value column from a row-major fp8 V
// tile.
__device__ __forceinline__ u32x2 lds_read_tr8(const unsigned char *__restrict__ p) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p));
    return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ bf16x8 concat_tr(s16x4 lo, s16x4 hi) {
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// Direct HBM -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane L's 16 bytes from `src` land at lds_base + 16*L.  lds_base must be
// the same in every lane of the wave (it goes to M0).
__device__ __forceinline__ void lds_dma16(const void *src, void *lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// Raw buffer descriptor over [base, base + nbytes): loads past nbytes return
// zeros (checked per dword), which bounds a tile at the sequence end without
// any per-lane clamping.  0x00020000 is the gfx9-family buffer format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nbytes, 0x00020000);
}

// Cache policy of a load whose data is used once (the "nt" bit of the
// gfx940-family cache-policy operand): streamed past L2 and the infinity
// cache instead of evicting data that is reused.
constexpr int kNonTemporal = 2;

// Buffer load of 16 bytes per lane straight into LDS (buffer_load_dwordx4 ...
// lds): lane L's bytes from byte offset voff land at lds_base + 16*L.
// `policy` is the cache-policy operand (0, or kNonTemporal for data read
// once).
template <int POLICY = 0>
__device__ __forceinline__ void buffer_lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 void *lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base,
                                             16, voff, 0, 0, POLICY);
}

// s_waitcnt on the vector-memory counter only (at most n loads outstanding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt on the LDS counter only: every LDS read of this wave has landed.
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier for LDS hand-off.  The waits it needs are issued
// explicitly by the caller: wait_vmcnt for direct loads, and for LDS reads
// either their use before the barrier (an operand must have arrived) or
// wait_lgkmcnt0; s_barrier itself waits for no memory access.  The signal
// fences only stop the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ u32x4 ld_global16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ bf16x8 ld_global_bf16x8(const void *p) {
    return __builtin_bit_cast(bf16x8, ld_global16(p));
}

__device__ __forceinline__ bf16x8 ld_lds_bf16x8(const __bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ void st_lds16(__bf16 *p, u32x4 v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

}  // namespace attn
