// kda_mfma.h -- gfx950 device helpers shared by the MFMA kernels: bf16 / fp16
// vector types, the bf16 and fp16 MFMA shapes, exp2 / reciprocal, bf16 packing
// and the transposed LDS read.
//
// gfx950 facts these helpers rely on (each checked on the device):
//  * v_mfma_f32_16x16x{32,16}_bf16: lane l holds accumulator rows 4*(l/16)+j of
//    column l%16 (j = 0..3).  A operand: lane l holds row l%16, k-slots
//    8*(l/16).. (x32) or 4*(l/16).. (x16); B operand: column l%16, the same
//    k-slots.  k-slots only have to agree between A and B, so any consistent
//    permutation of k may be used.
//  * ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4 of
//    the 8-byte loads of lanes i/4, 4+i/4, 8+i/4, 12+i/4.  With lane L
//    pointing at row base+L/4, columns c0+4*(L%4).., lane i gets column c0+i
//    of rows base..base+3: an operand with k running over rows, read straight
//    from a row-major array.
//  * v_cvt_pk_bf16_f32 and v_cvt_pk_f16_f32 round to nearest even.
#pragma once

#include "kda_internal.h"

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

static __device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
static __device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
// fp16 operands (v_mfma_f32_16x16x16_f16): same lane layout as the bf16 x16 shape
static __device__ __forceinline__ f32x4 mfma16h(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
static __device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
static __device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

static __device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
static __device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
static __device__ __forceinline__ f32x4 to_f32x4(bf16x4 v) {
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
static __device__ __forceinline__ bf16x8 pack8(const float* f) {
  return bf16x8{(bf16)f[0], (bf16)f[1], (bf16)f[2], (bf16)f[3],
                (bf16)f[4], (bf16)f[5], (bf16)f[6], (bf16)f[7]};
}
static __device__ __forceinline__ void unpack8(uint4 u, float* f) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

// Transposed 8-byte LDS read (see above): pointer of this lane.
static __device__ __forceinline__ bf16x4 tr4(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// The same value from the other lane of each even/odd lane pair.
static __device__ __forceinline__ float pair_swap(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

}  // namespace kda
