// Device pieces shared by the two attention kernels (k_attn.hip,
// k_attn_group.hip): the score and P.V products on the bf16 16x16x32 MFMA,
// with fp32 operands split into bf16 hi + lo parts.
#pragma once
#include "attn_group.h"

namespace vs {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStep = kAttnStepKeys;  // keys per attention step (two 16-key blocks)

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Value of another lane of the same 16-lane row (DPP: quad_perm, mirrors).
template <int CTRL>
__device__ __forceinline__ float row_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Max and sum over the 16 lanes of a row, left in every lane of it.  Lanes
// are combined as pairs, quads, quad pairs, then halves (quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror, row_mirror); at each stage every lane
// of a group holds the same value, so the sums carry the same bits as a
// butterfly over lane xor 1, 2, 4, 8, at one VALU operation per stage rather
// than an LDS permute.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, row_dpp<0xB1>(v));
  v = fmaxf(v, row_dpp<0x4E>(v));
  v = fmaxf(v, row_dpp<0x141>(v));
  return fmaxf(v, row_dpp<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += row_dpp<0xB1>(v);
  v += row_dpp<0x4E>(v);
  v += row_dpp<0x141>(v);
  return v + row_dpp<0x140>(v);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even), packed low first: one
// v_cvt_pk_bf16_f32, the same bits as rounding the bit patterns by hand.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2_t));
}

// 8 floats -> bf16 hi and lo parts (hi = bf16(x), lo = bf16(x - hi)),
// packed as two MFMA operand registers.
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    l[e] = pack_bf16x2(x[2 * e] - bf_lo(h[e]), x[2 * e + 1] - bf_hi(h[e]));
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

}  // namespace vs
