// Device pieces shared by the two GEMM forms (k_gemm.hip, k_gemm_tile.hip).
//
// A row's outputs must carry the same bits whichever form computes them and
// whichever rows share its pass (greedy verify equals plain decoding token
// for token only if a row's logits do not depend on its neighbours).  Both
// forms therefore use one MFMA shape with one K order, one grouping of the
// partial sums, and the arithmetic below; both files are compiled with
// floating-point contraction off, so no multiply-add is fused differently in
// one form than in the other.
#pragma once
#include "kernels.h"

namespace vs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Number of K chunks whose partial sums a column adds in chunk order: a
// property of the matrix alone (4 for the wide matrices, >= 512 n-tiles,
// else 8), never of the rows in the pass.
__host__ __device__ __forceinline__ int gemm_k_chunks(int n_tiles) { return n_tiles >= 512 ? 4 : 8; }
// The narrow matrices (< 512 n-tiles: too few n-ranges to fill the chip)
// run the row-tiled form with K split over workgroups, one K chunk each, at
// up to 64 rows when a chunk is long enough (>= 32 k-steps) to pay for the
// combine; their chunk sums are added in chunk order by the last workgroup
// of a tile.  Measured at 40 and 64 rows: the 7B down projection (43
// k-steps per chunk) gains a quarter to a third; O (16) and the tiny model
// (1) lose, and keep the skinny form.
__host__ __device__ __forceinline__ bool gemm_tile_split(int n_tiles, int k_steps, int M) {
  return n_tiles < 512 && M <= 64 && k_steps % gemm_k_chunks(n_tiles) == 0 && k_steps / gemm_k_chunks(n_tiles) >= 32;
}
// Whether the row-tiled form takes the product: the wide matrices with equal
// K chunks of a multiple of 8 k-steps, the narrow ones with K split.
__host__ __device__ __forceinline__ bool gemm_tile_fits(int n_tiles, int k_steps, int M) {
  if (n_tiles < 512) return gemm_tile_split(n_tiles, k_steps, M);
  return k_steps % (gemm_k_chunks(n_tiles) * 8) == 0;
}

// The widest matrices (>= 1024 n-tiles of 16 columns, an even count, K
// chunks that fit the row-tiled form: gate/up and the head at the 7B and 70B
// shapes) use v_mfma_f32_32x32x16_bf16 in both forms.  On gfx950 it issues
// about twice the flops per second of the 16x16x32 instruction (2.1-2.4
// against 0.9-1.5 PFLOP/s in a register-only loop at one to eight waves per
// SIMD) and gets twice the flops out of each activation fragment.  One
// instruction takes the hi parts of 16 rows (A rows 0-15) and their lo parts
// (A rows 16-31) against 32 columns over 16 inputs; a matrix's rows see the
// same instruction, K order and partial-sum grouping in every form.  The
// other matrices keep the 16x16x32 forms: with 32-column tiles the 7B QKV
// (768 n-tiles) has 384 skinny workgroups for 256 CUs and measured 1.6 us
// slower at 6 rows.
__host__ __device__ __forceinline__ bool gemm_wide32(int n_tiles, int k_steps) {
  return n_tiles >= 1024 && n_tiles % 2 == 0 && k_steps % (gemm_k_chunks(n_tiles) * 8) == 0;
}
// 32x32x16 lane layout (checked on the device): lane l holds A[l % 32][8 (l /
// 32) .. +8] and B[8 (l / 32) .. +8][l % 32]; result element e of lane l is
// D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32].  Packed weights of a wide matrix:
// fragment (32-column tile T, k-step s, half h) = 64 lanes x 16 bytes, lane l
// holding W[32 T + l % 32][32 s + 16 h + 8 (l / 32) .. +8], at
// ((T * k_steps + s) * 2 + h) * 64 + l.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
// Activation unit (part * 4 + quad) of half h read by lane l for A rows l % 32:
// rows 0-15 the hi parts, 16-31 the lo parts of the m-tile's 16 rows.
__device__ __forceinline__ int a32_unit(int lane, int h) { return ((lane & 31) >> 4) * 4 + 2 * h + (lane >> 5); }

// RMSNorm scale from the four strided partial sums S_q (q = group mod 4).
__device__ __forceinline__ float norm_scale(float s0, float s1, float s2, float s3, float inv_d, float eps) {
  const float t = (s0 + s1) + (s2 + s3);
  return 1.0f / sqrtf(t * inv_d + eps);
}

// RoPE rotation of the pair (y0, y1) = (x_i, x_{i + hd/2}) by (cos, sin).
__device__ __forceinline__ float rope_first(float y0, float y1, float2 r) { return y0 * r.x - y1 * r.y; }
__device__ __forceinline__ float rope_second(float y0, float y1, float2 r) { return y1 * r.x + y0 * r.y; }

// SwiGLU: silu(g) * u.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace vs
