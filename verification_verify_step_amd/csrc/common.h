// Internal types and device helpers of the verify-step library (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vstep.h"

namespace vs {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxSeq = VS_MAX_SEQS;
constexpr int kMaxRows = VS_MAX_ROWS;          // per sequence per pass; also per GEMM launch
constexpr int kMaxPassRows = VS_MAX_PASS_ROWS;  // per pass
constexpr int kBlock = 16;    // KV tokens per block
constexpr int kChunk = 64;    // keys per attention sub-chunk

// --------------------------------------------------------------------------
// Rows of one pass (passed by value to the kernels that place rows).
// Sequence i owns rows [row_start[i], row_start[i+1]); its row m has in-round
// index idx = idx_off + m - row_start[i], KV slot P + win + idx and position
// P + depth (depth = idx for a chain).  Visible keys: slots < P, plus slots
// P + win + j for every bit j of the row's mask.
struct RowMap {
  int n_seq;
  int M;
  int idx_off;
  int win;
  int seq[kMaxSeq];
  int row_start[kMaxSeq + 1];
  const int* depth;       // device [M] or null
  const uint64_t* mask;   // device [M] or null
};

struct KvView {
  uint16_t* k;            // layer pool [n_blocks][Hkv][hd/8][16][8] bf16 (kv_tile, k_tile_off)
  uint16_t* v;            // layer pool [n_blocks][Hkv][hd][16]
  const int* P;           // [max_seqs]
  const int* bt;          // [max_seqs][bps]
  int bps;
};

// Element offset of the (block, KV head) tile of kBlock keys x hd dims in a
// layer pool [n_blocks][Hkv][tile].
__device__ __forceinline__ size_t kv_tile(int blk, int kvh, int Hkv, int hd) {
  return ((size_t)blk * Hkv + kvh) * (size_t)(kBlock * hd);
}

// Offset of key slot j (0..15), dim d inside one (block, KV head) K tile:
// the dims are cut into 8-dim pieces and the tile is piece-major,
// [hd/8][16 keys][8 dims].  A wave's 16x16x32 MFMA operand for one k-step
// (16 keys x 4 pieces) is then 1 KiB of consecutive bytes, so each of its
// loads fills whole cache lines instead of half-lines of 16 key rows.
__device__ __forceinline__ size_t k_tile_off(int j, int d) {
  return (size_t)(d >> 3) * (kBlock * 8) + j * 8 + (d & 7);
}

// Fourth word of a raw buffer resource (__builtin_amdgcn_make_buffer_rsrc) on
// this GPU family: 32-bit data format, no swizzle, no index stride.  With
// stride 0 a load whose offset reaches the resource's byte extent returns
// zeros without a memory request; the kernels use that to bound their loads
// by a count known only at run time without branches.
constexpr int kRawBufferWord3 = 0x00020000;

// --------------------------------------------------------------------------
// bf16 helpers (bit patterns in uint16_t).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// The activation side of a GEMM is stored split into two bf16 parts
// (hi = bf16(x), lo = bf16(x - hi)) so that bf16 MFMA keeps ~16 bits of the
// fp32 activation.  Layout of a [M][K] activation: for k-step s = k/32, part
// p (0 = hi, 1 = lo), quad j = (k%32)/8, row m: 8 bf16 at
//   (((s*2 + p)*4 + j) * M + m) * 8.
// One k-step's hi parts are contiguous (then its lo parts), so the GEMM's
// 16-byte fragment loads of one part touch 4*M*16 contiguous bytes.
__device__ __forceinline__ size_t xa_index(int k, int m, int M, int part) {
  return ((size_t)(((k >> 5) * 2 + part) * 4 + ((k >> 3) & 3)) * M + m) * 8 + (k & 7);
}
__device__ __forceinline__ void xa_store(uint16_t* xa, int k, int m, int M, float v) {
  const uint16_t hi = f2bf(v);
  const uint16_t lo = f2bf(v - bf2f(hi));
  xa[xa_index(k, m, M, 0)] = hi;
  xa[xa_index(k, m, M, 1)] = lo;
}

// Row placement helpers for kernels that read a RowMap.
__device__ __forceinline__ int row_seq_index(const RowMap& rm, int m) {
  int i = 0;
  while (i + 1 < rm.n_seq && rm.row_start[i + 1] <= m) ++i;
  return i;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace vs
