// Small kernels of the round: weight packing, row loading (embedding or
// hidden rows), per-row vocabulary statistics, draft-token selection and
// sampling, acceptance, and commit / tree compaction (gfx950).
#include <climits>

#include "misc.h"

namespace vs {

// ---------------------------------------------------------------------------
// Weight packing: canonical row-major [rows][K] bf16 -> MFMA B fragments.
// Canonical row r lands on packed row p = row_off + map(r); fragment
// (tile, kstep) holds lane l = (p%16) + 16*j with k = 32*kstep + 8*j .. +8.
__global__ void pack_kernel(PackArgs a) {
  const size_t total = (size_t)a.rows * a.k_steps * 4;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int j = (int)(e % 4);
    const int s = (int)((e / 4) % a.k_steps);
    const int r = (int)(e / ((size_t)4 * a.k_steps));
    int p;
    if (a.map == PACK_HEADS) {  // pair (i, i + hd/2) of each head side by side
      const int h = r / a.hd, i = r % a.hd, half = a.hd / 2;
      p = h * a.hd + (i < half ? 2 * i : 2 * (i - half) + 1);
    } else if (a.map == PACK_EVEN) {
      p = 2 * r;
    } else if (a.map == PACK_ODD) {
      p = 2 * r + 1;
    } else {
      p = r;
    }
    p += a.row_off;
    size_t frag;  // 16-byte unit of (column p, inputs 32 s + 8 j .. +8)
    if (a.wide32)
      frag = ((((size_t)(p / 32) * a.k_steps + s) * 2 + (j >> 1)) * 64) + (p % 32) + 32 * (j & 1);
    else
      frag = ((size_t)(p / 16) * a.k_steps + s) * 64 + (p % 16) + 16 * j;
    const uint4 v = *reinterpret_cast<const uint4*>(a.src + (size_t)r * a.K + 32 * s + 8 * j);
    *reinterpret_cast<uint4*>(a.dst + frag * 8) = v;
  }
}

void launch_pack(const PackArgs& a, hipStream_t st) {
  const size_t total = (size_t)a.rows * a.k_steps * 4;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
}

__global__ void bf16_to_f32_kernel(const uint16_t* src, float* dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bf2f(src[i]);
}
void launch_bf16_to_f32(const uint16_t* src, float* dst, int n, hipStream_t st) {
  hipLaunchKernelGGL(bf16_to_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, src, dst, n);
}

__global__ void fill_i32_kernel(int* p, int v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}
void launch_fill_i32(int* p, int v, size_t n, hipStream_t st) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, v, n);
}

// Streaming read: workgroup b reads units [b*per, (b+1)*per) of the buffer,
// 8 16-byte loads per thread in flight per iteration; the XOR of everything
// it read goes to sink[b] so that no load is dropped.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  constexpr int kUnroll = 8;
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per, hi = lo + per < n16 ? lo + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = lo + threadIdx.x;
  for (; i + (kUnroll - 1) * 256 < hi; i += kUnroll * 256) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < hi; i += 256) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  x = wave_sum(x);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}
void launch_read_probe(const u32x4* src, size_t n16, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kReadProbeBlocks), dim3(256), 0, st, src, n16, sink);
}

__global__ void set_blocks_kernel(BlockSetArgs a) {
  const int i = threadIdx.x;
  if (i < a.n) a.bt[a.seq * a.bps + a.first + i] = a.ids[i];
  if (i == 0 && a.reset_state) {
    a.P[a.seq] = 0;
    a.pending[a.seq] = -1;
    a.committed[a.seq] = 0;
  }
}
void launch_set_blocks(const BlockSetArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(set_blocks_kernel, dim3(1), dim3(256), 0, st, a);
}

__global__ void set_state_kernel(int* P, int* pending, int* committed, int seq, int p, int pend) {
  P[seq] = p;
  pending[seq] = pend;
  committed[seq] = p + 1;
}
void launch_set_state(int* P, int* pending, int* committed, int seq, int p, int pend, hipStream_t st) {
  hipLaunchKernelGGL(set_state_kernel, dim3(1), dim3(1), 0, st, P, pending, committed, seq, p, pend);
}

// ---------------------------------------------------------------------------
// Row loading: h[m] = embed[token] (or a given hidden row); the next
// consumer's activation (h * g) as split-bf16 fragments; per 256-column group
// sums of h^2 for the fused RMSNorm.  One workgroup per (256-column group,
// row), so that no row waits on another's loads; the column group of row m
// adds its four wave sums in wave order.
__global__ __launch_bounds__(256) void load_rows_kernel(LoadArgs a) {
  const int bx = blockIdx.x, m = blockIdx.y;
  const int n = bx * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float wsum[4];
  float v = 0.f;
  if (n < a.d) {
    const int src = a.src_identity ? m : a.src_row[m % kMaxRows];
    if (a.tokens != nullptr) {
      const int t = min(max(a.tokens[src], 0), a.V - 1);  // never read outside the table
      v = bf2f(a.embed[(size_t)t * a.d + n]);
    } else {
      v = a.hidden[(size_t)src * a.d + n];
    }
    a.h[(size_t)m * a.d + n] = v;
    xa_store(a.xa, n, m, a.M, v * a.g[n]);
  }
  const float s = wave_sum(v * v);
  if (lane == 0) wsum[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) a.ss[(size_t)bx * a.M + m] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  if (a.rope != nullptr && bx == 0) {
    const int si = row_seq_index(a.rows, m);
    const int sq = a.rows.seq[si];
    const int idx = a.rows.idx_off + m - a.rows.row_start[si];
    const int pos = a.P[sq] + (a.rows.depth ? a.rows.depth[m] : idx);
    // angles in fp64: position up to ~1e4 times frequencies down to 1e-4
    for (int i = threadIdx.x; i < a.half; i += 256) {
      const double ang = (double)pos * pow((double)a.theta, -(double)i / (double)a.half);
      double sn, cs;
      sincos(ang, &sn, &cs);
      a.rope[(size_t)m * a.half + i] = make_float2((float)cs, (float)sn);
    }
    if (threadIdx.x == 0) {
      const int slot = a.P[sq] + a.rows.win + idx;
      a.kvrow[m] = a.bt[(size_t)sq * a.bps + slot / kBlock] * kBlock + slot % kBlock;
    }
  }
}
void launch_load_rows(const LoadArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(load_rows_kernel, dim3((a.d + 255) / 256, a.M), dim3(256), 0, st, a);
}

__global__ void copy_rows_kernel(const float* src, float* dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}
void launch_copy_rows(const float* src, float* dst, int M, int d, hipStream_t st) {
  const size_t n = (size_t)M * d;
  size_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, n);
}

// ---------------------------------------------------------------------------
// Workgroup reductions in a fixed order.
struct Top2 {
  float v1;
  int i1;
  float v2;
};
__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  Top2 r;
  if (a.v1 > b.v1 || (a.v1 == b.v1 && a.i1 < b.i1)) {
    r.v1 = a.v1;
    r.i1 = a.i1;
    r.v2 = fmaxf(a.v2, b.v1);
  } else {
    r.v1 = b.v1;
    r.i1 = b.i1;
    r.v2 = fmaxf(b.v2, a.v1);
  }
  return r;
}
// Row kernels: one 1024-thread workgroup per row, the row in registers
// (up to 32 values per thread, every load in flight at once).
constexpr int kStatsThreads = 1024;
constexpr int kStatsPer = 32;  // rows up to 32768 logits
// Workgroup top-2: butterfly over each wave with shuffles, then the wave
// results merged in wave order.  top2_merge is exact (max / min, no rounding)
// and its result does not depend on the merge order.
template <int NT>
__device__ Top2 block_top2_fast(Top2 t) {
  __shared__ Top2 sh[NT / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const Top2 u{__shfl_xor(t.v1, o, 64), __shfl_xor(t.i1, o, 64), __shfl_xor(t.v2, o, 64)};
    t = top2_merge(t, u);
  }
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = t;
  __syncthreads();
  Top2 r = sh[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = top2_merge(r, sh[w]);
  __syncthreads();
  return r;
}

// fp64 sum over a workgroup in a fixed order: lane 0 of each wave takes its
// wave's butterfly sum, then every thread adds the wave sums in wave order.
template <int NT>
__device__ double block_sum_fixed(double v, double* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) s += sh[w];
  __syncthreads();
  return s;
}

// Per-row statistics of logits: max, argmax (lowest id on ties), second
// largest value, and S = sum exp((z - max)/T) in fp64 when requested.  Thread
// t takes ids t, t + 1024, ..., so each load instruction of a wave reads 256
// contiguous bytes.
// Rows [0, M) of a, then rows [0, M) of b when b.logits is set (the
// target's and the draft's statistics of a stochastic accept in one launch).
__global__ __launch_bounds__(kStatsThreads) void row_stats_kernel(StatsArgs a0, StatsArgs b0, int M) {
  __shared__ double sh[kStatsThreads / 64];
  const bool second_set = (int)blockIdx.x >= M;
  const StatsArgs& a = second_set ? b0 : a0;
  const int m = second_set ? (int)blockIdx.x - M : (int)blockIdx.x;
  const float* z = a.logits + (size_t)m * a.V;
  float v[kStatsPer];
#pragma unroll
  for (int q = 0; q < kStatsPer; ++q) {
    const int j = q * kStatsThreads + (int)threadIdx.x;
    v[q] = j < a.V ? z[j] : -INFINITY;
  }
  Top2 t{-INFINITY, INT_MAX, -INFINITY};
#pragma unroll
  for (int q = 0; q < kStatsPer; ++q) {
    const int j = q * kStatsThreads + (int)threadIdx.x;
    if (j < a.V) t = top2_merge(t, Top2{v[q], j, -INFINITY});
  }
  t = block_top2_fast<kStatsThreads>(t);
  if (threadIdx.x == 0) {
    a.mx[m] = t.v1;
    a.amax[m] = t.i1;
    if (a.second) a.second[m] = t.v2;
  }
  if (a.sumexp != nullptr) {
    const double inv_t = 1.0 / (double)a.temp;
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < kStatsPer; ++q)
      if (q * kStatsThreads + (int)threadIdx.x < a.V) s += exp(((double)v[q] - (double)t.v1) * inv_t);
    s = block_sum_fixed<kStatsThreads>(s, sh);
    if (threadIdx.x == 0) a.sumexp[m] = s;
  }
}
void launch_row_stats(const StatsArgs& a, int M, hipStream_t st) {
  const StatsArgs none{};
  if (M > 0) hipLaunchKernelGGL(row_stats_kernel, dim3(M), dim3(kStatsThreads), 0, st, a, none, M);
}
void launch_row_stats2(const StatsArgs& a, const StatsArgs& b, int M, hipStream_t st) {
  if (M > 0) hipLaunchKernelGGL(row_stats_kernel, dim3(2 * M), dim3(kStatsThreads), 0, st, a, b, M);
}

// Order-preserving 32-bit image of a float: a > b as floats iff key(a) >
// key(b) as unsigned integers (for non-NaN values).
__device__ __forceinline__ unsigned ord_key(float z) {
  const unsigned u = __float_as_uint(z);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-p (nucleus) truncation of the target on the verify side ("self-
// speculative" page, §3.4: the draft keeps its full distribution, the verify
// truncates the target and renormalises on the kept set, then the ratio test
// runs on the full draft distribution).  Tokens are ordered by (logit desc,
// id asc), i.e. by probability; the kept set is the shortest prefix of that
// order whose probability reaches top_p.  One workgroup per row holds the row
// in registers.  A bisection over the 32-bit order keys finds the boundary
// key (the largest key whose tail mass still reaches top_p), a second one over
// the ids of the tokens tied at that key finds where the prefix ends among
// them; each step is one fixed-order fp64 sum over the row.
__global__ __launch_bounds__(kStatsThreads) void top_p_kernel(TopPArgs a) {
  __shared__ double sh[kStatsThreads / 64];
  const int m = blockIdx.x;
  const float* z = a.logits + (size_t)m * a.V;
  const double mx = a.mx[m], inv_t = 1.0 / (double)a.temp;
  auto id_of = [](int q) { return q * kStatsThreads + (int)threadIdx.x; };  // coalesced
  unsigned key[kStatsPer];
  double e[kStatsPer];
  double part = 0.0;
#pragma unroll
  for (int q = 0; q < kStatsPer; ++q) {
    const bool in = id_of(q) < a.V;
    const float zv = in ? z[id_of(q)] : -INFINITY;
    key[q] = in ? ord_key(zv) : 0u;
    e[q] = in ? exp(((double)zv - mx) * inv_t) : 0.0;
    part += e[q];
  }
  const double total = block_sum_fixed<kStatsThreads>(part, sh);
  const double thr = a.top_p * total;
  // largest key kappa with sum_{key >= kappa} e >= thr (kappa = 0 qualifies)
  uint64_t lo = 0, hi = 0xFFFFFFFFull;
  while (lo < hi) {
    const uint64_t mid = lo + (hi - lo + 1) / 2;
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < kStatsPer; ++q) s += key[q] >= (unsigned)mid ? e[q] : 0.0;
    if (block_sum_fixed<kStatsThreads>(s, sh) >= thr) lo = mid;
    else hi = mid - 1;
  }
  const unsigned kap = (unsigned)lo;
  double s_above = 0.0;
#pragma unroll
  for (int q = 0; q < kStatsPer; ++q) s_above += key[q] > kap ? e[q] : 0.0;
  const double above = block_sum_fixed<kStatsThreads>(s_above, sh);
  // smallest id iota with above + sum_{key == kappa, j <= iota} e >= thr
  int ilo = 0, ihi = a.V - 1;
  while (ilo < ihi) {
    const int mid = (ilo + ihi) / 2;
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < kStatsPer; ++q) s += (key[q] == kap && id_of(q) <= mid) ? e[q] : 0.0;
    if (above + block_sum_fixed<kStatsThreads>(s, sh) >= thr) ihi = mid;
    else ilo = mid + 1;
  }
  double s_tie = 0.0;
#pragma unroll
  for (int q = 0; q < kStatsPer; ++q) s_tie += (key[q] == kap && id_of(q) <= ilo) ? e[q] : 0.0;
  const double kept = above + block_sum_fixed<kStatsThreads>(s_tie, sh);
  if (threadIdx.x == 0) {
    a.key[m] = kap;
    a.id[m] = ilo;
    a.mass[m] = kept;
  }
}
void launch_top_p(const TopPArgs& a, int M, hipStream_t st) {
  if (M > 0) hipLaunchKernelGGL(top_p_kernel, dim3(M), dim3(kStatsThreads), 0, st, a);
}

// Inverse-CDF draw from weights w_j >= 0 (fp64), ids ascending: the smallest
// j with u*S < C_j, else the largest j with w_j > 0.  For 1024-thread
// workgroups with the weights already in registers, in the layout of
// sample_id(): wave w holds ids [2048 w, 2048 (w + 1)), lane l the 32
// consecutive ids 2048 w + 32 l + q.  C_j = (sum of earlier waves) + (sum of
// the wave's earlier lanes) + (the lane's own ids up to j), each in a fixed
// order: a lane adds its ids in order, one scan across the wave adds the lane
// sums, the wave sums are added in wave order.  Only ids with w_j > 0 are
// candidates: sums of the same weights grouped differently may differ in the
// last bit, so C_j can step up by a rounding error over a run of zero
// weights.  Returns -1 when every weight is zero; *total receives S.
__device__ __forceinline__ int sample_id(int q) {
  return (int)(threadIdx.x >> 6) * (64 * kStatsPer) + (int)(threadIdx.x & 63) * kStatsPer + q;
}
// This thread's kStatsPer logits of row z in the sample_id() layout, with
// 16-byte loads; ids at or past V read as `fill`.  V is a multiple of 16 (the
// entry points check it), so a load lies wholly inside or wholly past the row.
__device__ __forceinline__ void load_ids(const float* z, int V, float (&v)[kStatsPer], float fill) {
  const int j0 = sample_id(0);
#pragma unroll
  for (int c = 0; c < kStatsPer / 4; ++c) {
    float4 x = make_float4(fill, fill, fill, fill);
    if (j0 + 4 * c < V) x = *reinterpret_cast<const float4*>(z + j0 + 4 * c);
    v[4 * c] = x.x;
    v[4 * c + 1] = x.y;
    v[4 * c + 2] = x.z;
    v[4 * c + 3] = x.w;
  }
}
__device__ int block_sample_reg(double (&w)[kStatsPer], double u, double* total) {
  __shared__ double wsum[kStatsThreads / 64];
  __shared__ int s_pick, s_last;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int last = -1;
  unsigned pos = 0;  // bit q: w[q] > 0
#pragma unroll
  for (int q = 0; q < kStatsPer; ++q)
    if (w[q] > 0.0) {
      last = sample_id(q);
      pos |= 1u << q;
    }
  // w[q] <- the lane's ids 0..q added in order; then the lane sums scanned
  // across the wave (inclusive), and the lane's exclusive prefix
  double run = 0.0;
#pragma unroll
  for (int q = 0; q < kStatsPer; ++q) {
    run += w[q];
    w[q] = run;
  }
  double incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  double excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.0;
  const double wave_tot = __shfl(incl, 63, 64);
  if (lane == 0) wsum[wave] = wave_tot;
  if (t == 0) {
    s_pick = INT_MAX;
    s_last = -1;
  }
  __syncthreads();
  atomicMax(&s_last, last);
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int i = 0; i < kStatsThreads / 64; ++i) {
    if (i == wave) base = tot;
    tot += wsum[i];
  }
  const double target = u * tot;
  const double lb = base + excl;
#pragma unroll
  for (int q = 0; q < kStatsPer; ++q) {
    if (((pos >> q) & 1u) && target < lb + w[q]) {
      atomicMin(&s_pick, sample_id(q));
      break;
    }
  }
  __syncthreads();
  const int pick = s_pick == INT_MAX ? s_last : s_pick;
  __syncthreads();
  *total = tot;
  return tot > 0.0 ? pick : -1;
}

// ---------------------------------------------------------------------------
// Draft-token selection (one workgroup per sequence).
__global__ __launch_bounds__(kStatsThreads) void pick_kernel(PickArgs a) {
  const int i = blockIdx.x;
  int tok;
  if (a.src[i] < 0) {
    tok = a.pending[a.seq[i]];
  } else if (a.mode == VS_GREEDY) {
    Top2 t{-INFINITY, INT_MAX, -INFINITY};
    for (int g = threadIdx.x; g < a.groups; g += kStatsThreads) {
      const int e = g * a.Mprev + a.src[i];
      t = top2_merge(t, Top2{a.amax_val[e], a.amax_idx[e], -INFINITY});
    }
    t = block_top2_fast<kStatsThreads>(t);
    tok = t.i1;
  } else {
    // draw from softmax(z / T): the row in registers, its max, the weights
    // exp((z - max) / T) once, then the inverse-CDF draw
    const float* z = a.logits + (size_t)a.lrow[i] * a.V;
    float v[kStatsPer];
    load_ids(z, a.V, v, -INFINITY);
    Top2 t{-INFINITY, INT_MAX, -INFINITY};
#pragma unroll
    for (int q = 0; q < kStatsPer; ++q) {
      const int j = sample_id(q);
      if (j < a.V) t = top2_merge(t, Top2{v[q], j, -INFINITY});
    }
    t = block_top2_fast<kStatsThreads>(t);
    const double mx = t.v1, inv_t = 1.0 / (double)a.temp;
    double w[kStatsPer];
#pragma unroll
    for (int q = 0; q < kStatsPer; ++q) w[q] = sample_id(q) < a.V ? exp(((double)v[q] - mx) * inv_t) : 0.0;
    double tot;
    tok = block_sample_reg(w, a.u[(size_t)a.uidx[i] * VS_N_UNIFORMS + a.slot], &tot);
  }
  // Every written id lies in [0, V): with finite logits the draw and the
  // argmax always are; non-finite logits (an overflowed pass) would give -1
  // or INT_MAX, which later kernels use as indices.
  if (threadIdx.x == 0) a.tokens[a.dst[i]] = min(max(tok, 0), a.V - 1);
}
void launch_pick(const PickArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(pick_kernel, dim3(a.n), dim3(kStatsThreads), 0, st, a);
}

// ---------------------------------------------------------------------------
// Acceptance (one workgroup per sequence).
__device__ __forceinline__ int row_parent(const RowMap& rm, int r0, int c) {
  if (rm.mask == nullptr) return c - 1;
  const uint64_t anc = rm.mask[r0 + c] & ~(1ull << c);
  return anc == 0 ? -1 : 63 - __clzll((long long)anc);
}

__global__ __launch_bounds__(kStatsThreads) void accept_kernel(AcceptArgs a) {
  const int i = blockIdx.x;
  const int r0 = a.rows.row_start[i];
  const int nr = a.rows.row_start[i + 1] - r0;
  int* res = a.result + i * VS_RESULT_INTS;
  if (a.mode == VS_GREEDY) {
    if (threadIdx.x == 0) {
      int cur = 0, n_path = 0, flags = 0;
      int path[VS_RESULT_INTS - 4];
      while (true) {
        if (a.mx[r0 + cur] - a.second[r0 + cur] < 4e-2f) flags |= 1;
        const int t = a.amax[r0 + cur];
        int nxt = -1;
        for (int c = cur + 1; c < nr; ++c)
          if (row_parent(a.rows, r0, c) == cur && a.tokens[r0 + c] == t) {
            nxt = c;
            break;
          }
        if (nxt < 0 || n_path >= VS_RESULT_INTS - 4) break;
        path[n_path++] = nxt;
        cur = nxt;
      }
      res[0] = n_path;
      res[1] = min(max(a.amax[r0 + cur], 0), a.V - 1);  // in range also for non-finite logits
      res[2] = flags;
      res[3] = n_path;
      for (int j = 0; j < VS_RESULT_INTS - 4; ++j) res[4 + j] = j < n_path ? path[j] : -1;
    }
    return;
  }
  // Stochastic chain: rows r0 .. r0+k, row j judges token of row j+1.  With
  // top-p the target of row r is exp((z - max)/T) on its kept set over the
  // kept mass, and zero elsewhere.
  const int k = nr - 1;
  const double inv_t = 1.0 / (double)a.temp;
  const double* u = a.u + (size_t)i * VS_N_UNIFORMS;
  const bool tp = a.tp_key != nullptr;
  auto kept = [&](int r, int j, float zj) {
    if (!tp) return true;
    const unsigned kk = ord_key(zj);
    return kk > a.tp_key[r] || (kk == a.tp_key[r] && j <= a.tp_id[r]);
  };
  __shared__ int s_a, s_flags, s_reject;
  __shared__ double s_ratio[kMaxRows], s_u[kMaxRows];
  if ((int)threadIdx.x < k) {  // every row's p / q and uniform at once (their loads in flight together)
    const int j = threadIdx.x, r = r0 + j;
    s_u[j] = u[16 + j];
    const int d = min(max(a.tokens[r + 1], 0), a.V - 1);  // an index: kept in the row whatever the caller passed
    const float zd_t = a.logits[(size_t)r * a.V + d];
    const double p = kept(r, d, zd_t) ? exp(((double)zd_t - (double)a.mx[r]) * inv_t) / (tp ? a.tp_mass[r] : a.sumexp[r])
                                      : 0.0;
    const double q = exp(((double)a.dlogits[(size_t)r * a.V + d] - (double)a.dmx[r]) * inv_t) / a.dsumexp[r];
    s_ratio[j] = q > 0.0 ? p / q : 0.0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // the walk: accept row j's token while u_j < min(1, p / q)
    int acc = 0, flags = 0, reject = -1;
    for (int j = 0; j < k; ++j) {
      const double ratio = s_ratio[j];
      const double uj = s_u[j];
      if (fabs(ratio - uj) < 1e-3) flags |= 1;
      if (uj < fmin(1.0, ratio)) {
        ++acc;
        continue;
      }
      reject = j;
      break;
    }
    s_a = acc;
    s_flags = flags;
    s_reject = reject;
  }
  __syncthreads();
  const int reject = s_reject;
  int y;
  // weights of the draw in registers, in the layout of sample_id()
  double w[kStatsPer];
  double tot;
  auto target_weights = [&](int r) {  // exp((z - max)/T) on the (top-p) support
    float zt[kStatsPer];
    load_ids(a.logits + (size_t)r * a.V, a.V, zt, 0.f);
    const double mt = a.mx[r];
#pragma unroll
    for (int q = 0; q < kStatsPer; ++q) {
      const int j = sample_id(q);
      w[q] = (j < a.V && kept(r, j, zt[q])) ? exp(((double)zt[q] - mt) * inv_t) : 0.0;
    }
  };
  if (reject < 0) {
    target_weights(r0 + k);
    y = block_sample_reg(w, u[32], &tot);
  } else {
    const int r = r0 + reject;
    float zt[kStatsPer], zd[kStatsPer];
    load_ids(a.logits + (size_t)r * a.V, a.V, zt, 0.f);
    load_ids(a.dlogits + (size_t)r * a.V, a.V, zd, 0.f);
    const double mt = a.mx[r], md = a.dmx[r], st = tp ? a.tp_mass[r] : a.sumexp[r], sd = a.dsumexp[r];
#pragma unroll
    for (int q = 0; q < kStatsPer; ++q) {  // residual max(0, p - q)
      const int j = sample_id(q);
      if (j < a.V) {
        const double p = kept(r, j, zt[q]) ? exp(((double)zt[q] - mt) * inv_t) / st : 0.0;
        const double qd = exp(((double)zd[q] - md) * inv_t) / sd;
        w[q] = p > qd ? p - qd : 0.0;
      } else {
        w[q] = 0.0;
      }
    }
    y = block_sample_reg(w, u[32], &tot);
    if (y < 0) {  // the residual vanished: draw from p
      target_weights(r);
      y = block_sample_reg(w, u[32], &tot);
    }
  }
  if (threadIdx.x == 0) {
    res[0] = s_a;
    res[1] = min(max(y, 0), a.V - 1);  // -1 only if every weight vanished (non-finite logits)
    res[2] = s_flags;
    res[3] = s_a;
    for (int j = 0; j < VS_RESULT_INTS - 4; ++j) res[4 + j] = j < s_a ? j + 1 : -1;
  }
}
void launch_accept(const AcceptArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3(a.rows.n_seq), dim3(kStatsThreads), 0, st, a);
}

// ---------------------------------------------------------------------------
// Tree compaction: K/V of accepted path rows P + path[j] -> P + 1 + j in
// every layer (tiles kv_tile; K piece-major, k_tile_off; V columns [hd][16]).
// Sources increase along the path and never lie below their destination, so
// copying j in increasing order per element is safe.
__global__ void compact_kernel(CommitArgs a) {
  const int i = blockIdx.x;
  const int layer = blockIdx.y / 2, is_v = blockIdx.y % 2;
  const int* res = a.result + i * VS_RESULT_INTS;
  const int nr = a.rows.row_start[i + 1] - a.rows.row_start[i];
  const int n_path = min(max(res[3], 0), nr - 1);
  const int sq = a.rows.seq[i];
  const int P = a.P[sq];
  uint16_t* pool = is_v ? a.vpool[layer] : a.kpool[layer];
  for (int e = threadIdx.x; e < a.Hkv * a.hd; e += blockDim.x) {  // one (kv head, dim) per thread
    const int kvh = e / a.hd, d = e % a.hd;
    for (int j = 0; j < n_path; ++j) {
      const int r = res[4 + j];
      if (r < 1 || r >= nr) break;  // a path row outside this sequence's rows
      const int src = P + r, dst = P + 1 + j;
      if (src == dst) continue;
      const size_t bs = kv_tile(a.bt[sq * a.bps + src / kBlock], kvh, a.Hkv, a.hd);
      const size_t bd = kv_tile(a.bt[sq * a.bps + dst / kBlock], kvh, a.Hkv, a.hd);
      if (is_v)
        pool[bd + (size_t)d * kBlock + dst % kBlock] = pool[bs + (size_t)d * kBlock + src % kBlock];
      else
        pool[bd + k_tile_off(dst % kBlock, d)] = pool[bs + k_tile_off(src % kBlock, d)];
    }
  }
}
void launch_compact(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(a.rows.n_seq, 2 * a.n_layers), dim3(256), 0, st, a);
}

__global__ void commit_kernel(CommitArgs a) {
  const int i = threadIdx.x;
  if (i >= a.rows.n_seq) return;
  const int* res = a.result + i * VS_RESULT_INTS;
  const int sq = a.rows.seq[i];
  // at most the sequence's rows minus one are accepted: the host's bound on
  // the KV length (and so every later table lookup) relies on it
  const int acc = min(max(res[0], 0), a.rows.row_start[i + 1] - a.rows.row_start[i] - 1);
  const int P = a.P[sq] + acc + 1;
  a.P[sq] = P;
  a.pending[sq] = res[1];
  a.committed[sq] += acc + 1;
  if (a.mirror != nullptr)
    __hip_atomic_store(a.mirror + sq, ((uint64_t)a.commit_no[i] << 32) | (uint32_t)P, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
}
void launch_commit(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(64), 0, st, a);
}

// One thread per sequence; its rows are averaged in row order in fp64
// ("DSpark" page, §2.2: the mean top-1 probability and the mean top-1 minus
// top-2 gap over the verify block).
__global__ void confidence_kernel(ConfArgs a) {
  const int i = threadIdx.x;
  if (i >= a.rows.n_seq) return;
  const int r0 = a.rows.row_start[i], r1 = a.rows.row_start[i + 1];
  const double inv_t = 1.0 / (double)a.temp;
  double s1 = 0.0, sg = 0.0;
  for (int r = r0; r < r1; ++r) {
    const double p1 = 1.0 / a.sumexp[r];
    const double p2 = exp(((double)a.second[r] - (double)a.mx[r]) * inv_t) / a.sumexp[r];
    s1 += p1;
    sg += p1 - p2;
  }
  const double n = (double)max(1, r1 - r0);
  a.conf[2 * i] = s1 / n;
  a.conf[2 * i + 1] = sg / n;
}
void launch_confidence(const ConfArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(confidence_kernel, dim3(1), dim3(kMaxSeq), 0, st, a);
}

__global__ void advance_kernel(int* P, int* committed, int seq, int dP, int dC) {
  if (threadIdx.x == 0) {
    P[seq] += dP;
    committed[seq] += dC;
  }
}
void launch_advance(int* P, int* committed, int seq, int dP, int dC, hipStream_t st) {
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, st, P, committed, seq, dP, dC);
}

}  // namespace vs
