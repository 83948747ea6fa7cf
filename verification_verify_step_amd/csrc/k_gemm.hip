// Skinny-M weight-streaming GEMM for the verify step (gfx950, bf16 MFMA).
//
// A decode-time pass multiplies a handful of rows (k+1 = 6 at the 7B chain
// workload) by every weight matrix once; the pass is bound by streaming the
// weights from HBM (self-speculative decoding page, m.lqnn.cn/news/278124,
// §1.1-§1.2: one weight read serves all k+1 positions).  Design:
//  * Weights are packed once into v_mfma_f32_16x16x32_bf16 B-operand order:
//    fragment (n-tile t, k-step s) = 64 lanes x 16 bytes, lane l holding
//    W[16t + l%16][32s + 8(l/16) .. +8].  A wave's 16-byte non-temporal load
//    reads one contiguous kilobyte; a weight byte is read exactly once.
//  * The activations arrive pre-split into bf16 hi + lo parts (written by the
//    producing kernel), so two MFMAs per weight fragment keep ~16 mantissa
//    bits of the fp32 activation while the weights stay bf16.
//  * A workgroup owns NTW n-tiles over the full K; its NW waves split K and
//    reduce through LDS in a fixed order (deterministic, no atomics).
//  * RMSNorm is fused: the producer wrote x*g and per-group sums of x^2; the
//    1/rms scale is applied to the outputs here.  Epilogues: residual add,
//    q/k RoPE + KV-cache append, SwiGLU, logits + argmax partials.
#include "kernels.h"

namespace vs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

template <int MT, int NTW, int NW, int PD, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(const GemmArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tile0 = blockIdx.x * NTW;
  const int M = a.M;
  const int per = (a.k_steps + NW - 1) / NW;
  const int s0 = min(wave * per, a.k_steps);
  const int s1 = min(s0 + per, a.k_steps);
  const int n = s1 - s0;
  const int mrow = lane & 15, kq = lane >> 4;

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4* wbase[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
    wbase[t] = reinterpret_cast<const u32x4*>(a.W) + (size_t)(tile0 + t) * a.k_steps * 64 + lane;
  const u32x4* xbase = reinterpret_cast<const u32x4*>(a.xa);

  u32x4 wb[PD][NTW];
  u32x4 xh[PD][MT], xl[PD][MT];

  // Rows >= M are loaded from row M-1 (no divergent branch, so the loads stay
  // in flight across iterations) and zeroed by a select before the MFMA.
  bool row_ok[MT];
  int row_ld[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + mrow;
    row_ok[mt] = m < M;
    row_ld[mt] = min(m, M - 1);
  }
  auto load = [&](int p, int s) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) wb[p][t] = __builtin_nontemporal_load(wbase[t] + (size_t)s * 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4* px = xbase + ((size_t)(s * 4 + kq) * M + row_ld[mt]) * 2;
      xh[p][mt] = px[0];
      xl[p][mt] = px[1];
    }
  };
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto compute = [&](int p) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 ah = row_ok[mt] ? xh[p][mt] : zero4;
      const u32x4 al = row_ok[mt] ? xl[p][mt] : zero4;
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        acc[mt][t] = mfma(ah, wb[p][t], acc[mt][t]);
        acc[mt][t] = mfma(al, wb[p][t], acc[mt][t]);
      }
    }
  };

  // Software pipeline: PD k-steps of loads in flight ahead of the MFMAs.
  // (unconditional, clamped to a valid k-step: a branch here would make the
  // loop's wait counts conservative)
#pragma unroll
  for (int p = 0; p < PD; ++p) load(p, max(0, min(s0 + p, a.k_steps - 1)));
  int i = 0;
  for (; i + 2 * PD <= n; i += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      // keep "consume stage p, refill stage p" in this order so that each MFMA
      // waits only for its own stage's loads
      compute(p);
      load(p, s0 + i + p + PD);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (; i < n; i += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      if (i + p < n) compute(p);
      if (i + p + PD < n) load(p, s0 + i + p + PD);
    }
  }

  // ---- cross-wave reduction through LDS (fixed order) ----
  __shared__ float red[NW * NTW * MT * 256];
  __shared__ float rs[kMaxRows];
  __shared__ float rowtmp[kMaxRows * NTW * 16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(((wave * NTW + t) * MT + mt) * 64 + lane) * 4 + r] = acc[mt][t][r];

  const int tid = threadIdx.x;
  if (tid < M) {
    float scale = 1.0f;
    if (a.ss != nullptr) {
      float s = 0.f;
      for (int g = 0; g < a.ss_groups; ++g) s += a.ss[g * M + tid];
      scale = 1.0f / sqrtf(s * a.inv_d + a.eps);
    }
    rs[tid] = scale;
  }
  __syncthreads();

  auto result = [&](int m, int c) -> float {
    const int t = c >> 4, col = c & 15, mt = m >> 4, row = m & 15;
    const int src = ((row >> 2) * 16 + col) * 4 + (row & 3);
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) y += red[((w * NTW + t) * MT + mt) * 256 + src];
    return y;
  };
  constexpr int NC = NTW * 16;

  if constexpr (EPI == EPI_RESID) {
    for (int idx = tid; idx < M * NC; idx += NW * 64) {
      const int m = idx / NC, c = idx % NC;
      const int nn = tile0 * 16 + c;
      const float hv = a.h[(size_t)m * a.d + nn] + result(m, c);
      a.h[(size_t)m * a.d + nn] = hv;
      if (a.h_copy != nullptr) a.h_copy[(size_t)a.out_row[m] * a.d + nn] = hv;
      xa_store(a.xa_next, nn, m, M, hv * a.g_next[nn]);
      rowtmp[m * NC + c] = hv * hv;
    }
    __syncthreads();
    if (tid < M) {
      float s = 0.f;
      for (int c = 0; c < NC; ++c) s += rowtmp[tid * NC + c];
      a.ss_out[blockIdx.x * M + tid] = s;
    }
  } else if constexpr (EPI == EPI_QKV) {
    __shared__ int s_pos[kMaxRows], s_slot[kMaxRows], s_seq[kMaxRows];
    if (tid < M) {
      const int i = row_seq_index(a.rows, tid);
      const int sq = a.rows.seq[i];
      const int idx = a.rows.idx_off + tid - a.rows.row_start[i];
      const int depth = a.rows.depth ? a.rows.depth[tid] : idx;
      const int P = a.kv.P[sq];
      s_seq[tid] = sq;
      s_slot[tid] = P + a.rows.win + idx;
      s_pos[tid] = P + depth;
    }
    __syncthreads();
    const int hd = a.hd, half = hd >> 1;
    for (int idx = tid; idx < M * (NC / 2); idx += NW * 64) {
      const int m = idx / (NC / 2), pr = idx % (NC / 2);
      const int c = 2 * pr;
      const int nn = tile0 * 16 + c;  // packed column: pair (i, i + hd/2) of one head
      const float y0 = result(m, c) * rs[m];
      const float y1 = result(m, c + 1) * rs[m];
      const int hb = nn / hd;
      const int ci = (nn % hd) >> 1;
      float o0 = y0, o1 = y1;
      if (hb < a.H + a.Hkv) {
        const double inv_freq = pow((double)a.theta, -2.0 * (double)ci / (double)hd);
        const double ang = (double)s_pos[m] * inv_freq;
        double sn, cs;
        sincos(ang, &sn, &cs);
        o0 = (float)((double)y0 * cs - (double)y1 * sn);
        o1 = (float)((double)y1 * cs + (double)y0 * sn);
      }
      if (hb < a.H) {
        float* qo = a.q + ((size_t)m * a.H + hb) * hd;
        qo[ci] = o0;
        qo[ci + half] = o1;
      } else {
        const bool is_k = hb < a.H + a.Hkv;
        const int kvh = is_k ? hb - a.H : hb - a.H - a.Hkv;
        const int slot = s_slot[m];
        const int blk = a.kv.bt[s_seq[m] * a.kv.bps + slot / kBlock];
        uint16_t* dst = (is_k ? a.kv.k : a.kv.v) + (((size_t)blk * a.Hkv + kvh) * kBlock + (slot % kBlock)) * hd;
        dst[ci] = f2bf(o0);
        dst[ci + half] = f2bf(o1);
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int idx = tid; idx < M * (NC / 2); idx += NW * 64) {
      const int m = idx / (NC / 2), pr = idx % (NC / 2);
      const int f = (tile0 * 16) / 2 + pr;  // packed pair (gate f, up f)
      const float g = result(m, 2 * pr) * rs[m];
      const float u = result(m, 2 * pr + 1) * rs[m];
      const float act = g / (1.0f + expf(-g)) * u;
      xa_store(a.xa_act, f, m, M, act);
    }
  } else {  // EPI_LOGITS
    for (int idx = tid; idx < M * NC; idx += NW * 64) {
      const int m = idx / NC, c = idx % NC;
      const int nn = tile0 * 16 + c;
      const float z = result(m, c) * rs[m];
      const int orow = a.out_row_identity ? m : a.out_row[m];
      if (a.logits != nullptr && orow >= 0) a.logits[(size_t)orow * a.V + nn] = z;
      rowtmp[m * NC + c] = z;
    }
    __syncthreads();
    if (tid < M) {
      float best = rowtmp[tid * NC];
      int bi = 0;
      for (int c = 1; c < NC; ++c) {
        const float z = rowtmp[tid * NC + c];
        if (z > best) {
          best = z;
          bi = c;
        }
      }
      a.amax_val[blockIdx.x * M + tid] = best;
      a.amax_idx[blockIdx.x * M + tid] = tile0 * 16 + bi;
    }
  }
}

int gemm_groups(int n_tiles) {
  return (n_tiles % 2 == 0 && n_tiles / 2 >= 384) ? n_tiles / 2 : n_tiles;
}

template <int EPI>
static void launch_epi(const GemmArgs& a, hipStream_t st, int groups) {
  const int mt = (a.M + 15) / 16;
  const bool wide = groups * 2 == a.n_tiles;
  dim3 grid(groups);
#define VS_GEMM(MT, NTW, NW, PD) hipLaunchKernelGGL((gemm_kernel<MT, NTW, NW, PD, EPI>), grid, dim3(NW * 64), 0, st, a)
  if (wide) {
    if (mt == 1) VS_GEMM(1, 2, 4, 4);
    else if (mt == 2) VS_GEMM(2, 2, 4, 4);
    else VS_GEMM(4, 2, 4, 2);
  } else {
    if (mt == 1) VS_GEMM(1, 1, 8, 8);
    else if (mt == 2) VS_GEMM(2, 1, 8, 4);
    else VS_GEMM(4, 1, 8, 4);
  }
#undef VS_GEMM
}

int launch_gemm(const GemmArgs& a, int epi, hipStream_t st) {
  const int groups = gemm_groups(a.n_tiles);
  switch (epi) {
    case EPI_RESID: launch_epi<EPI_RESID>(a, st, groups); break;
    case EPI_QKV: launch_epi<EPI_QKV>(a, st, groups); break;
    case EPI_SWIGLU: launch_epi<EPI_SWIGLU>(a, st, groups); break;
    default: launch_epi<EPI_LOGITS>(a, st, groups); break;
  }
  return groups;
}

}  // namespace vs
