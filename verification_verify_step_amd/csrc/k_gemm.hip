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
//  * Passes of more than 8 rows run the row-tiled form in k_gemm_tile.hip
//    where its K chunks fit (every wide matrix; narrow ones with long K
//    chunks), which keeps every row's arithmetic identical.
#pragma clang fp contract(off)
#include "gemm_dev.h"

namespace vs {

// MT = 0 is the packed form for M <= 8: one 16-row A operand holds the hi
// parts of the rows in A rows 0-7 and their lo parts in rows 8-15, so a
// k-step takes one activation load and one MFMA; output rows m and m + 8 are
// added per wave.  With MT >= 1 tiles the hi and lo parts accumulate
// separately and are added per wave the same way, so a row's sum is grouped
// identically whichever form computes it.
template <int MT, int NTW, int NW, int PD, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(const GemmArgs a) {
  constexpr bool PK = MT == 0;
  constexpr int T = PK ? 1 : MT;  // 16-row tiles
  constexpr int TL = PK ? 1 : MT;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tile0 = blockIdx.x * NTW;
  const int M = a.M, m0 = a.m0, ld = a.ld;
  const int per = (a.k_steps + NW - 1) / NW;
  const int s0 = min(wave * per, a.k_steps);
  const int s1 = min(s0 + per, a.k_steps);
  const int n = s1 - s0;
  const int mrow = lane & 15, kq = lane >> 4;

  f32x4 acc[T][NTW], acl[TL][NTW];  // hi (packed: hi and lo) and lo accumulators
#pragma unroll
  for (int mt = 0; mt < T; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < TL; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acl[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4* wbase[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
    wbase[t] = reinterpret_cast<const u32x4*>(a.W) + (size_t)(tile0 + t) * a.k_steps * 64 + lane;
  const u32x4* xbase = reinterpret_cast<const u32x4*>(a.xa);

  u32x4 wb[PD][NTW];
  u32x4 xh[PD][T], xl[PD][TL];

  // Rows >= M are loaded from row M-1 (no divergent branch, so the loads stay
  // in flight across iterations) and zeroed by a select before the MFMA.
  bool row_ok[T];
  int row_ld[T];
  const int part = PK ? (mrow >> 3) : 0;  // packed: A rows 8-15 carry the lo parts
#pragma unroll
  for (int mt = 0; mt < T; ++mt) {
    const int m = PK ? (mrow & 7) : mt * 16 + mrow;
    row_ok[mt] = m < M;
    row_ld[mt] = min(m, M - 1);
  }
  auto load = [&](int p, int s) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) wb[p][t] = __builtin_nontemporal_load(wbase[t] + (size_t)s * 64);
#pragma unroll
    for (int mt = 0; mt < T; ++mt) {
      if constexpr (PK) {
        xh[p][mt] = xbase[(size_t)((s * 2 + part) * 4 + kq) * ld + m0 + row_ld[mt]];
      } else {
        xh[p][mt] = xbase[(size_t)((s * 2) * 4 + kq) * ld + m0 + row_ld[mt]];
        xl[p][mt] = xbase[(size_t)((s * 2 + 1) * 4 + kq) * ld + m0 + row_ld[mt]];
      }
    }
  };
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto compute = [&](int p) {
#pragma unroll
    for (int mt = 0; mt < T; ++mt) {
      const u32x4 ah = row_ok[mt] ? xh[p][mt] : zero4;
      if constexpr (PK) {
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[mt][t] = mfma(ah, wb[p][t], acc[mt][t]);
      } else {
        const u32x4 al = row_ok[mt] ? xl[p][mt] : zero4;
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          acc[mt][t] = mfma(ah, wb[p][t], acc[mt][t]);
          acl[mt][t] = mfma(al, wb[p][t], acl[mt][t]);
        }
      }
    }
  };

  // RMSNorm scale of the input rows from the producer's per-group sums of
  // squares: loaded before the weight prologue (so waiting for them leaves the
  // weight loads in flight) and reduced in a fixed order through LDS.
  constexpr int NT = NW * 64;
  constexpr int kSS = 2048;             // sums held by the fast path
  constexpr int RSS = kSS / NT;
  __shared__ float rs[kMaxRows];
  __shared__ float sstmp[kSS];
  const int tid = threadIdx.x;
  const int n_ss = a.ss != nullptr ? a.ss_groups * M : 0;
  // Row m's sum is (S_0 + S_1) + (S_2 + S_3) with S_q = sum of groups g = q mod 4
  // in increasing g: the order does not depend on M, so a row's scale (and
  // everything after it) is the same whichever rows share the pass.
  constexpr int kQ = 4;
  auto first_level = [&](auto val) {
    float s = 0.f;
    if (tid < kQ * M) {
      const int m = tid % M;
      for (int g = tid / M; g < a.ss_groups; g += kQ) s += val(g, m);
    }
    return s;
  };
  auto finish_rs = [&]() {
    __syncthreads();
    if (tid < M) rs[tid] = norm_scale(sstmp[tid], sstmp[M + tid], sstmp[2 * M + tid], sstmp[3 * M + tid], a.inv_d, a.eps);
  };
  if (n_ss > kSS) {  // many sums (large M): reduce straight from memory, before the weight stream starts
    const float s = first_level([&](int g, int m) { return a.ss[(size_t)g * ld + m0 + m]; });
    sstmp[tid] = s;
    finish_rs();
  } else if (n_ss == 0 && tid < M) {
    rs[tid] = 1.0f;
  }
  float ssv[RSS];
#pragma unroll
  for (int j = 0; j < RSS; ++j) {
    const int e = tid + j * NT;
    ssv[j] = (n_ss <= kSS && e < n_ss) ? a.ss[(size_t)(e / M) * ld + m0 + e % M] : 0.f;
  }

  // Operands of the epilogue that do not depend on the product are requested
  // now, so the epilogue waits on no memory: residual rows and the next
  // norm's gains (residual), RoPE pairs and KV destinations (QKV).  Indexes
  // are clamped to valid entries; entries past M * NC are never used.
  constexpr int NC = NTW * 16;
  constexpr int EP = (kMaxRows * NC + NT - 1) / NT;
  constexpr int EQ = (kMaxRows * NC / 2 + NT - 1) / NT;
  float pre_h[EPI == EPI_RESID ? EP : 1], pre_g[EPI == EPI_RESID ? EP : 1];
  float2 pre_rope[EPI == EPI_QKV ? EQ : 1];
  int pre_kv[EPI == EPI_QKV ? EQ : 1];
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int j = 0; j < EP; ++j) {
      const int idx = min(tid + j * NT, M * NC - 1);
      const int m = idx / NC, nn = tile0 * 16 + idx % NC;
      pre_h[j] = a.h[(size_t)(m0 + m) * a.d + nn];
      pre_g[j] = a.g_next[nn];
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int half = a.hd >> 1;
#pragma unroll
    for (int j = 0; j < EQ; ++j) {
      const int idx = min(tid + j * NT, M * (NC / 2) - 1);
      const int m = idx / (NC / 2), nn = tile0 * 16 + 2 * (idx % (NC / 2));
      pre_rope[j] = a.rope[(size_t)(m0 + m) * half + ((nn % a.hd) >> 1)];
      pre_kv[j] = a.kvrow[m0 + m];
    }
  }

  // Software pipeline: PD k-steps of loads in flight ahead of the MFMAs.
  // (unconditional, clamped to a valid k-step: a branch here would make the
  // loop's wait counts conservative)
#pragma unroll
  for (int p = 0; p < PD; ++p) load(p, max(0, min(s0 + p, a.k_steps - 1)));
  // the norm scale is reduced while the first weight loads are in flight
  if (n_ss > 0 && n_ss <= kSS) {
#pragma unroll
    for (int j = 0; j < RSS; ++j) sstmp[tid + j * NT] = ssv[j];
    __syncthreads();
    const float s = first_level([&](int g, int m) { return sstmp[g * M + m]; });
    __syncthreads();
    sstmp[tid] = s;
    finish_rs();
  }
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
  __shared__ float red[NW * NTW * T * 256];
  __shared__ float rowtmp[kMaxRows * NTW * 16];
#pragma unroll
  for (int mt = 0; mt < T; ++mt)
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[(((wave * NTW + t) * T + mt) * 64 + lane) * 4 + r] =
            PK ? acc[mt][t][r] : acc[mt][t][r] + acl[PK ? 0 : mt][t][r];
  __syncthreads();

  auto result = [&](int m, int c) -> float {
    const int t = c >> 4, col = c & 15, mt = PK ? 0 : m >> 4, row = PK ? m : m & 15;
    const int src = ((row >> 2) * 16 + col) * 4 + (row & 3);
    float y = 0.f;
    if constexpr (PK) {  // per wave: hi (row m) + lo (row m + 8), then over waves
      const int src_lo = (((row + 8) >> 2) * 16 + col) * 4 + ((row + 8) & 3);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float* tile = red + ((w * NTW + t) * T + mt) * 256;
        y += tile[src] + tile[src_lo];
      }
    } else {
#pragma unroll
      for (int w = 0; w < NW; ++w) y += red[((w * NTW + t) * T + mt) * 256 + src];
    }
    return y;
  };

  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int j = 0; j < EP; ++j) {
      const int idx = tid + j * NT;
      if (idx < M * NC) {
        const int m = idx / NC, c = idx % NC;
        const int nn = tile0 * 16 + c;
        const float hv = pre_h[j] + result(m, c);
        a.h[(size_t)(m0 + m) * a.d + nn] = hv;
        if (a.h_copy != nullptr) a.h_copy[(size_t)a.out_row[m] * a.d + nn] = hv;
        xa_store(a.xa_next, nn, m0 + m, ld, hv * pre_g[j]);
        rowtmp[m * NC + c] = hv * hv;
      }
    }
    __syncthreads();
    if (tid < M) {
      float s = 0.f;
      for (int c = 0; c < NC; ++c) s += rowtmp[tid * NC + c];
      a.ss_out[(size_t)blockIdx.x * ld + m0 + tid] = s;
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int hd = a.hd, half = hd >> 1;
#pragma unroll
    for (int j = 0; j < EQ; ++j) {
      const int idx = tid + j * NT;
      if (idx < M * (NC / 2)) {
        const int m = idx / (NC / 2), pr = idx % (NC / 2);
        const int c = 2 * pr;
        const int nn = tile0 * 16 + c;  // packed column: pair (i, i + hd/2) of one head
        const float y0 = result(m, c) * rs[m];
        const float y1 = result(m, c + 1) * rs[m];
        const int hb = nn / hd;
        const int ci = (nn % hd) >> 1;
        float o0 = y0, o1 = y1;
        if (hb < a.H + a.Hkv) {
          o0 = rope_first(y0, y1, pre_rope[j]);
          o1 = rope_second(y0, y1, pre_rope[j]);
        }
        if (hb < a.H) {
          float* qo = a.q + ((size_t)(m0 + m) * a.H + hb) * hd;
          qo[ci] = o0;
          qo[ci + half] = o1;
        } else {
          const bool is_k = hb < a.H + a.Hkv;
          const int kvh = is_k ? hb - a.H : hb - a.H - a.Hkv;
          const int dst = pre_kv[j];  // block * 16 + offset in the block
          const size_t head = kv_tile(dst / kBlock, kvh, a.Hkv, hd);
          if (is_k) {  // K tile: piece-major (k_tile_off)
            uint16_t* kp = a.kv.k + head;
            kp[k_tile_off(dst % kBlock, ci)] = f2bf(o0);
            kp[k_tile_off(dst % kBlock, ci + half)] = f2bf(o1);
          } else {     // V columns: [hd][16 keys]
            uint16_t* vp = a.kv.v + head + (dst % kBlock);
            vp[(size_t)ci * kBlock] = f2bf(o0);
            vp[(size_t)(ci + half) * kBlock] = f2bf(o1);
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int idx = tid; idx < M * (NC / 2); idx += NW * 64) {
      const int m = idx / (NC / 2), pr = idx % (NC / 2);
      const int f = (tile0 * 16) / 2 + pr;  // packed pair (gate f, up f)
      const float g = result(m, 2 * pr) * rs[m];
      const float u = result(m, 2 * pr + 1) * rs[m];
      const float act = silu_mul(g, u);
      xa_store(a.xa_act, f, m0 + m, ld, act);
    }
  } else {  // EPI_LOGITS
    for (int idx = tid; idx < M * NC; idx += NW * 64) {
      const int m = idx / NC, c = idx % NC;
      const int nn = tile0 * 16 + c;
      const float z = result(m, c) * rs[m];
      const int orow = a.out_row_identity ? m0 + m : a.out_row[m];
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
      a.amax_val[(size_t)blockIdx.x * ld + m0 + tid] = best;
      a.amax_idx[(size_t)blockIdx.x * ld + m0 + tid] = tile0 * 16 + bi;
    }
  }
}

GemmCfg gemm_cfg(int id) {
  static const GemmCfg t[kGemmCfgs] = {{0, 0}, {1, 4}, {1, 8}, {2, 4}, {2, 8}};
  return t[(id > 0 && id < kGemmCfgs) ? id : 0];
}

// The number of waves splitting K fixes the order of every column's sum, so
// it depends on the matrix only, never on M: a row's result is then the same
// whichever rows share its pass.  Measured on MI355X (7B shapes): 4 waves for
// the wide matrices (>= 512 n-tiles: QKV, gate/up, head, and every 70B
// matrix), two n-tiles per workgroup above 16 rows (half the activation
// traffic per weight byte); 8 waves and one n-tile for the narrow ones
// (O and down at d = 4096), at every M.
int gemm_pick(int n_tiles, int k_steps, int M) {
  (void)k_steps;
  if (n_tiles < 512) return 2;                    // (1,8)
  return (M > 16 && n_tiles % 2 == 0) ? 3 : 1;    // (2,4) / (1,4)
}

struct Ev {
  hipEvent_t a, b;
};

template <int EPI, int MT, int NTW, int NW>
static void go(const GemmArgs& a, hipStream_t st, Ev ev) {
  // Ring depth per shape, measured: at up to 8 rows (MT 0) one 16-column
  // tile per workgroup streams best 6 k-steps ahead with 4 waves (QKV: 19.2
  // -> 18.9 us at the 7B shape) and 8 ahead with 8 waves (O, down); at 33-64
  // rows (MT 3-4: O at 40 and 64 rows) 2 ahead (19.8 -> 19.2 us at 64 rows;
  // 6 and 8 spill).
  constexpr int PD = MT >= 3 ? 2 : (NTW == 2 ? 4 : (MT == 0 && NW == 4 ? 6 : 8));
  if (ev.a != nullptr || ev.b != nullptr)
    hipExtLaunchKernelGGL((gemm_kernel<MT, NTW, NW, PD, EPI>), dim3(a.n_tiles / NTW), dim3(NW * 64), 0, st, ev.a,
                          ev.b, 0, a);
  else
    hipLaunchKernelGGL((gemm_kernel<MT, NTW, NW, PD, EPI>), dim3(a.n_tiles / NTW), dim3(NW * 64), 0, st, a);
}

template <int EPI, int MT>
static void launch_mt(const GemmArgs& a, int cfg, hipStream_t st, Ev ev) {
  switch (cfg) {
    case 1: go<EPI, MT, 1, 4>(a, st, ev); break;
    case 2: go<EPI, MT, 1, 8>(a, st, ev); break;
    case 3: go<EPI, MT, 2, 4>(a, st, ev); break;
    default: go<EPI, MT, 2, 8>(a, st, ev); break;
  }
}

template <int EPI>
static void launch_epi(const GemmArgs& a, int cfg, hipStream_t st, Ev ev) {
  const int mt = (a.M + 15) / 16;
  if (a.M <= 8) launch_mt<EPI, 0>(a, cfg, st, ev);
  else if (mt == 1) launch_mt<EPI, 1>(a, cfg, st, ev);
  else if (mt == 2) launch_mt<EPI, 2>(a, cfg, st, ev);
  else if (mt == 3) launch_mt<EPI, 3>(a, cfg, st, ev);
  else launch_mt<EPI, 4>(a, cfg, st, ev);
}

bool gemm_uses_tile(int n_tiles, int k_steps, int M, int cfg) {
  if (M <= 8 || !gemm_tile_fits(n_tiles, k_steps, M)) return false;
  return cfg >= kGemmCfgTile || cfg == 0;
}

int launch_gemm(const GemmArgs& a, int epi, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  // the wide matrices: the 32x32x16 forms (skinny up to 8 rows, else row-tiled)
  if (gemm_wide32(a.n_tiles, a.k_steps)) {
    if (a.M <= 8) return launch_gemm32(a, epi, st, ev0, ev1);
    return launch_gemm_tile32(a, epi, a.cfg >= kGemmCfgTile ? a.cfg - kGemmCfgTile : 0, st, ev0, ev1);
  }
  if (gemm_uses_tile(a.n_tiles, a.k_steps, a.M, a.cfg)) return launch_gemm_tile(a, epi, a.cfg - kGemmCfgTile, st, ev0, ev1);
  const Ev ev{ev0, ev1};
  int cfg = (a.cfg > 0 && a.cfg < kGemmCfgs) ? a.cfg : gemm_pick(a.n_tiles, a.k_steps, a.M);
  if (gemm_cfg(cfg).ntw == 2 && a.n_tiles % 2 != 0) cfg -= 2;  // same waves, one n-tile
  // configurations whose reduction buffer would not fit fall back inside launch_mt
  int ntw = gemm_cfg(cfg).ntw;
  switch (epi) {
    case EPI_RESID: launch_epi<EPI_RESID>(a, cfg, st, ev); break;
    case EPI_QKV: launch_epi<EPI_QKV>(a, cfg, st, ev); break;
    case EPI_SWIGLU: launch_epi<EPI_SWIGLU>(a, cfg, st, ev); break;
    default: launch_epi<EPI_LOGITS>(a, cfg, st, ev); break;
  }
  return a.n_tiles / ntw;
}

}  // namespace vs
