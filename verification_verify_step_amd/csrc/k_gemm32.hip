// Skinny GEMM over the wide matrices with v_mfma_f32_32x32x16_bf16 (gfx950)
// for passes of up to 8 rows: the chain verify (k+1 = 6 rows) and the draft's
// one-row passes (self-speculative decoding page, §1.1-§1.2: the pass streams
// every weight once).  The structure is the 16x16x32 skinny form's
// (k_gemm.hip):
//  * a workgroup owns one tile of 32 columns over the full K; its NW waves
//    split K into the matrix's NW chunks (gemm_k_chunks: 4 or 8) and reduce
//    through LDS in chunk order;
//  * per k-step a wave issues two MFMAs (the two 16-input halves in order)
//    from one weight fragment and one activation fragment each; A rows 0-15
//    carry the rows' hi parts and 16-31 their lo parts, rows past M are zero;
//  * the weight fragments stream PD k-steps ahead in a register ring with
//    non-temporal loads;
//  * RMSNorm scale, epilogue operands and the epilogues follow the 16x16x32
//    skinny form, with norm sums and argmax partials per 16 columns.
// A row's sums are grouped as in the 32x32 row-tiled form (k_gemm_tile32.hip):
// per chunk hi + lo, chunks in order, so the two forms give a row the same
// bits.
#pragma clang fp contract(off)
#include "gemm_dev.h"

namespace vs {

template <int NW, int PD, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm32_kernel(const GemmArgs a) {
  constexpr int NT = NW * 64, NC = 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int tile = blockIdx.x;  // 32-column tile
  const int M = a.M, m0 = a.m0, ld = a.ld, ks = a.k_steps;
  const int per = ks / NW;
  const int s0 = wave * per;

  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  const u32x4* wbase = reinterpret_cast<const u32x4*>(a.W) + (size_t)tile * ks * 128 + lane;
  const u32x4* xbase = reinterpret_cast<const u32x4*>(a.xa);
  // A row lane % 32: part (lane % 32) / 16, pass row lane % 16 (zero past M)
  const int part = (lane & 31) >> 4, arow = lane & 15;
  const bool row_ok = arow < M;
  const int row_ld = min(arow, M - 1);
  u32x4 wb[PD][2], xa[PD][2];
  auto load = [&](int p, int s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      wb[p][h] = __builtin_nontemporal_load(wbase + (size_t)s * 128 + h * 64);
      xa[p][h] = xbase[(size_t)((s * 2 + part) * 4 + 2 * h + (lane >> 5)) * ld + m0 + row_ld];
    }
  };
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto compute = [&](int p) {
    acc = mfma32(row_ok ? xa[p][0] : zero4, wb[p][0], acc);
    acc = mfma32(row_ok ? xa[p][1] : zero4, wb[p][1], acc);
  };

  // RMSNorm scale of the input rows from the producer's per-group sums of
  // squares, reduced in a fixed order through LDS: S_q = sum of groups
  // g = q mod 4 in increasing g, scale = norm_scale(S_0..S_3), the order every
  // form uses (loaded before the weight prologue, reduced while it is in
  // flight).
  constexpr int kSS = 2048;
  constexpr int RSS = kSS / NT;
  __shared__ float rs[kMaxRows];
  __shared__ float sstmp[kSS];
  const int n_ss = a.ss != nullptr ? a.ss_groups * M : 0;
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
  if (n_ss > kSS) {
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

  // epilogue operands, requested before the weight stream
  constexpr int EP = (8 * NC + NT - 1) / NT;
  constexpr int EQ = (8 * NC / 2 + NT - 1) / NT;
  float pre_h[EPI == EPI_RESID ? EP : 1], pre_g[EPI == EPI_RESID ? EP : 1];
  float2 pre_rope[EPI == EPI_QKV ? EQ : 1];
  int pre_kv[EPI == EPI_QKV ? EQ : 1];
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int j = 0; j < EP; ++j) {
      const int idx = min(tid + j * NT, M * NC - 1);
      const int m = idx / NC, nn = tile * NC + idx % NC;
      pre_h[j] = a.h[(size_t)(m0 + m) * a.d + nn];
      pre_g[j] = a.g_next[nn];
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int half = a.hd >> 1;
#pragma unroll
    for (int j = 0; j < EQ; ++j) {
      const int idx = min(tid + j * NT, M * (NC / 2) - 1);
      const int m = idx / (NC / 2), nn = tile * NC + 2 * (idx % (NC / 2));
      pre_rope[j] = a.rope[(size_t)(m0 + m) * half + ((nn % a.hd) >> 1)];
      pre_kv[j] = a.kvrow[m0 + m];
    }
  }

  // Software pipeline: PD k-steps of loads in flight ahead of the MFMAs
  // (unconditional, so that the loop's wait counts stay exact).
#pragma unroll
  for (int p = 0; p < PD; ++p) load(p, min(s0 + p, ks - 1));
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
  for (; i + 2 * PD <= per; i += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      compute(p);
      load(p, s0 + i + p + PD);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (; i < per; i += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      if (i + p < per) compute(p);
      if (i + p + PD < per) load(p, s0 + i + p + PD);
    }
  }

  // ---- cross-wave reduction through LDS, chunks (waves) in order ----
  // Element e of every lane of wave w is one row of RS floats, lanes
  // consecutive: the stores of a wave and the reads of 32 consecutive
  // columns each touch distinct banks, and the half-row padding puts the
  // next element's row (the next result row, read by the other half-wave)
  // on the other 32 banks.
  constexpr int RS = 96;
  __shared__ float red[NW * 16 * RS];
  __shared__ float rowtmp[8 * NC];
#pragma unroll
  for (int e = 0; e < 16; ++e) red[(wave * 16 + e) * RS + lane] = acc[e];
  __syncthreads();
  // row m (< 8), column c: hi at A row m, lo at A row m + 16, both in lane
  // c + 32 ((m / 4) % 2), elements 4 (m / 8) + m % 4 and that + 8
  auto result = [&](int m, int c) -> float {
    const int l = c + 32 * ((m >> 2) & 1), e = 4 * (m >> 3) + (m & 3);
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) y += red[(w * 16 + e) * RS + l] + red[(w * 16 + e + 8) * RS + l];
    return y;
  };

  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int j = 0; j < EP; ++j) {
      const int idx = tid + j * NT;
      if (idx < M * NC) {
        const int m = idx / NC, c = idx % NC;
        const int nn = tile * NC + c;
        const float hv = pre_h[j] + result(m, c);
        a.h[(size_t)(m0 + m) * a.d + nn] = hv;
        if (a.h_copy != nullptr) a.h_copy[(size_t)a.out_row[m] * a.d + nn] = hv;
        xa_store(a.xa_next, nn, m0 + m, ld, hv * pre_g[j]);
        rowtmp[m * NC + c] = hv * hv;
      }
    }
    __syncthreads();
    if (tid < 2 * M) {  // one sum per row and 16 columns, columns in increasing order
      const int m = tid >> 1, hf = tid & 1;
      float s = 0.f;
      for (int k = 0; k < 16; ++k) s += rowtmp[m * NC + 16 * hf + k];
      a.ss_out[(size_t)(2 * tile + hf) * ld + m0 + m] = s;
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int hd = a.hd, half = hd >> 1;
#pragma unroll
    for (int j = 0; j < EQ; ++j) {
      const int idx = tid + j * NT;
      if (idx < M * (NC / 2)) {
        const int m = idx / (NC / 2), pr = idx % (NC / 2);
        const int c = 2 * pr;
        const int nn = tile * NC + c;  // packed column: pair (i, i + hd/2) of one head
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
          const int dst = pre_kv[j];
          const size_t head = kv_tile(dst / kBlock, kvh, a.Hkv, hd);
          if (is_k) {
            uint16_t* kp = a.kv.k + head;
            kp[k_tile_off(dst % kBlock, ci)] = f2bf(o0);
            kp[k_tile_off(dst % kBlock, ci + half)] = f2bf(o1);
          } else {
            uint16_t* vp = a.kv.v + head + (dst % kBlock);
            vp[(size_t)ci * kBlock] = f2bf(o0);
            vp[(size_t)(ci + half) * kBlock] = f2bf(o1);
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int idx = tid; idx < M * (NC / 2); idx += NT) {
      const int m = idx / (NC / 2), pr = idx % (NC / 2);
      const int f = tile * (NC / 2) + pr;  // packed pair (gate f, up f)
      const float g = result(m, 2 * pr) * rs[m];
      const float u = result(m, 2 * pr + 1) * rs[m];
      xa_store(a.xa_act, f, m0 + m, ld, silu_mul(g, u));
    }
  } else {  // EPI_LOGITS
    for (int idx = tid; idx < M * NC; idx += NT) {
      const int m = idx / NC, c = idx % NC;
      const int nn = tile * NC + c;
      const float z = result(m, c) * rs[m];
      const int orow = a.out_row_identity ? m0 + m : a.out_row[m];
      if (a.logits != nullptr && orow >= 0) a.logits[(size_t)orow * a.V + nn] = z;
      rowtmp[m * NC + c] = z;
    }
    __syncthreads();
    if (tid < 2 * M) {  // argmax per row and 16 columns, lowest column on ties
      const int m = tid >> 1, hf = tid & 1;
      float best = rowtmp[m * NC + 16 * hf];
      int bi = 0;
      for (int k = 1; k < 16; ++k) {
        const float z = rowtmp[m * NC + 16 * hf + k];
        if (z > best) {
          best = z;
          bi = k;
        }
      }
      a.amax_val[(size_t)(2 * tile + hf) * ld + m0 + m] = best;
      a.amax_idx[(size_t)(2 * tile + hf) * ld + m0 + m] = tile * NC + 16 * hf + bi;
    }
  }
}

namespace {

template <int NW, int EPI>
void go32_nw(const GemmArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int PD = 4;  // 4 k-steps x 2 KB of weights in flight per wave
  const dim3 grid(a.n_tiles / 2);
  if (ev0 != nullptr || ev1 != nullptr)
    hipExtLaunchKernelGGL((gemm32_kernel<NW, PD, EPI>), grid, dim3(NW * 64), 0, st, ev0, ev1, 0, a);
  else
    hipLaunchKernelGGL((gemm32_kernel<NW, PD, EPI>), grid, dim3(NW * 64), 0, st, a);
}
template <int EPI>
void go32(const GemmArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (gemm_k_chunks(a.n_tiles) == 8) go32_nw<8, EPI>(a, st, ev0, ev1);
  else go32_nw<4, EPI>(a, st, ev0, ev1);
}

}  // namespace

int launch_gemm32(const GemmArgs& a, int epi, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  switch (epi) {
    case EPI_RESID: go32<EPI_RESID>(a, st, ev0, ev1); break;
    case EPI_QKV: go32<EPI_QKV>(a, st, ev0, ev1); break;
    case EPI_SWIGLU: go32<EPI_SWIGLU>(a, st, ev0, ev1); break;
    default: go32<EPI_LOGITS>(a, st, ev0, ev1); break;
  }
  return a.n_tiles;
}

}  // namespace vs
