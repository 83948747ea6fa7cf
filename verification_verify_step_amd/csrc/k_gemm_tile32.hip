// Row-tiled GEMM over the wide matrices with v_mfma_f32_32x32x16_bf16
// (gfx950): passes of more than 8 rows (self-speculative decoding page,
// §1.1-§1.2: one weight read serves every position of the round; a tree or a
// batch of rounds multiplies the rows).  The structure is the 16x16x32
// row-tiled form's (k_gemm_tile.hip), with 32-column tiles:
//  * a workgroup of 4 waves owns a block of BM = 16*MW rows and 4*NWT tiles of
//    32 columns; each k-step's activation fragments of the block (hi and lo
//    parts, 8*BM 16-byte units) are staged once in LDS and read by all four
//    waves, each wave streams its own tiles' weight fragments (2 per tile and
//    k-step) into a register ring PD = 8 k-steps deep;
//  * the k-steps run in supersteps of 4 with one workgroup barrier each: the
//    next superstep's activations are written during the current one into
//    the other half of eight LDS buffers;
//  * per k-step a wave issues 2*MW*NWT MFMAs: for each m-tile and tile, the
//    two 16-input halves in order, A rows 0-15 carrying the rows' hi parts and
//    16-31 their lo parts, so hi and lo accumulate apart in one accumulator;
//  * a workgroup runs all K chunks of its tiles (gemm_k_chunks, each a
//    multiple of 8 k-steps), adding each chunk's hi + lo to the running sum
//    in chunk order -- the skinny 32x32 form's grouping (k_gemm32.hip) -- so
//    a row's bits do not depend on the rows beside it or on the form;
//  * the row blocks of one n-range run back to back on one XCD (workgroup
//    index mod 8), so the second and later blocks read the weights from that
//    XCD's L2;
//  * norm sums and argmax partials are written per 16 columns, as by every
//    form.
#pragma clang fp contract(off)
#include "gemm_dev.h"

namespace vs {

namespace {

constexpr int kT32Threads = 256;  // 4 waves

template <int CTRL>
__device__ __forceinline__ float dpp32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp32(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
// (value, column) maximum over the 16 lanes of a DPP row (16 consecutive
// columns of a tile), lowest column on ties: an exact, order-free merge.
template <int CTRL>
__device__ __forceinline__ void amax_step32(float& v, int& i) {
  const float ov = dpp32<CTRL>(v);
  const int oi = dpp32<CTRL>(i);
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

}  // namespace

template <int MW, int NWT, int PD, int EPI>
__global__ __launch_bounds__(kT32Threads) void gemm_tile32_kernel(const GemmArgs a, const int n_chunks,
                                                                  const int n_mblk, const int n_grp) {
  static_assert(PD == 8, "ring slots and LDS buffers rotate together: 8 buffers, supersteps of 4");
  constexpr int NT = kT32Threads, BM = 16 * MW, UA = 8 * BM, UPT = (UA + NT - 1) / NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // workgroup -> (row block, n-range): XCD = index mod 8, the row blocks of
  // an n-range consecutive on it; padding workgroups return
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
  const int mb = pos % n_mblk, grp = (pos / n_mblk) * 8 + xcd;
  if (grp >= n_grp) return;
  const int M = a.M, m0 = a.m0, ld = a.ld, ks = a.k_steps;
  const int per = ks / n_chunks;
  const int mrow0 = mb * BM, Mb = min(BM, M - mrow0);
  const int n32 = a.n_tiles / 2;                 // 32-column tiles
  const int tile0 = (grp * 4 + wave) * NWT;

  __shared__ u32x4 As[8][UPT * NT];  // [k-step & 7][part*4 + quad][row], then unused padding
  __shared__ float rs[BM];

  const u32x4* wbase[NWT];
#pragma unroll
  for (int t = 0; t < NWT; ++t)
    wbase[t] = reinterpret_cast<const u32x4*>(a.W) + (size_t)min(tile0 + t, n32 - 1) * ks * 128 + lane;
  const u32x4* xbase = reinterpret_cast<const u32x4*>(a.xa);
  // this thread's activation units: u = tid + i*NT -> (part*4 + quad, row);
  // rows past the block repeat its last row (never stored), units past UA
  // land in the padding
  size_t aoff[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = min(tid + i * NT, UA - 1), r = u % BM, pq = u / BM;
    aoff[i] = (size_t)pq * ld + m0 + mrow0 + min(r, Mb - 1);
  }

  u32x4 wb[PD][NWT][2], ar[PD][UPT];
  auto load = [&](int p, int j) {  // ring slot p <- k-step j (clamped)
    const int s = min(j, ks - 1);
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      wb[p][t][0] = wbase[t][(size_t)s * 128];
      wb[p][t][1] = wbase[t][(size_t)s * 128 + 64];
    }
#pragma unroll
    for (int i = 0; i < UPT; ++i) ar[p][i] = xbase[(size_t)s * 8 * ld + aoff[i]];
  };
  auto put = [&](int p, int buf) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) As[buf][tid + i * NT] = ar[p][i];
  };
  // A operands of one k-step (m-tile, half), double-buffered by parity
  u32x4 af[2][MW][2];
  auto fetch = [&](int q, int buf) {
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) af[q][mt][h] = As[buf][a32_unit(lane, h) * BM + mt * 16 + (lane & 15)];
  };

  f32x16 acc[MW][NWT];
  float y[MW][NWT][8];
#pragma unroll
  for (int mt = 0; mt < MW; ++mt)
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mt][t][e] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[mt][t][e] = 0.f;
    }
  auto compute = [&](int q, int p) {
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int t = 0; t < NWT; ++t) {
        acc[mt][t] = mfma32(af[q][mt][0], wb[p][t][0], acc[mt][t]);
        acc[mt][t] = mfma32(af[q][mt][1], wb[p][t][1], acc[mt][t]);
      }
  };
  // end of a K chunk: its sum (hi + lo) joins the running sum in chunk order
  auto close_chunk = [&]() {
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int t = 0; t < NWT; ++t) {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[mt][t][e] += acc[mt][t][e] + acc[mt][t][e + 8];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mt][t][e] = 0.f;
      }
  };

  // operand prologue (PD k-steps)
#pragma unroll
  for (int p = 0; p < PD; ++p) load(p, p);

  // RMSNorm scales of the block's rows (row_scale_kernel ran just before)
  for (int r = tid; r < BM; r += NT) rs[r] = a.rs != nullptr ? a.rs[m0 + mrow0 + min(r, Mb - 1)] : 1.0f;

  // Main loop over k-steps j, in unrolled groups of 8 (chunks close between
  // groups), as supersteps of 4.  A(j) sits in LDS buffer j & 7, written
  // during the previous superstep (from ring slot j % 8, loaded 4 steps
  // before that).  Step j reads A(j) first if it opens a superstep and A(j +
  // 1) if the superstep goes on, runs its MFMAs, stores A(j + 4) into buffer
  // (j + 4) & 7 (last read during the previous superstep) and refills its
  // ring slot with k-step j + 8; the superstep's last step meets the
  // workgroup at the barrier.
#pragma unroll
  for (int p = 0; p < 4; ++p) put(p, p);
  __syncthreads();
  auto step = [&](int p, int j0) {
    const int i = p & 3;  // place in the superstep (j0 is a multiple of 8)
    if (i == 0) fetch(p & 1, p & 7);
    if (i < 3) fetch((p + 1) & 1, (p + 1) & 7);
    compute(p & 1, p);
    put((p + 4) & 7, (p + 4) & 7);
    load(p, j0 + p + PD);
    if (i == 3) __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int j0 = 0; j0 + 8 <= ks; j0 += 8) {
#pragma unroll
    for (int p = 0; p < 8; ++p) step(p, j0);
    if ((j0 + 8) % per == 0) close_chunk();
  }
  __syncthreads();  // the epilogues reuse the operand buffers

  // ---- epilogues.  Element e < 8 of a lane's accumulator of m-tile mt is
  // block row mt*16 + 8 (e / 4) + 4 (lane / 32) + e % 4, column lane % 32 of
  // the tile.  Every load an epilogue needs is issued before its first store;
  // neighbouring columns are exchanged with DPP.
  const int c = lane & 31;
  int lrow[MW][8];
  bool mok[MW][8];
  float rsv[MW][8];
#pragma unroll
  for (int mt = 0; mt < MW; ++mt)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int lr = mt * 16 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      lrow[mt][e] = lr;
      mok[mt][e] = mrow0 + lr < M;
      rsv[mt][e] = rs[lr];
    }
  auto mrow_c = [&](int mt, int e) { return min(mrow0 + lrow[mt][e], M - 1); };  // launch-relative row, clamped
  if constexpr (EPI == EPI_RESID) {
    float hv[NWT][MW][8], gv[NWT];
    int crow[MW][8];
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int nn = min(tile0 + t, n32 - 1) * 32 + c;
      gv[t] = a.g_next[nn];
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[t][mt][e] = a.h[(size_t)(m0 + mrow_c(mt, e)) * a.d + nn];
    }
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int e = 0; e < 8; ++e) crow[mt][e] = a.h_copy != nullptr ? a.out_row[mrow_c(mt, e)] : 0;
    float* sqt = reinterpret_cast<float*>(&As[0][0]) + wave * BM * 32;  // [BM][32] squares per wave
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int tile = tile0 + t;
      const bool tok = tile < n32;
      const int nn = min(tile, n32 - 1) * 32 + c;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = mrow0 + lrow[mt][e];
          const float v = hv[t][mt][e] + y[mt][t][e];
          if (tok && mok[mt][e]) {
            a.h[(size_t)(m0 + m) * a.d + nn] = v;
            if (a.h_copy != nullptr) a.h_copy[(size_t)crow[mt][e] * a.d + nn] = v;
            xa_store(a.xa_next, nn, m0 + m, ld, v * gv[t]);
          }
          sqt[lrow[mt][e] * 32 + c] = v * v;
        }
      __syncthreads();
      // one sum per row and 16 columns, columns in increasing order
      for (int u = lane; u < 2 * BM; u += 64) {
        const int lr = u >> 1, hf = u & 1, m = mrow0 + lr;
        if (tok && m < M) {
          float sum = 0.f;
#pragma unroll
          for (int k = 0; k < 16; ++k) sum += sqt[lr * 32 + 16 * hf + k];
          a.ss_out[(size_t)(2 * tile + hf) * ld + m0 + m] = sum;
        }
      }
      __syncthreads();
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int hd = a.hd, half = hd >> 1;
    const bool odd = c & 1;
    float2 rp[NWT][MW][8];
    int kvr[MW][8];
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int nn = min(tile0 + t, n32 - 1) * 32 + c;  // packed: pair (i, i + hd/2) at columns (2j, 2j + 1)
      const int ci = (nn % hd) >> 1;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int e = 0; e < 8; ++e) rp[t][mt][e] = a.rope[(size_t)(m0 + mrow_c(mt, e)) * half + ci];
    }
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int e = 0; e < 8; ++e) kvr[mt][e] = a.kvrow[m0 + mrow_c(mt, e)];
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int tile = tile0 + t;
      const bool tok = tile < n32;
      const int nn = min(tile, n32 - 1) * 32 + c;
      const int hb = nn / hd, ci = (nn % hd) >> 1;
      const bool rot = hb < a.H + a.Hkv;
      const int el = odd ? ci + half : ci;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = mrow_c(mt, e);
          const float own = y[mt][t][e] * rsv[mt][e];
          const float other = dpp32<0xB1>(own);  // lanes 2j <-> 2j + 1: columns 2j <-> 2j + 1, same row
          const float y0 = odd ? other : own, y1 = odd ? own : other;
          if (!(tok && mok[mt][e])) continue;
          float o = odd ? y1 : y0;
          if (rot) o = odd ? rope_second(y0, y1, rp[t][mt][e]) : rope_first(y0, y1, rp[t][mt][e]);
          if (hb < a.H) {
            a.q[((size_t)(m0 + m) * a.H + hb) * hd + el] = o;
          } else {
            const bool is_k = rot;
            const int kvh = is_k ? hb - a.H : hb - a.H - a.Hkv;
            const int dst = kvr[mt][e];
            const size_t head = kv_tile(dst / kBlock, kvh, a.Hkv, hd);
            if (is_k)
              a.kv.k[head + k_tile_off(dst % kBlock, el)] = f2bf(o);
            else
              a.kv.v[head + (size_t)el * kBlock + dst % kBlock] = f2bf(o);
          }
        }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int tile = tile0 + t;
      const bool tok = tile < n32;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float own = y[mt][t][e] * rsv[mt][e];
          const float up = dpp32<0xB1>(own);  // packed: (gate f, up f) at columns (2j, 2j + 1)
          if (tok && mok[mt][e] && !(c & 1))
            xa_store(a.xa_act, tile * 16 + (c >> 1), m0 + mrow0 + lrow[mt][e], ld, silu_mul(own, up));
        }
    }
  } else {  // EPI_LOGITS
    int orow[MW][8];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int e = 0; e < 8; ++e) orow[mt][e] = a.out_row_identity ? m0 + mrow_c(mt, e) : a.out_row[mrow_c(mt, e)];
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int tile = tile0 + t;
      const bool tok = tile < n32;
      const int nn = tile * 32 + c;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = mrow0 + lrow[mt][e];
          const bool ok = tok && mok[mt][e];
          const float z = y[mt][t][e] * rsv[mt][e];
          if (ok && a.logits != nullptr && orow[mt][e] >= 0) a.logits[(size_t)orow[mt][e] * a.V + nn] = z;
          // argmax over the 16 columns of this lane's DPP row, lowest column on ties
          float bv = z;
          int bi = nn;
          amax_step32<0xB1>(bv, bi);   // quad_perm [1, 0, 3, 2]
          amax_step32<0x4E>(bv, bi);   // quad_perm [2, 3, 0, 1]
          amax_step32<0x141>(bv, bi);  // row_half_mirror
          amax_step32<0x140>(bv, bi);  // row_mirror
          if (ok && (lane & 15) == 0) {
            const int g = 2 * tile + ((lane >> 4) & 1);
            a.amax_val[(size_t)g * ld + m0 + m] = bv;
            a.amax_idx[(size_t)g * ld + m0 + m] = bi;
          }
        }
    }
  }
}

namespace {

struct Ev32 {
  hipEvent_t a, b;
};

template <int EPI, int MW, int NWT>
void go_tile32(const GemmArgs& a, int n_mblk, hipStream_t st, Ev32 ev) {
  constexpr int PD = 8;  // with supersteps; 4 at the 70B batch's shapes was slower (gate/up 722 against 670 us)
  const int n32 = a.n_tiles / 2;
  const int n_grp = (n32 + 4 * NWT - 1) / (4 * NWT);
  const int nc = gemm_k_chunks(a.n_tiles);
  const dim3 grid(8 * n_mblk * ((n_grp + 7) / 8));
  GemmArgs g = a;
  hipEvent_t start = ev.a;
  if (a.ss != nullptr) {
    launch_row_scale(a, st, start);
    start = nullptr;
    g.rs = a.rs_buf;
  }
  if (start != nullptr || ev.b != nullptr)
    hipExtLaunchKernelGGL((gemm_tile32_kernel<MW, NWT, PD, EPI>), grid, dim3(kT32Threads), 0, st, start, ev.b, 0, g,
                          nc, n_mblk, n_grp);
  else
    hipLaunchKernelGGL((gemm_tile32_kernel<MW, NWT, PD, EPI>), grid, dim3(kT32Threads), 0, st, g, nc, n_mblk, n_grp);
}

template <int EPI, int MW>
void go32_ntw(const GemmArgs& a, int n_mblk, int ntw, hipStream_t st, Ev32 ev) {
  if (ntw == 2) go_tile32<EPI, MW, 2>(a, n_mblk, st, ev);
  else go_tile32<EPI, MW, 1>(a, n_mblk, st, ev);
}

template <int EPI>
void go32_epi(const GemmArgs& a, const TileShape& sh, hipStream_t st, Ev32 ev) {
  switch (sh.mw) {
    case 1: go32_ntw<EPI, 1>(a, sh.n_mblk, sh.ntw, st, ev); break;
    case 2: go32_ntw<EPI, 2>(a, sh.n_mblk, sh.ntw, st, ev); break;
    case 4: go32_ntw<EPI, 4>(a, sh.n_mblk, sh.ntw, st, ev); break;
    default: go32_ntw<EPI, 3>(a, sh.n_mblk, sh.ntw, st, ev); break;
  }
}

}  // namespace

// Shape of a wide matrix's row-tiled launch: tiles of 32 columns, ntw of them
// per wave (1 or 2), row blocks of 16*mw rows.
TileShape gemm_tile32_shape(int n_tiles, int M, int ntw) {
  TileShape sh;
  const int mt = (M + 15) / 16;
  const int n32 = n_tiles / 2;
  sh.split = false;
  sh.mw = mt <= 4 ? std::min(mt, 2) : 3;
  sh.n_mblk = (mt + sh.mw - 1) / sh.mw;
  if (ntw == 1 || ntw == 2) {
    sh.ntw = ntw;
  } else {
    // the wider tile where the grid still holds >= 200 workgroups
    sh.ntw = (n32 + 7) / 8 * sh.n_mblk >= 200 ? 2 : 1;
    // the widest matrices (>= 1024 n-tiles of 16 columns) at 33 to 64 rows:
    // one row block of all rows, one tile per wave
    if (mt >= 3 && mt <= 4 && n_tiles >= 1024) {
      sh.mw = mt;
      sh.n_mblk = 1;
      sh.ntw = 1;
    }
  }
  return sh;
}

int launch_gemm_tile32(const GemmArgs& a, int epi, int ntw, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const Ev32 ev{ev0, ev1};
  const TileShape sh = gemm_tile32_shape(a.n_tiles, a.M, ntw);
  switch (epi) {
    case EPI_RESID: go32_epi<EPI_RESID>(a, sh, st, ev); break;
    case EPI_QKV: go32_epi<EPI_QKV>(a, sh, st, ev); break;
    case EPI_SWIGLU: go32_epi<EPI_SWIGLU>(a, sh, st, ev); break;
    default: go32_epi<EPI_LOGITS>(a, sh, st, ev); break;
  }
  return a.n_tiles;
}

}  // namespace vs
