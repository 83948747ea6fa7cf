// Row-tiled GEMM for verify passes of more than 8 rows (gfx950, bf16 MFMA).
//
// A tree or a batch of chains puts tens to hundreds of rows through each
// weight matrix; the 70B ragged batch puts 327 (self-speculative decoding
// page, §1.1-§1.2: one weight read serves every position of the round, and a
// batch of rounds multiplies the rows).  The skinny form re-reads the
// activations from L2 in every wave, which caps it far below the weight
// stream at these sizes.  Here:
//  * A workgroup of 4 waves owns a block of BM = 16*MW rows (MW = 1, 2 or 3)
//    and 4*NWT n-tiles.  Each k-step's activation fragments of the block (hi
//    and lo parts, 8*BM 16-byte units) are staged once in LDS and read by
//    all four waves; each wave streams the packed weight fragments of its
//    own NWT n-tiles straight into registers.
//  * Per k-step a wave issues 2*MW*NWT MFMAs from 2*MW LDS fragments and
//    NWT weight fragments.  Global loads run PD k-steps ahead (a register
//    ring for both operands); the staged activations rotate through four
//    LDS buffers, and the A operands of the next k-step are read from LDS
//    during the current one.  A workgroup runs all K chunks (equal, a
//    multiple of 8 k-steps), or, for the narrow matrices, one chunk with K
//    split over workgroups (gemm_tile_fits).
//  * Rows stay bit-identical to the skinny form: the same 16x16x32 MFMA over
//    the same k-steps in increasing order, hi and lo accumulated apart and
//    added at the end of each K chunk (the chunks the skinny form gives to
//    its waves), the chunk sums added in chunk order; the same norm sums,
//    the same epilogue arithmetic and the same 16-column groups for the
//    norm and argmax partials.
//  * The row blocks of one n-range are launched back to back on one XCD, so
//    the second and later blocks find the weights in that XCD's L2.
#pragma clang fp contract(off)
#include "gemm_dev.h"

namespace vs {

namespace {

constexpr int kTileThreads = 256;  // 4 waves
constexpr int kScaleRows = 64;     // rows per row_scale_kernel workgroup
constexpr int kScaleBatch = 32;    // norm-sum loads in flight per thread

}  // namespace

// Lane exchanges inside a row of 16 lanes through DPP (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float dpp_swap1(float v) { return dpp<0xB1>(v); }  // lanes 2j <-> 2j + 1
// (value, column) maximum over the 16 lanes of a row, lowest column on ties:
// swap neighbours, pairs, then mirror halves of 8 and of 16 (a butterfly
// whose merge is exact and order-free).
template <int CTRL>
__device__ __forceinline__ void amax_step(float& v, int& i) {
  const float ov = dpp<CTRL>(v);
  const int oi = dpp<CTRL>(i);
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}
__device__ __forceinline__ void argmax16(float& v, int& i) {
  amax_step<0xB1>(v, i);   // quad_perm [1, 0, 3, 2]
  amax_step<0x4E>(v, i);   // quad_perm [2, 3, 0, 1]
  amax_step<0x141>(v, i);  // row_half_mirror
  amax_step<0x140>(v, i);  // row_mirror
}

// RMSNorm scale of each row of a pass, once per GEMM instead of once per
// workgroup: S_q = sum of the producer's 16-column partial sums over groups
// g = q mod 4 in increasing g, rs = norm_scale(S_0..S_3) -- the order the
// skinny form uses.  Thread (q, row): loads kScaleBatch sums at a time
// (coalesced over rows), adds them in order.
__global__ __launch_bounds__(4 * kScaleRows) void row_scale_kernel(const float* ss, int groups, int ld, int m0, int M,
                                                                   float inv_d, float eps, float* rs) {
  __shared__ float part[4][kScaleRows];
  const int r = threadIdx.x % kScaleRows, q = threadIdx.x / kScaleRows;
  const int m = min(blockIdx.x * kScaleRows + r, M - 1);
  float s = 0.f;
  for (int g0 = q; g0 < groups; g0 += 4 * kScaleBatch) {
    float v[kScaleBatch];
#pragma unroll
    for (int j = 0; j < kScaleBatch; ++j) {
      const int g = g0 + 4 * j;
      v[j] = g < groups ? ss[(size_t)g * ld + m0 + m] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kScaleBatch; ++j)
      if (g0 + 4 * j < groups) s += v[j];
  }
  part[q][r] = s;
  __syncthreads();
  if (q == 0 && blockIdx.x * kScaleRows + r < M)
    rs[m0 + m] = norm_scale(part[0][r], part[1][r], part[2][r], part[3][r], inv_d, eps);
}

template <int MW, int NWT, int PD, int EPI, bool SK, bool SS>
__global__ __launch_bounds__(kTileThreads) void gemm_tile_kernel(const GemmArgs a, const int n_chunks,
                                                                 const int n_mblk, const int n_grp) {
  static_assert(PD % 2 == 0, "the LDS buffer of a k-step is its parity");
  constexpr int NT = kTileThreads, BM = 16 * MW, UA = 8 * BM, UPT = (UA + NT - 1) / NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // workgroup -> (K chunk when split, row block, n-range): XCD = index mod
  // 8; the row blocks of an n-range are consecutive on that XCD.  Padding
  // workgroups return.
  const int xcd = blockIdx.x & 7, pos0 = blockIdx.x >> 3;
  const int chunk = SK ? pos0 % n_chunks : 0, pos = SK ? pos0 / n_chunks : pos0;
  const int mb = pos % n_mblk, grp = (pos / n_mblk) * 8 + xcd;
  if (grp >= n_grp) return;
  const int M = a.M, m0 = a.m0, ld = a.ld, ks = a.k_steps;
  const int per = ks / n_chunks;                // k-steps of a K chunk
  const int c0 = SK ? chunk * per : 0;          // this workgroup's k-steps: c0 .. c0 + ns - 1
  const int ns = SK ? per : ks;
  const int mrow0 = mb * BM, Mb = min(BM, M - mrow0);  // rows of this block, launch-relative
  const int tile0 = (grp * 4 + wave) * NWT;
  const int mrow = lane & 15, kq = lane >> 4;

  // Staged activations: [k-step % NB][part*4 + quad][row], then unused
  // padding.  With supersteps (SS) the k-steps run 4 per barrier, the next
  // superstep's activations written during the current one: NB = 8.
  static_assert(!SS || (PD == 8 && !SK), "supersteps need the 8-deep ring and whole-K workgroups");
  constexpr int NB = SS ? 8 : 4;
  __shared__ u32x4 As[NB][UPT * NT];
  __shared__ float rs[BM];

  const u32x4* wbase[NWT];
#pragma unroll
  for (int t = 0; t < NWT; ++t)
    wbase[t] = reinterpret_cast<const u32x4*>(a.W) + (size_t)min(tile0 + t, a.n_tiles - 1) * ks * 64 + lane;
  const u32x4* xbase = reinterpret_cast<const u32x4*>(a.xa);
  // this thread's activation units: u = tid + i*NT -> (part*4 + quad, row).
  // Rows past the block repeat its last row: an MFMA output row depends on
  // its own A row only, and those rows are never stored.  Units past UA land
  // in the padding of the buffer, so the stores need no branch.
  size_t aoff[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = min(tid + i * NT, UA - 1), r = u % BM, pq = u / BM;
    aoff[i] = (size_t)pq * ld + m0 + mrow0 + min(r, Mb - 1);
  }

  u32x4 wb[PD][NWT], ar[PD][UPT];
  auto load = [&](int p, int j) {  // ring slot p <- k-step c0 + j (clamped to the workgroup's range)
    const int s = c0 + min(j, ns - 1);
#pragma unroll
    for (int t = 0; t < NWT; ++t) wb[p][t] = wbase[t][(size_t)s * 64];
#pragma unroll
    for (int i = 0; i < UPT; ++i) ar[p][i] = xbase[(size_t)s * 8 * ld + aoff[i]];
  };
  auto put = [&](int p, int buf) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) As[buf][tid + i * NT] = ar[p][i];
  };
  // A operands of one k-step (hi, lo per m-tile), double-buffered by parity
  u32x4 ah[2][MW], al[2][MW];
  auto fetch = [&](int q, int buf) {
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
      ah[q][mt] = As[buf][kq * BM + mt * 16 + mrow];
      al[q][mt] = As[buf][(4 + kq) * BM + mt * 16 + mrow];
    }
  };

  f32x4 hi[MW][NWT], lo[MW][NWT], y[MW][NWT];
#pragma unroll
  for (int mt = 0; mt < MW; ++mt)
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      hi[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      lo[mt][t] = hi[mt][t];
      y[mt][t] = hi[mt][t];
    }
  auto compute = [&](int q, int p) {
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int t = 0; t < NWT; ++t) {
        hi[mt][t] = mfma(ah[q][mt], wb[p][t], hi[mt][t]);
        lo[mt][t] = mfma(al[q][mt], wb[p][t], lo[mt][t]);
      }
  };
  // end of a K chunk: its sum (hi + lo) joins the running sum in chunk order
  auto close_chunk = [&]() {
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int t = 0; t < NWT; ++t) {
        y[mt][t] += hi[mt][t] + lo[mt][t];
        hi[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        lo[mt][t] = hi[mt][t];
      }
  };

  // operand prologue (PD k-steps)
#pragma unroll
  for (int p = 0; p < PD; ++p) load(p, p);

  // RMSNorm scales of the block's rows (row_scale_kernel ran just before)
  for (int r = tid; r < BM; r += NT) rs[r] = a.rs != nullptr ? a.rs[m0 + mrow0 + min(r, Mb - 1)] : 1.0f;

  // Main loop over the workgroup's k-steps j = 0 .. ns - 1 (k-step c0 + j).
  // Without supersteps, step j: its A operands were fetched from LDS buffer j & 3 during step
  // j - 1; it fetches step j + 1's, runs its MFMAs, stores A(j + 2) into
  // buffer (j + 2) & 3, refills ring slot j % PD with step j + PD and meets
  // the workgroup at a barrier (so A(j + 2) is visible when step j + 1
  // fetches it, and buffer (j + 2) & 3, last read during step j - 3, is
  // free).  Steps run in unrolled groups of 8; a whole-K workgroup's chunks
  // are multiples of 8 steps (gemm_tile_fits) and close between groups, a
  // K-split workgroup runs one chunk and a guarded tail.
  // With supersteps of 4: A(j) sits in buffer j & 7, written during the
  // previous superstep (from ring slot j % 8, loaded 4 steps before that);
  // step j reads A(j) first if it opens a superstep, A(j + 1) if the
  // superstep goes on, runs its MFMAs, stores A(j + 4) into buffer (j + 4) &
  // 7 (last read during the previous superstep), refills its ring slot with
  // k-step j + 8, and the superstep's last step meets the workgroup at the
  // barrier.  The MFMAs and their order are the same either way.
  static_assert(PD == 4 || PD == 8, "ring slots and LDS buffers rotate together");
  if constexpr (SS) {
#pragma unroll
    for (int p = 0; p < 4; ++p) put(p, p);
    __syncthreads();
  } else {
    put(0, 0);
    put(1, 1);
    __syncthreads();
    fetch(0, 0);
  }
  auto step = [&](int p, int j0) {
    if constexpr (SS) {
      const int i = p & 3;  // place in the superstep (j0 is a multiple of 8)
      if (i == 0) fetch(p & 1, p & 7);
      if (i < 3) fetch((p + 1) & 1, (p + 1) & 7);
      compute(p & 1, p);
      put((p + 4) & 7, (p + 4) & 7);
      load(p, j0 + p + PD);
      if (i == 3) __syncthreads();
    } else {
      fetch((p + 1) & 1, (p + 1) & 3);
      compute(p & 1, p % PD);
      put((p + 2) % PD, (p + 2) & 3);
      load(p % PD, j0 + p + PD);
      __syncthreads();
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int j0 = 0;
  for (; j0 + 8 <= ns; j0 += 8) {
#pragma unroll
    for (int p = 0; p < 8; ++p) step(p, j0);
    if (!SK && (j0 + 8) % per == 0) close_chunk();
  }
  if (SK && j0 < ns) {
#pragma unroll
    for (int p = 0; p < 8; ++p)
      if (j0 + p < ns) step(p, j0);
  }

  if constexpr (SK) {
    // Publish this chunk's sum (hi + lo) with device-coherent stores, count
    // the workgroup in, and let the last of the tile's n_chunks workgroups
    // add the chunk sums in chunk order -- the skinny form's order -- before
    // the epilogue.
    __shared__ int s_last;
    const size_t tile_rec = (size_t)MW * NWT * 64 * 2;  // uint64 pairs per wave
    const size_t cell = (size_t)grp * n_mblk + mb;
    uint64_t* pw = reinterpret_cast<uint64_t*>(a.kpart) + ((cell * n_chunks + chunk) * 4 + wave) * tile_rec;
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int t = 0; t < NWT; ++t) {
        const f32x4 v = hi[mt][t] + lo[mt][t];
        const size_t e = ((size_t)(mt * NWT + t) * 64 + lane) * 2;
        __hip_atomic_store(pw + e, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pw + e + 1, (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    // the stores must have completed before the count (a workgroup-scope
    // fence does not wait for stores on this target)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(a.kcnt + cell, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old == (unsigned)(n_chunks - 1);
      if (s_last) __hip_atomic_store(a.kcnt + cell, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    const uint64_t* pr = reinterpret_cast<const uint64_t*>(a.kpart) + (cell * n_chunks * 4 + wave) * tile_rec;
    for (int c = 0; c < n_chunks; ++c) {
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int t = 0; t < NWT; ++t) {
          const size_t e = (size_t)c * 4 * tile_rec + ((size_t)(mt * NWT + t) * 64 + lane) * 2;
          const uint64_t u0 = __hip_atomic_load(pr + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t u1 = __hip_atomic_load(pr + e + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const f32x4 v = {__uint_as_float((uint32_t)u0), __uint_as_float((uint32_t)(u0 >> 32)),
                           __uint_as_float((uint32_t)u1), __uint_as_float((uint32_t)(u1 >> 32))};
          y[mt][t] += v;
        }
    }
  }
  __syncthreads();  // the epilogues reuse the operand buffers

  // ---- epilogues.  Lane holds column lane % 16 of each n-tile and rows
  // 4 * (lane / 16) + r of each m-tile.  Every load an epilogue needs is
  // issued before its first store (a load issued after a store waits for
  // that store too); neighbours are exchanged with DPP, not through LDS.
  const int cl = lane & 15, rq = lane >> 4;
  float rsv[MW][4];
  int mrow_[MW][4];
  bool mok[MW][4];
#pragma unroll
  for (int mt = 0; mt < MW; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = mt * 16 + rq * 4 + r;
      rsv[mt][r] = rs[lr];
      mok[mt][r] = mrow0 + lr < M;
      mrow_[mt][r] = min(mrow0 + lr, M - 1);  // launch-relative row, clamped for loads
    }
  if constexpr (EPI == EPI_RESID) {
    float hv[NWT][MW][4], gv[NWT];
    int crow[MW][4];
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int nn = min(tile0 + t, a.n_tiles - 1) * 16 + cl;
      gv[t] = a.g_next[nn];
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hv[t][mt][r] = a.h[(size_t)(m0 + mrow_[mt][r]) * a.d + nn];
    }
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) crow[mt][r] = a.h_copy != nullptr ? a.out_row[mrow_[mt][r]] : 0;
    float* sqt = reinterpret_cast<float*>(&As[0][0]) + wave * BM * 16;  // [BM][16] squares per wave
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int tile = tile0 + t;
      const bool tok = tile < a.n_tiles;
      const int nn = min(tile, a.n_tiles - 1) * 16 + cl;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = mt * 16 + rq * 4 + r, m = mrow0 + lr;
          const float v = hv[t][mt][r] + y[mt][t][r];
          if (tok && mok[mt][r]) {
            a.h[(size_t)(m0 + m) * a.d + nn] = v;
            if (a.h_copy != nullptr) a.h_copy[(size_t)crow[mt][r] * a.d + nn] = v;
            xa_store(a.xa_next, nn, m0 + m, ld, v * gv[t]);
          }
          sqt[lr * 16 + cl] = v * v;
        }
      __syncthreads();
      for (int lr = lane; lr < BM; lr += 64) {
        const int m = mrow0 + lr;
        if (tok && m < M) {
          float sum = 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c) sum += sqt[lr * 16 + c];
          a.ss_out[(size_t)tile * ld + m0 + m] = sum;
        }
      }
      __syncthreads();
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int hd = a.hd, half = hd >> 1;
    const bool odd = cl & 1;
    float2 rp[NWT][MW][4];
    int kvr[MW][4];
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int nn = min(tile0 + t, a.n_tiles - 1) * 16 + cl;  // packed: pair (i, i + hd/2) at columns (2j, 2j + 1)
      const int ci = (nn % hd) >> 1;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) rp[t][mt][r] = a.rope[(size_t)(m0 + mrow_[mt][r]) * half + ci];
    }
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) kvr[mt][r] = a.kvrow[m0 + mrow_[mt][r]];
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int tile = tile0 + t;
      const bool tok = tile < a.n_tiles;
      const int nn = min(tile, a.n_tiles - 1) * 16 + cl;
      const int hb = nn / hd, ci = (nn % hd) >> 1;
      const bool rot = hb < a.H + a.Hkv;
      const int el = odd ? ci + half : ci;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mrow_[mt][r];
          const float own = y[mt][t][r] * rsv[mt][r];
          const float other = dpp_swap1(own);
          const float y0 = odd ? other : own, y1 = odd ? own : other;
          if (!(tok && mok[mt][r])) continue;
          float o = odd ? y1 : y0;
          if (rot) o = odd ? rope_second(y0, y1, rp[t][mt][r]) : rope_first(y0, y1, rp[t][mt][r]);
          if (hb < a.H) {
            a.q[((size_t)(m0 + m) * a.H + hb) * hd + el] = o;
          } else {
            const bool is_k = rot;
            const int kvh = is_k ? hb - a.H : hb - a.H - a.Hkv;
            const int dst = kvr[mt][r];
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
      const bool tok = tile < a.n_tiles;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float own = y[mt][t][r] * rsv[mt][r];
          const float up = dpp_swap1(own);  // packed: (gate f, up f) at columns (2j, 2j + 1)
          if (tok && mok[mt][r] && !(cl & 1))
            xa_store(a.xa_act, tile * 8 + (cl >> 1), m0 + mrow0 + mt * 16 + rq * 4 + r, ld, silu_mul(own, up));
        }
    }
  } else {  // EPI_LOGITS
    int orow[MW][4];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) orow[mt][r] = a.out_row_identity ? m0 + mrow_[mt][r] : a.out_row[mrow_[mt][r]];
#pragma unroll
    for (int t = 0; t < NWT; ++t) {
      const int tile = tile0 + t;
      const bool tok = tile < a.n_tiles;
      const int nn = tile * 16 + cl;
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mrow0 + mt * 16 + rq * 4 + r;
          const bool ok = tok && mok[mt][r];
          const float z = y[mt][t][r] * rsv[mt][r];
          if (ok && a.logits != nullptr && orow[mt][r] >= 0) a.logits[(size_t)orow[mt][r] * a.V + nn] = z;
          // argmax over the tile's 16 columns, lowest column on ties
          float bv = z;
          int bi = nn;
          argmax16(bv, bi);
          if (ok && cl == 0) {
            a.amax_val[(size_t)tile * ld + m0 + m] = bv;
            a.amax_idx[(size_t)tile * ld + m0 + m] = bi;
          }
        }
    }
  }
}

void launch_row_scale(const GemmArgs& a, hipStream_t st, hipEvent_t start) {
  const dim3 sg((a.M + kScaleRows - 1) / kScaleRows);
  if (start != nullptr)
    hipExtLaunchKernelGGL(row_scale_kernel, sg, dim3(4 * kScaleRows), 0, st, start, nullptr, 0, a.ss, a.ss_groups, a.ld,
                          a.m0, a.M, a.inv_d, a.eps, a.rs_buf);
  else
    hipLaunchKernelGGL(row_scale_kernel, sg, dim3(4 * kScaleRows), 0, st, a.ss, a.ss_groups, a.ld, a.m0, a.M, a.inv_d,
                       a.eps, a.rs_buf);
}

namespace {

struct Ev {
  hipEvent_t a, b;
};

template <int EPI, int MW, int NWT, bool SK>
void go_tile(const GemmArgs& a, int n_mblk, hipStream_t st, Ev ev) {
  // A 4-deep ring for the K-split form, whose workgroups run one chunk (the
  // 7B down projection at 40 and 64 rows: 35.6 -> 34.8 and 38.8 -> 38.2 us);
  // otherwise 8, with supersteps where the k-step is long (12 or more
  // MFMA tiles per wave: the 70B batch, QKV 223 -> 216 us, down 353 -> 350
  // us; at 40-64 rows they gained nothing)
  constexpr int PD = SK ? 4 : 8;
  constexpr bool SS = !SK && MW * NWT >= 12;
  const int n_grp = (a.n_tiles + 4 * NWT - 1) / (4 * NWT);
  const int nc = gemm_k_chunks(a.n_tiles);
  const dim3 grid(8 * (SK ? nc : 1) * n_mblk * ((n_grp + 7) / 8));
  GemmArgs g = a;
  hipEvent_t start = ev.a;
  if (a.ss != nullptr) {
    launch_row_scale(a, st, start);
    start = nullptr;
    g.rs = a.rs_buf;
  }
  if (start != nullptr || ev.b != nullptr)
    hipExtLaunchKernelGGL((gemm_tile_kernel<MW, NWT, PD, EPI, SK, SS>), grid, dim3(kTileThreads), 0, st, start, ev.b, 0, g,
                          nc, n_mblk, n_grp);
  else
    hipLaunchKernelGGL((gemm_tile_kernel<MW, NWT, PD, EPI, SK, SS>), grid, dim3(kTileThreads), 0, st, g, nc, n_mblk, n_grp);
}

// Four n-tiles per wave only with up to three m-tiles: beyond that the
// accumulators and the operand rings do not fit the registers.  The K split
// is only used with blocks of up to 2 m-tiles (passes of up to 64 rows).
template <int EPI, int MW, bool SK>
void go_ntw(const GemmArgs& a, int n_mblk, int ntw, hipStream_t st, Ev ev) {
  if (ntw == 1) go_tile<EPI, MW, 1, SK>(a, n_mblk, st, ev);
  else if (ntw == 2 || MW > 3) go_tile<EPI, MW, 2, SK>(a, n_mblk, st, ev);
  else go_tile<EPI, MW, (MW > 3 ? 2 : 4), SK>(a, n_mblk, st, ev);
}

template <int EPI>
void go_epi(const GemmArgs& a, const TileShape& sh, hipStream_t st, Ev ev) {
  if (sh.split) {
    if (sh.mw == 1) go_ntw<EPI, 1, true>(a, sh.n_mblk, sh.ntw, st, ev);
    else go_ntw<EPI, 2, true>(a, sh.n_mblk, sh.ntw, st, ev);
    return;
  }
  switch (sh.mw) {
    case 1: go_ntw<EPI, 1, false>(a, sh.n_mblk, sh.ntw, st, ev); break;
    case 2: go_ntw<EPI, 2, false>(a, sh.n_mblk, sh.ntw, st, ev); break;
    case 4: go_ntw<EPI, 4, false>(a, sh.n_mblk, sh.ntw, st, ev); break;
    default: go_ntw<EPI, 3, false>(a, sh.n_mblk, sh.ntw, st, ev); break;
  }
}

}  // namespace

// Up to 4 m-tiles (64 rows, bound by the weight stream): blocks of 2
// m-tiles, which keeps more workgroups and waves in flight (measured at 17,
// 40 and 64 rows on the 7B QKV, gate/up and head), except on the widest
// matrices at 3 or 4 m-tiles (one block, below); the narrow matrices
// split K over workgroups as well (gemm_tile_split).  More rows (bound by
// MFMA issue and LDS reads): blocks of 3 m-tiles, whose waves take 4
// n-tiles each where the grid stays full (an LDS fragment then feeds 8
// MFMAs).  N-range: the widest (4, 2 or 1 n-tiles per wave; 4 only with up
// to 3 m-tiles) that still gives >= 200 workgroups (>= 400 with K split).
TileShape gemm_tile_shape(int n_tiles, int M, int ntw) {
  TileShape sh;
  const int mt = (M + 15) / 16;
  sh.split = n_tiles < 512;  // the launcher only sends narrow matrices that split K (gemm_tile_fits)
  sh.mw = mt <= 4 ? std::min(mt, 2) : 3;
  sh.n_mblk = (mt + sh.mw - 1) / sh.mw;
  const long per_grp = (long)sh.n_mblk * (sh.split ? gemm_k_chunks(n_tiles) : 1);
  const long want = sh.split ? 400 : 200;  // split: measured best at about two workgroups per CU
  if (ntw == 1 || ntw == 2 || ntw == 4) {
    sh.ntw = ntw;
  } else {
    sh.ntw = 1;
    for (int w : {4, 2})
      if ((n_tiles + 4 * w - 1) / (4 * w) * per_grp >= want) {
        sh.ntw = w;
        break;
      }
  }
  if (sh.mw > 3 && sh.ntw == 4) sh.ntw = 2;
  // The widest matrices (>= 1024 n-tiles: the 7B gate/up and head) at 33 to
  // 64 rows: one row block of all rows (3 or 4 m-tiles) with 2 n-tiles per
  // wave.  Measured on gate/up: 54.0 against 61-63 us at 40 rows, 62.3
  // against 66-68 us at 64 rows; QKV (768 n-tiles) lost (51-59 against
  // 42-47 us) and keeps two 32-row blocks.
  if (!sh.split && mt >= 3 && mt <= 4 && n_tiles >= 1024 && ntw != 1 && ntw != 4) {
    sh.mw = mt;
    sh.n_mblk = 1;
    sh.ntw = 2;
  }
  return sh;
}

int launch_gemm_tile(const GemmArgs& a, int epi, int ntw, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const Ev ev{ev0, ev1};
  const TileShape sh = gemm_tile_shape(a.n_tiles, a.M, ntw);
  switch (epi) {
    case EPI_RESID: go_epi<EPI_RESID>(a, sh, st, ev); break;
    case EPI_QKV: go_epi<EPI_QKV>(a, sh, st, ev); break;
    case EPI_SWIGLU: go_epi<EPI_SWIGLU>(a, sh, st, ev); break;
    default: go_epi<EPI_LOGITS>(a, sh, st, ev); break;
  }
  return a.n_tiles;
}

}  // namespace vs
