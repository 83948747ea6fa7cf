// Masked multi-query attention over the paged KV cache (gfx950), for passes
// whose KV heads carry one query group (at most 16 query vectors: the rows
// of a chain times the query heads of a KV head).
//
// A verify pass has a few rows per sequence (k+1 chain positions); each row
// attends to every committed key of its sequence plus the in-round keys its
// ancestor mask selects ("FlashSpec" page, lnrk.cn/news/47842, §2.2:
// level-order tree batch with a parent mask; §5.2: nothing outside the mask
// may leak).  All query rows and grouped heads of a KV head share one read
// of each K/V block.
//
// KV layout per layer: K [block][kv head][16 keys][head_dim], V [block][kv
// head][head_dim][16 keys].  With that layout both MFMA operands come straight
// from HBM as 16-byte pieces: for S = Q.K^T a lane reads 8 dims of one key
// row, for O += P.V a lane reads 8 consecutive keys of one dim.
//
// Split structure, fixed by absolute key index and the sequence's own KV
// length P (read here on the device), so that a row's bits never depend on
// the other sequences of its pass or on how the work is spread:
//  * committed split j holds keys [32 j, 32 j + 32) below P (one step); the
//    in-round window is split ceil(P / 32);
//  * chunk c is splits [8 c, 8 c + 8), one per wave; its waves' (max, sum,
//    o) are merged in LDS in wave order into the chunk's partial;
//  * the chunks of a unit (sequence, KV head) are combined in chunk order.
// A workgroup runs cpw consecutive chunks of one unit (the host picks cpw
// for the pass): the loads of a wave's next step, in the next chunk too, are
// in flight while the current chunk merges.  A unit of one chunk writes its
// result directly; otherwise every chunk's partial is published with
// device-coherent stores (they write through this XCD's L2), the workgroup
// waits on its vector memory counter (which counts stores too) and, when the
// unit has more than one workgroup, counts itself in on a per-unit counter.
// The last workgroup of a unit reads every chunk partial with
// device-coherent loads, sums them in chunk order, writes the result as
// split-bf16 activation fragments for the O projection and resets the
// counter.  No agent-scope fence is used: a fence would write back or
// invalidate the whole L2.
#include "attn_dev.h"

namespace vs {

namespace {

// LDS writes of this wave done, then the workgroup barrier; global loads
// stay in flight (unlike __syncthreads(), which waits for them too).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int cmax(int x, int y) { return x > y ? x : y; }

}  // namespace

// Sequence of workgroup b: the last i with wg_start[i] <= b.
__device__ __forceinline__ int attn_seq_of(const AttnArgs& a, int b) {
  int lo = 0, hi = a.rows.n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.wg_start[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Query vector v of a unit maps to row r0 + v % nr and head kvh*G + v / nr.
template <int HD, int WV>
__global__ __launch_bounds__(WV * 64) void attn_kernel(const AttnArgs a) {
  constexpr int kThreads = WV * 64;
  constexpr int KSQ = HD / 32;  // k-steps of S over head dims
  constexpr int NDT = HD / 16;  // 16-dim output tiles
  constexpr int QR = 16;        // query vectors of the MFMA tile
  constexpr int PS = kStep + 4;  // P scratch row stride (floats)
  constexpr int HDP = HD + 4;    // merge row stride (floats): rows one lane group apart in other banks
  constexpr int PL_FLOATS = WV * QR * PS;
  constexpr int MG_FLOATS = WV * QR * HDP + 2 * WV * QR + 2 * QR + WV * QR;
  constexpr int CB_FLOATS = 3 * kAttnCombineSlots + kAttnQG;
  constexpr int SM_FLOATS = cmax(cmax(PL_FLOATS, MG_FLOATS), CB_FLOATS);
  __shared__ float smem[SM_FLOATS];
  __shared__ int last_wg;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x;
  if (b >= a.wg_start[a.rows.n_seq]) return;
  const int i = attn_seq_of(a, b);
  const int nwg_ub = (a.wg_start[i + 1] - a.wg_start[i]) / a.Hkv;
  const int local = b - a.wg_start[i];
  const int kvh = local / nwg_ub, wgi = local - kvh * nwg_ub;
  const int sq = a.rows.seq[i];
  const int r0 = a.rows.row_start[i];
  const int nr = a.rows.row_start[i + 1] - r0;
  const int G = a.H / a.Hkv;
  const int nq = min(QR, nr * G);
  const int P = a.kv.P[sq];
  const int ns = (P + kStep - 1) / kStep;          // committed splits
  // + the in-round window; never past the host's layout (P <= its bound)
  const int n_chunks = min((ns + 1 + WV - 1) / WV, a.nsplit[i]);
  const int c0 = wgi * a.cpw;
  if (c0 >= n_chunks) return;  // past what this sequence's context needs
  const int c1 = min(n_chunks, c0 + a.cpw);
  const int nwg = (n_chunks + a.cpw - 1) / a.cpw;  // workgroups of the unit with chunks
  const int unit = i * a.Hkv + kvh;
  const int wlo = P + a.rows.win, whi = wlo + a.rows.idx_off + nr;  // in-round keys
  const int* bt = a.kv.bt + (size_t)sq * a.kv.bps;
  const int mrow = lane & 15, kq = lane >> 4;
  const size_t head_stride = (size_t)kBlock * HD;  // elements per (block, kv head)

  // Steps of 32 keys aligned to blocks: [base, base+32) covers slots of two
  // blocks.  This wave's split in chunk c: a committed split is one step;
  // the window covers the steps that hold slots wlo .. whi-1.
  auto split_steps = [&](int c, int& first, int& last) {
    const int sp = c * WV + wave;
    if (sp < ns) {
      first = sp * kStep;
      last = first + kStep;
    } else if (sp == ns) {
      first = wlo / kStep * kStep;
      last = (whi + kStep - 1) / kStep * kStep;
    } else {
      first = last = 0;
    }
  };
  u32x4 kb[2][KSQ], vb[NDT];
  int nb0 = 0, nb1 = 0;  // blocks of the step being loaded
  auto blocks_of = [&](int base) {
    nb0 = bt[min(base / kBlock, a.kv.bps - 1)];  // clamped to the table; data outside the split is masked
    nb1 = bt[min(base / kBlock + 1, a.kv.bps - 1)];
  };
  auto load_k = [&]() {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* kr = a.kv.k + ((size_t)(t ? nb1 : nb0) * a.Hkv + kvh) * head_stride + mrow * HD + 8 * kq;
#pragma unroll
      for (int s = 0; s < KSQ; ++s) kb[t][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 32 * s));
    }
  };
  auto load_v = [&]() {  // lane: keys 8*kq .. +8 of dim 16t + lane%16, i.e. block kq/2, keys 8*(kq%2) ..
    const uint16_t* vr = a.kv.v + ((size_t)((kq >> 1) ? nb1 : nb0) * a.Hkv + kvh) * head_stride + 8 * (kq & 1);
#pragma unroll
    for (int t = 0; t < NDT; ++t)
      vb[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vr + (size_t)(16 * t + mrow) * kBlock));
  };

  // Request order: block-table entries of the first step, the query vectors
  // and masks, then the first K/V step (which waits only for the table
  // entries); the queries are split while K/V are in flight.
  int first, last;
  split_steps(c0, first, last);
  if (first < last) blocks_of(first);
  float4 qraw[KSQ][2];
  uint64_t qmask[4];  // visibility masks of the 4 rows this lane holds in S
  {
    const int gq = min(mrow, nq - 1);
    const float* src = a.q + ((size_t)(r0 + gq % nr) * a.H + kvh * G + gq / nr) * HD;
#pragma unroll
    for (int s = 0; s < KSQ; ++s) {
      qraw[s][0] = *reinterpret_cast<const float4*>(src + 32 * s + 8 * kq);
      qraw[s][1] = *reinterpret_cast<const float4*>(src + 32 * s + 8 * kq + 4);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * kq + r;
      const int rl = min(row, nq - 1) % nr;
      const int idx = a.rows.idx_off + rl;
      const uint64_t mk = a.rows.mask ? a.rows.mask[r0 + rl] : (idx >= 63 ? ~0ull : ((2ull << idx) - 1ull));
      qmask[r] = row < nq ? mk : 0ull;
    }
  }
  if (first < last) {
    load_k();
    load_v();
  }
  // query fragments (A operand of S), pre-scaled and split hi/lo.  Scores
  // are kept in base-2 units (the scale carries log2 e), so every softmax
  // exponential is one hardware exp2; max, sum and partials all use base 2.
  const float qscale = a.scale * 1.4426950408889634f;
  u32x4 qh[KSQ], ql[KSQ];
  {
    const bool qok = mrow < nq;
#pragma unroll
    for (int s = 0; s < KSQ; ++s) {
      const float4 u = qraw[s][0], v = qraw[s][1];
      const float x[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = qok ? x[e] * qscale : 0.f;
      split8(y, qh[s], ql[s]);
    }
  }

  const bool single = n_chunks == 1;  // the unit's only chunk: write the result
  const size_t QG = a.qg_size;
  float* po = a.part;                                              // [units][n_split][QG][HD]
  uint64_t* pml = reinterpret_cast<uint64_t*>(a.part + a.ml_off);  // [units][n_split][QG] (max, sum)
  float* pw = smem + wave * QR * PS;
  constexpr int DS = HD / WV;  // dims merged by one wave
  float* xo = smem;                                               // [WV][QR][HDP]
  float2* xml = reinterpret_cast<float2*>(smem + WV * QR * HDP);  // [WV][QR]
  float* rl = reinterpret_cast<float*>(xml + WV * QR);            // [QR] merged sum
  float* rm = rl + QR;                                            // [QR] merged max
  float* wts = rm + QR;                                           // [WV][QR]

  for (int c = c0; c < c1; ++c) {
    const int sp = c * WV + wave;
    const bool window = sp == ns;
    const int key_lo = window ? wlo : sp * kStep;
    const int key_hi = window ? whi : min(P, sp * kStep + kStep);
    float mrun[4], lrun[4];
    f32x4 oacc[NDT];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mrun[r] = -INFINITY;
      lrun[r] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < NDT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int base = first; base < last; base += kStep) {
      // the next step to load: this split's next one, else the first step
      // of this wave's split in the next chunk of the workgroup
      int nbase = base + kStep;
      bool more = nbase < last;
      if (!more && c + 1 < c1) {
        int nf, nl;
        split_steps(c + 1, nf, nl);
        nbase = nf;
        more = nf < nl;
      }
      if (more) blocks_of(nbase);
      // S = Q.K^T for the two 16-key tiles
      f32x4 sacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSQ; ++s) {
          cc = mfma16(qh[s], kb[t][s], cc);
          cc = mfma16(ql[s], kb[t][s], cc);
        }
        sacc[t] = cc;
      }
      if (more) load_k();
      // mask, online softmax update, P into the scratch (row, key) layout; a
      // step of committed keys inside the split needs no mask, and the
      // accumulators are rescaled only when some factor is not exactly 1
      const bool full = !window && base >= key_lo && base + kStep <= key_hi;
      float corr[4];
      bool same = true;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * kq + r;
        float v[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (full) {
            v[t] = sacc[t][r];
          } else {
            const int slot = base + 16 * t + mrow;
            bool vis = slot >= key_lo && slot < key_hi;
            if (vis && window) vis = (qmask[r] >> ((slot - key_lo) & 63)) & 1ull;  // count kept in 0..63
            v[t] = vis ? sacc[t][r] : -INFINITY;
          }
        }
        const float mx = row16_max(fmaxf(v[0], v[1]));
        const float mnew = fmaxf(mrun[r], mx);
        corr[r] = (mrun[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun[r] - mnew);
        same &= corr[r] == 1.f;
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float p = v[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(v[t] - mnew);
          pw[row * PS + 16 * t + mrow] = p;
          ps += p;
        }
        ps = row16_sum(ps);
        lrun[r] = lrun[r] * corr[r] + ps;
        mrun[r] = mnew;
      }
      if (!__all(same)) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int t = 0; t < NDT; ++t) oacc[t][r] *= corr[r];
      }
      // O += P.V (P rows in A-operand order: row = lane%16, keys 8*(lane/16) .. +8)
      {
        u32x4 ph, pl;
        split8(pw + mrow * PS + 8 * kq, ph, pl);
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          oacc[t] = mfma16(ph, vb[t], oacc[t]);
          oacc[t] = mfma16(pl, vb[t], oacc[t]);
        }
      }
      if (more) load_v();
    }

    // ---- merge the chunk's WV split partials: every wave puts its (max,
    // sum, o) for the rows below nq in LDS; the per-row weights
    // exp2(m_j - max) and the merged (max, sum) are computed once per row;
    // then wave w merges dims [w*DS, (w+1)*DS) of all WV partials in wave
    // order and writes that slice of the chunk's partial (or of the result).
    lds_sync();  // every wave is done with its P scratch (the merge area)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * kq + r;
      if (row < nq) {
#pragma unroll
        for (int t = 0; t < NDT; ++t) xo[(wave * QR + row) * HDP + 16 * t + mrow] = oacc[t][r];
        if (mrow == 0) xml[wave * QR + row] = make_float2(mrun[r], lrun[r]);
      }
    }
    lds_sync();
    for (int row = threadIdx.x; row < nq; row += kThreads) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < WV; ++j) {
        const float2 v = xml[j * QR + row];
        if (v.y > 0.f) mx = fmaxf(mx, v.x);  // a split that saw no key has sum 0
      }
      float l = 0.f;
#pragma unroll
      for (int j = 0; j < WV; ++j) {
        const float2 v = xml[j * QR + row];
        const float w = v.y > 0.f ? __builtin_amdgcn_exp2f(v.x - mx) : 0.f;
        wts[j * QR + row] = w;
        l += w * v.y;
      }
      rl[row] = l;
      rm[row] = mx;
    }
    lds_sync();
    const size_t rec = (size_t)unit * a.n_split + c;
    for (int e = lane; e < nq * DS; e += 64) {
      const int row = e / DS, d = wave * DS + e % DS;
      float o = 0.f;
#pragma unroll
      for (int j = 0; j < WV; ++j) o += wts[j * QR + row] * xo[(j * QR + row) * HDP + d];
      if (single)
        xa_store(a.xa_o, (kvh * G + row / nr) * HD + d, r0 + row % nr, a.M, o / rl[row]);
      else
        __hip_atomic_store(po + (rec * QG + row) * HD + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!single && threadIdx.x < nq) {
      const int row = threadIdx.x;
      const uint64_t bits = (uint64_t)__float_as_uint(rm[row]) | ((uint64_t)__float_as_uint(rl[row]) << 32);
      __hip_atomic_store(pml + rec * QG + row, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (c + 1 < c1) {
      lds_sync();  // the merge area is the next chunk's P scratch
      split_steps(c + 1, first, last);
    }
  }
  if (single) return;

  // The partial stores must have completed (written through to device
  // scope) before the workgroup is counted in or the partials are read back.
  // A workgroup-scope fence does not wait for stores on this target, so wait
  // on the vector memory counter itself (it counts stores too); the clobber
  // keeps the compiler from moving memory operations across the wait.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (nwg > 1) {
    if (threadIdx.x == 0) {
      const unsigned old = __hip_atomic_fetch_add(a.cnt + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int is_last = old == (unsigned)(nwg - 1);
      if (is_last) __hip_atomic_store(a.cnt + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_wg = is_last;
    }
    __syncthreads();
    if (!last_wg) return;
  }

  // ---- the unit's last workgroup: combine its n_chunks partials in chunk
  // order.  Each row's weights exp2(m_j - max) and total are computed once in
  // LDS; a thread then sums one pair of dims of one query vector over the
  // partials, with the loads of up to kCB partials in flight at once (the
  // first batch is requested before the weights exist).
  constexpr int HP = HD / 2;  // dim pairs
  constexpr int kCG = 8;      // partials per guarded group
  constexpr int kCB = 16;     // partials requested per batch
  const int nc = n_chunks;
  float2* cml = reinterpret_cast<float2*>(smem);  // [nc][nq] (max, sum)
  float* cwt = smem + 2 * kAttnCombineSlots;      // [nc][nq] weights
  float* ctot = cwt + kAttnCombineSlots;          // [nq]
  const uint64_t* src0 = reinterpret_cast<const uint64_t*>(po) + (size_t)unit * a.n_split * QG * HP;
  const int S = (int)QG * HP;  // pairs between consecutive partials
  const int npair = nq * HP;
  uint64_t xc[kCB];
  auto load_batch = [&](int p, int j0) {
    const uint64_t* src = src0 + min(p, npair - 1);
#pragma unroll
    for (int g = 0; g < kCB / kCG; ++g)
      if (j0 + g * kCG < nc) {
#pragma unroll
        for (int e = g * kCG; e < (g + 1) * kCG; ++e)
          xc[e] = __hip_atomic_load(src + min(j0 + e, nc - 1) * S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  };
  if (threadIdx.x < npair) load_batch(threadIdx.x, 0);
  for (int e = threadIdx.x; e < nc * nq; e += kThreads) {
    const int j = e / nq, r = e - j * nq;
    const uint64_t bits = __hip_atomic_load(pml + ((size_t)unit * a.n_split + j) * QG + r, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    cml[e] = make_float2(__uint_as_float((uint32_t)bits), __uint_as_float((uint32_t)(bits >> 32)));
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nq; r += kThreads) {
    float mx = -INFINITY;
    for (int j = 0; j < nc; ++j)
      if (cml[j * nq + r].y > 0.f) mx = fmaxf(mx, cml[j * nq + r].x);
    float tot = 0.f;
    for (int j = 0; j < nc; ++j) {
      const float2 v = cml[j * nq + r];
      const float w = v.y > 0.f ? __builtin_amdgcn_exp2f(v.x - mx) : 0.f;
      cwt[j * nq + r] = w;
      tot += w * v.y;
    }
    ctot[r] = tot;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < npair; p += kThreads) {
    const int r = p / HP, cp = p - r * HP;
    float o0 = 0.f, o1 = 0.f;
    for (int j0 = 0; j0 < nc; j0 += kCB) {
      if (p != threadIdx.x || j0 > 0) load_batch(p, j0);
#pragma unroll
      for (int g = 0; g < kCB / kCG; ++g)
        if (j0 + g * kCG < nc) {
#pragma unroll
          for (int e = g * kCG; e < (g + 1) * kCG; ++e) {
            const int j = j0 + e;
            const float w = j < nc ? cwt[j * nq + r] : 0.f;
            o0 += w * __uint_as_float((uint32_t)xc[e]);
            o1 += w * __uint_as_float((uint32_t)(xc[e] >> 32));
          }
        }
    }
    const float tot = ctot[r];
    const int m = r0 + r % nr, h = kvh * G + r / nr;
    xa_store(a.xa_o, h * HD + 2 * cp, m, a.M, o0 / tot);
    xa_store(a.xa_o, h * HD + 2 * cp + 1, m, a.M, o1 / tot);
  }
}

hipError_t attn_init() { return hipSuccess; }

void launch_attention(const AttnArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid(a.wg_start[a.rows.n_seq]);
#define VS_ATT(HD)                                                                                          \
  do {                                                                                                      \
    if (ev0 != nullptr || ev1 != nullptr)                                                                   \
      hipExtLaunchKernelGGL((attn_kernel<HD, kAttnWaves>), grid, dim3(kAttnWaves * 64), 0, st, ev0, ev1, 0, a); \
    else                                                                                                    \
      hipLaunchKernelGGL((attn_kernel<HD, kAttnWaves>), grid, dim3(kAttnWaves * 64), 0, st, a);            \
  } while (0)
  if (a.hd == 128) VS_ATT(128);
  else VS_ATT(64);
#undef VS_ATT
}

}  // namespace vs
