// Masked multi-query attention over the paged KV cache (gfx950).
//
// A verify pass has a few rows per sequence (k+1 chain positions or up to 64
// tree nodes); each row attends to every committed key of its sequence plus
// the in-round keys its ancestor mask selects ("FlashSpec" page,
// lnrk.cn/news/47842, §2.2: level-order tree batch with a parent mask; §5.2:
// nothing outside the mask may leak).  All query rows and grouped heads of a
// KV head share one read of each K/V block.
//
// KV layout per layer: K [block][kv head][16 keys][head_dim], V [block][kv
// head][head_dim][16 keys].  With that layout both MFMA operands come straight
// from HBM as 16-byte pieces: for S = Q.K^T a lane reads 8 dims of one key
// row, for O += P.V a lane reads 8 consecutive keys of one dim.
//
// Work split: a wave owns one split of the keys (a range of committed keys,
// or the in-round window) of one (sequence, KV head, query group) and keeps
// its own online softmax, with no K/V staging.  Per 32-key step: S for two
// 16-key tiles (bf16 16x16x32 MFMA, the query split into bf16 hi + lo parts so
// scores keep fp32 precision), masking, softmax update in fp32, P through a
// small per-wave LDS scratch into A-operand order (again split hi/lo), then
// O += P.V.  The next step's K/V loads are in flight while the current one
// computes.
//
// Combining the splits happens in the same launch.  The waves of a
// workgroup put their (max, sum, o) in LDS; each wave then merges one slice
// of the head dims over all of them in wave order and publishes that slice
// of the workgroup's partial with device-coherent stores (they write
// through this XCD's L2).  Thread 0 then counts the workgroup in on a
// per-unit counter.  The last workgroup of a unit to arrive reads every
// partial with device-coherent loads, sums them in workgroup order, and
// writes the result as split-bf16 activation fragments for the O
// projection; it also resets the counter to zero.  The result does not
// depend on which workgroup arrives last.  No agent-scope fence is used: a
// fence would write back or invalidate the whole L2.  Ordering comes from
// waiting on the vector memory counter before the count, so the
// device-coherent stores have completed.
#include "attn_dev.h"

namespace vs {

// Query vectors of a unit: vector gq of the query group maps to row
// r0 + gq % nr and head kvh*G + gq / nr.
template <int MTQ, int HD, int WV>
__global__ __launch_bounds__(WV * 64) void attn_kernel(const AttnArgs a) {
  constexpr int kWaves = WV, kThreads = WV * 64;
  constexpr int KSQ = HD / 32;  // k-steps of S over head dims
  constexpr int NDT = HD / 16;  // 16-dim output tiles
  constexpr int QR = MTQ * 16;
  constexpr int PS = kStep + 4;  // P scratch row stride (floats)
  constexpr int PL_FLOATS = kWaves * QR * PS;
  constexpr int MG_FLOATS = WV * QR * (HD + 4) + 2 * WV * QR + 2 * QR + WV * QR;
  constexpr int SM_FLOATS = PL_FLOATS > MG_FLOATS ? PL_FLOATS : MG_FLOATS;
  static_assert(SM_FLOATS >= 3 * kAttnCombineSlots + kAttnQG, "combine scratch");
  __shared__ float smem[SM_FLOATS];
  __shared__ int last_wg;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wps = (a.n_split + 1 + kWaves - 1) / kWaves;  // partial records per unit (layout)
  // The query groups of one (sequence, KV head, key range) read the same
  // K/V.  Workgroups are handed to the 8 XCDs round-robin by index, so the
  // index b is read as XCD b % 8 and position b / 8 on it; the host lays the
  // work out (map) so that the query groups of a key range run back to back
  // on one XCD and the later ones find the K/V in its L2.  Without a map:
  // every sequence takes n_split splits and n_qg query groups, the query
  // group varying fastest along the position.
  int i, kvh, qg, wgi;
  if (a.map != nullptr) {
    const int e = a.map[blockIdx.x];
    if (e < 0) return;  // grid padding
    i = e & 63;
    kvh = (e >> 6) & 127;
    qg = (e >> 13) & 127;
    wgi = e >> 20;
  } else {
    const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
    qg = pos % a.n_qg;
    const int g = (pos / a.n_qg) * 8 + xcd;  // (sequence, workgroup of the unit, KV head)
    const int X = a.rows.n_seq * wps;
    if (g >= X * a.Hkv) return;  // grid padding
    i = (g % X) / wps;
    wgi = (g % X) % wps;
    kvh = g / X;
  }
  const int n_split = a.map != nullptr ? a.nsplit[i] : a.n_split;  // this sequence's committed splits
  const int n_parts = n_split + 1;
  const int wpb = (n_parts + kWaves - 1) / kWaves;  // workgroups of this unit
  const int split = wgi * kWaves + wave;
  const int sq = a.rows.seq[i];
  const int r0 = a.rows.row_start[i];
  const int nr = a.rows.row_start[i + 1] - r0;
  const int G = a.H / a.Hkv;
  const int q0 = qg * a.qg_size;
  const int nq = max(0, min(a.qg_size, nr * G - q0));
  if (nq == 0) return;  // whole unit: nothing to attend for this query group
  const int unit = (i * a.Hkv + kvh) * a.n_qg + qg;
  const bool active = split < n_parts;
  const int P = a.kv.P[sq];
  const int W = a.rows.idx_off + nr;  // in-round keys present: window indices 0..W-1
  const bool window = split == n_split;
  int key_lo, key_hi;  // valid slots of this split
  if (!window) {
    key_lo = split * a.kps;
    key_hi = min(P, key_lo + a.kps);
  } else {
    key_lo = P + a.rows.win;
    key_hi = key_lo + W;
  }
  const int* bt = a.kv.bt + (size_t)sq * a.kv.bps;
  const int mrow = lane & 15, kq = lane >> 4;
  const size_t head_stride = (size_t)kBlock * HD;  // elements per (block, kv head)

  // Steps of 32 keys aligned to blocks: [base, base+32) covers slots of two
  // blocks.  A committed split's steps and block-table entries follow from
  // the split index alone (P only masks), so its first K/V loads do not wait
  // for P.  K of the next step is requested right after this step's S, V of
  // the next step right after this step's P.V.
  const int first = window ? (key_lo / kStep) * kStep : split * a.kps;
  // exclusive; a committed split stops at the last step holding committed
  // keys (splits wholly past P run no step: their first loads, issued
  // before P is known, go unused)
  const int last = !active ? first : window ? key_hi : min(split * a.kps + a.kps, (P + kStep - 1) / kStep * kStep);
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
  if (active) blocks_of(first);
  float4 qraw[MTQ][KSQ][2];
  uint64_t qmask[MTQ][4];  // visibility masks of the 4 rows this lane holds in S
#pragma unroll
  for (int mt = 0; mt < MTQ; ++mt) {
    const int qv = mt * 16 + mrow;
    const int gq = q0 + min(qv, nq - 1);
    const float* src = a.q + ((size_t)(r0 + gq % nr) * a.H + kvh * G + gq / nr) * HD;
#pragma unroll
    for (int s = 0; s < KSQ; ++s) {
      qraw[mt][s][0] = *reinterpret_cast<const float4*>(src + 32 * s + 8 * kq);
      qraw[mt][s][1] = *reinterpret_cast<const float4*>(src + 32 * s + 8 * kq + 4);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mt * 16 + 4 * kq + r;
      const int rl = (q0 + min(row, nq - 1)) % nr;
      const int idx = a.rows.idx_off + rl;
      const uint64_t mk = a.rows.mask ? a.rows.mask[r0 + rl] : (idx >= 63 ? ~0ull : ((2ull << idx) - 1ull));
      qmask[mt][r] = row < nq ? mk : 0ull;
    }
  }
  if (active) {  // a wave past the last split only takes part in the merge
    load_k();
    load_v();
  }
  // query fragments (A operand of S), pre-scaled and split hi/lo.  Scores
  // are kept in base-2 units (the scale carries log2 e), so every softmax
  // exponential is one hardware exp2; max, sum and partials all use base 2.
  const float qscale = a.scale * 1.4426950408889634f;
  u32x4 qh[MTQ][KSQ], ql[MTQ][KSQ];
#pragma unroll
  for (int mt = 0; mt < MTQ; ++mt) {
    const bool qok = mt * 16 + mrow < nq;
#pragma unroll
    for (int s = 0; s < KSQ; ++s) {
      const float4 u = qraw[mt][s][0], v = qraw[mt][s][1];
      const float x[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = qok ? x[e] * qscale : 0.f;
      split8(y, qh[mt][s], ql[mt][s]);
    }
  }

  float mrun[MTQ][4], lrun[MTQ][4];
  f32x4 oacc[MTQ][NDT];
#pragma unroll
  for (int mt = 0; mt < MTQ; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mrun[mt][r] = -INFINITY;
      lrun[mt][r] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < NDT; ++t) oacc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float* pw = smem + wave * QR * PS;
  for (int base = first; base < last; base += kStep) {
    const bool more = base + kStep < last;
    if (more) blocks_of(base + kStep);
    // S = Q.K^T for the two 16-key tiles
    f32x4 sacc[MTQ][2];
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSQ; ++s) {
          c = mfma16(qh[mt][s], kb[t][s], c);
          c = mfma16(ql[mt][s], kb[t][s], c);
        }
        sacc[mt][t] = c;
      }
    if (more) load_k();
    // mask, online softmax update, P into the scratch (row, key) layout; a
    // step of committed keys inside the split needs no mask, and the
    // accumulators are rescaled only when some factor is not exactly 1
    const bool full = !window && base >= key_lo && base + kStep <= key_hi;
    float corr[MTQ][4];
    bool same = true;
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mt * 16 + 4 * kq + r;
        float v[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          if (full) {
            v[t] = sacc[mt][t][r];
          } else {
            const int slot = base + 16 * t + mrow;
            bool vis = slot >= key_lo && slot < key_hi;
            if (vis && window) vis = (qmask[mt][r] >> ((slot - key_lo) & 63)) & 1ull;  // count kept in 0..63
            v[t] = vis ? sacc[mt][t][r] : -INFINITY;
          }
        }
        const float mx = row16_max(fmaxf(v[0], v[1]));
        const float mnew = fmaxf(mrun[mt][r], mx);
        corr[mt][r] = (mrun[mt][r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun[mt][r] - mnew);
        same &= corr[mt][r] == 1.f;
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float p = v[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(v[t] - mnew);
          pw[row * PS + 16 * t + mrow] = p;
          ps += p;
        }
        ps = row16_sum(ps);
        lrun[mt][r] = lrun[mt][r] * corr[mt][r] + ps;
        mrun[mt][r] = mnew;
      }
    if (!__all(same)) {
#pragma unroll
      for (int mt = 0; mt < MTQ; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int t = 0; t < NDT; ++t) oacc[mt][t][r] *= corr[mt][r];
    }
    // O += P.V (P rows in A-operand order: row = lane%16, keys 8*(lane/16) .. +8)
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt) {
      u32x4 ph, pl;
      split8(pw + (mt * 16 + mrow) * PS + 8 * kq, ph, pl);
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        oacc[mt][t] = mfma16(ph, vb[t], oacc[mt][t]);
        oacc[mt][t] = mfma16(pl, vb[t], oacc[mt][t]);
      }
    }
    if (more) load_v();
  }


  // ---- merge the waves' partials: every wave puts its (max, sum, o) for
  // the rows below nq in LDS; the per-row weights exp2(m_j - max) and the
  // merged (max, sum) are computed once per row; then wave w merges dims
  // [w*DS, (w+1)*DS) of all WV partials in wave order and writes that slice
  // of the workgroup's partial (or, for a unit of one workgroup, of the
  // result).  The P scratch is reused; rows are padded so that the rows one
  // lane group apart fall in different LDS banks.
  constexpr int HDP = HD + 4;   // padded row stride (floats)
  constexpr int DS = HD / WV;   // dims merged by one wave
  float* xo = smem;                                               // [WV][QR][HDP]
  float2* xml = reinterpret_cast<float2*>(smem + WV * QR * HDP);  // [WV][QR]
  float* rl = reinterpret_cast<float*>(xml + WV * QR);            // [QR] merged sum
  float* rm = rl + QR;                                            // [QR] merged max
  float* wts = rm + QR;                                           // [WV][QR]
  __syncthreads();  // every wave is done with the P scratch
#pragma unroll
  for (int mt = 0; mt < MTQ; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mt * 16 + 4 * kq + r;
      if (row < nq) {
#pragma unroll
        for (int t = 0; t < NDT; ++t) xo[(wave * QR + row) * HDP + 16 * t + mrow] = oacc[mt][t][r];
        if (mrow == 0) xml[wave * QR + row] = make_float2(mrun[mt][r], lrun[mt][r]);
      }
    }
  __syncthreads();
  for (int row = threadIdx.x; row < nq; row += kThreads) {
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < WV; ++j) {
      const float2 v = xml[j * QR + row];
      if (v.y > 0.f) mx = fmaxf(mx, v.x);  // a partial that saw no key has sum 0
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
  __syncthreads();

  const size_t QG = a.qg_size;
  float* po = a.part;                                              // [units][wpb][QG][HD]
  uint64_t* pml = reinterpret_cast<uint64_t*>(a.part + a.ml_off);  // [units][wpb][QG] (max, sum)
  const size_t rec = (size_t)unit * wps + wgi;
  for (int e = lane; e < nq * DS; e += 64) {
    const int row = e / DS, d = wave * DS + e % DS;
    float o = 0.f;
#pragma unroll
    for (int j = 0; j < WV; ++j) o += wts[j * QR + row] * xo[(j * QR + row) * HDP + d];
    if (wpb == 1) {  // the only workgroup of its unit: write the result
      const int gq = q0 + row;
      xa_store(a.xa_o, (kvh * G + gq / nr) * HD + d, r0 + gq % nr, a.M, o / rl[row]);
    } else {
      __hip_atomic_store(po + (rec * QG + row) * HD + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (wpb == 1) return;
  if (threadIdx.x < nq) {
    const int row = threadIdx.x;
    const uint64_t b = (uint64_t)__float_as_uint(rm[row]) | ((uint64_t)__float_as_uint(rl[row]) << 32);
    __hip_atomic_store(pml + rec * QG + row, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The partial stores must have completed (written through to device
  // scope) before the workgroup is counted in.  A workgroup-scope fence does
  // not wait for stores on this target, so wait on the vector memory counter
  // itself (it counts stores too); the clobber keeps the compiler from
  // moving memory operations across the wait.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(a.cnt + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int is_last = old == (unsigned)(wpb - 1);
    if (is_last) __hip_atomic_store(a.cnt + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_wg = is_last;
  }
  __syncthreads();
  if (!last_wg) return;

  // ---- last workgroup of the unit: combine the wpb partials in workgroup
  // order.  Each row's weights exp2(m_j - max) and total are computed once in
  // LDS; a thread then sums one pair of dims of one query vector over the
  // partials, with the loads of up to kCB partials in flight at once (the
  // first batch is requested before the weights exist).
  constexpr int HP = HD / 2;  // dim pairs
  constexpr int kCG = 8;      // partials per guarded group
  constexpr int kCB = 16;     // partials requested per batch
  float2* cml = reinterpret_cast<float2*>(smem);  // [wpb][nq] (max, sum)
  float* cwt = smem + 2 * kAttnCombineSlots;      // [wpb][nq] weights
  float* ctot = cwt + kAttnCombineSlots;          // [nq]
  const uint64_t* src0 = reinterpret_cast<const uint64_t*>(po) + (size_t)unit * wps * QG * HP;
  const int S = (int)QG * HP;  // pairs between consecutive partials
  const int npair = nq * HP;
  uint64_t xc[kCB];
  auto load_batch = [&](int p, int j0) {
    const uint64_t* src = src0 + min(p, npair - 1);
#pragma unroll
    for (int g = 0; g < kCB / kCG; ++g)
      if (j0 + g * kCG < wpb) {
#pragma unroll
        for (int e = g * kCG; e < (g + 1) * kCG; ++e)
          xc[e] = __hip_atomic_load(src + min(j0 + e, wpb - 1) * S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  };
  if (threadIdx.x < npair) load_batch(threadIdx.x, 0);
  for (int e = threadIdx.x; e < wpb * nq; e += kThreads) {
    const int j = e / nq, r = e - j * nq;
    const uint64_t b = __hip_atomic_load(pml + ((size_t)unit * wps + j) * QG + r, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    cml[e] = make_float2(__uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nq; r += kThreads) {
    float mx = -INFINITY;
    for (int j = 0; j < wpb; ++j)
      if (cml[j * nq + r].y > 0.f) mx = fmaxf(mx, cml[j * nq + r].x);
    float tot = 0.f;
    for (int j = 0; j < wpb; ++j) {
      const float2 v = cml[j * nq + r];
      const float w = v.y > 0.f ? __builtin_amdgcn_exp2f(v.x - mx) : 0.f;
      cwt[j * nq + r] = w;
      tot += w * v.y;
    }
    ctot[r] = tot;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < npair; p += kThreads) {
    const int r = p / HP, c = p - r * HP;
    float o0 = 0.f, o1 = 0.f;
    for (int j0 = 0; j0 < wpb; j0 += kCB) {
      if (p != threadIdx.x || j0 > 0) load_batch(p, j0);
#pragma unroll
      for (int g = 0; g < kCB / kCG; ++g)
        if (j0 + g * kCG < wpb) {
#pragma unroll
          for (int e = g * kCG; e < (g + 1) * kCG; ++e) {
            const int j = j0 + e;
            const float w = j < wpb ? cwt[j * nq + r] : 0.f;
            o0 += w * __uint_as_float((uint32_t)xc[e]);
            o1 += w * __uint_as_float((uint32_t)(xc[e] >> 32));
          }
        }
    }
    const float tot = ctot[r];
    const int gq = q0 + r;
    const int m = r0 + gq % nr, h = kvh * G + gq / nr;
    xa_store(a.xa_o, h * HD + 2 * c, m, a.M, o0 / tot);
    xa_store(a.xa_o, h * HD + 2 * c + 1, m, a.M, o1 / tot);
  }
}

hipError_t attn_init() { return hipSuccess; }

void launch_attention(const AttnArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const int n_parts = a.n_split + 1;
  const int wv = attn_waves(a.qg_size);
  const int wpb = (n_parts + wv - 1) / wv;
  const int groups = a.rows.n_seq * wpb * a.Hkv;
  dim3 grid(a.map != nullptr ? a.map_n : 8 * a.n_qg * ((groups + 7) / 8));
  static_assert(kAttnQG <= 16, "one 16-row query tile per wave");
#define VS_ATT(MTQ, HD, WV)                                                                                 \
  do {                                                                                                      \
    if (ev0 != nullptr || ev1 != nullptr)                                                                   \
      hipExtLaunchKernelGGL((attn_kernel<MTQ, HD, WV>), grid, dim3(WV * 64), 0, st, ev0, ev1, 0, a);        \
    else                                                                                                    \
      hipLaunchKernelGGL((attn_kernel<MTQ, HD, WV>), grid, dim3(WV * 64), 0, st, a);                        \
  } while (0)
  if (a.hd == 128) VS_ATT(1, 128, 8);
  else VS_ATT(1, 64, 8);
#undef VS_ATT
}

}  // namespace vs
