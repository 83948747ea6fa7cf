// Masked multi-query attention with the K/V of a step shared by the query
// groups of a KV head (gfx950).
//
// What is computed is the same as in k_attn.hip ("FlashSpec" page,
// lnrk.cn/news/47842, §2.2: every row attends to the committed keys of its
// sequence and to the in-round keys its ancestor mask selects; §5.2: nothing
// outside the mask may leak).  The work is cut differently.  k_attn.hip gives
// each wave its own key range of one query group, so when a KV head has many
// query vectors (GQA heads, or the 64 rows of a token tree) every group reads
// the same K/V again.  Here a workgroup owns one key range (split) of one KV
// head and up to WV query groups, one per wave (WV = 4: three workgroups
// per CU, so that one's pipeline start and waits overlap the others' steps):
//
//  * the workgroup's threads load each 32-key step (two 16-key blocks of K
//    and of V, 16 KB at head_dim 128) in 16-byte pieces, kDepth = 2 steps
//    ahead in registers (a ring short enough for three waves per SIMD), and put a step into one of two LDS stages (K rows padded
//    by 16 bytes so the fragment reads of one MFMA do not collide in a bank);
//  * every wave then computes its group's step transposed, S^T = K.Q^T on
//    the bf16 16x16x32 MFMA (query split hi/lo), so that a lane holds eight
//    scores of one query: masking and the base-2 online softmax reduce them
//    in the lane and then across the four lane groups, and the
//    probabilities (split hi/lo) are directly the B operand of
//    O^T += V^T.P^T, with no trip through LDS;
//  * one barrier per step (LDS counter only: loads stay in flight across it).
//
// A sequence's committed keys are cut into splits of kps keys; its last split
// also takes the in-round keys, so a sequence with one split needs no merge
// and its workgroups write the result.  Otherwise each wave writes its (max,
// sum, o) partial and attn_group_combine merges the splits of each query
// group in split order.
#include "attn_dev.h"
#include "attn_group.h"

namespace vs {

namespace {

// This wave's LDS writes are done, then the workgroup barrier.  Unlike
// __syncthreads() it does not wait for global loads, so the steps loaded
// ahead stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace

template <int HD, int WV>
// At least three waves per SIMD: the register budget (168 per lane) that
// lets three workgroups share a CU, which measured faster than a deeper ring
// at two (the 70B batch 255 against 310 us per launch pair, the 64-row tree
// 35.5 against 39.5).
__global__ __launch_bounds__(WV * 64, 3) void attn_group_kernel(const AttnArgs a) {
  constexpr int kThreads = WV * 64;
  constexpr int KSQ = HD / 32;        // k-steps of S over head dims
  constexpr int NDT = HD / 16;        // 16-dim output tiles
  constexpr int KROW = HD + 8;        // padded K row in LDS (elements)
  constexpr int KPART = 2 * kBlock * KROW;
  constexpr int STAGE = KPART + 2 * kBlock * HD;  // one step: K (padded rows), then V as in HBM
  constexpr int PIECES = 8 * HD;                  // 16-byte pieces of one step's K and V
  constexpr int PPT = PIECES / kThreads;
  static_assert(PPT >= 1 && PPT * kThreads == PIECES, "pieces per thread");
  constexpr int kDepth = 2;  // steps loaded ahead of the one in LDS (even: the loop alternates the two stages)
  __shared__ __attribute__((aligned(16))) uint16_t stg[2 * STAGE];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x;  // the grid is exactly the pass's wg_start[n_seq] workgroups
  // Memory round trips before the first step: (1) every per-sequence field
  // of the arguments at once, lane l holding sequence l's, the workgroup's
  // sequence being the last whose first workgroup is <= b; (2) P, the
  // split's block-table entries, the query vector and its mask together;
  // (3) the ring of K/V steps.
  const int ls = min(lane, kMaxSeq - 1);
  const int ws_l = a.wg_start[ls], sq_l = a.rows.seq[ls], r0_l = a.rows.row_start[ls];
  const int r1_l = a.rows.row_start[ls + 1], nsp_l = a.nsplit[ls];
  const int i = __popcll(__ballot(lane < a.rows.n_seq && ws_l <= b)) - 1;
  const int sq = __builtin_amdgcn_readlane(sq_l, i);
  const int r0 = __builtin_amdgcn_readlane(r0_l, i);
  const int nr = __builtin_amdgcn_readlane(r1_l, i) - r0;
  const int G = a.H / a.Hkv;
  const int nqb = ((nr * G + a.qg_size - 1) / a.qg_size + WV - 1) / WV;
  const int l = b - __builtin_amdgcn_readlane(ws_l, i), t8 = l / kAttnXcds;
  const int g = (t8 / nqb) * kAttnXcds + l % kAttnXcds, qb = t8 % nqb;
  const int ns_ub = __builtin_amdgcn_readlane(nsp_l, i);
  if (g >= a.Hkv * ns_ub) return;  // padding of the group count to the XCDs
  const int s = g / a.Hkv, kvh = g - s * a.Hkv;  // splits in order, KV heads fastest: unneeded splits come last
  const int qg = qb * WV + wave;
  const int q0 = qg * a.qg_size;
  const int nq = qg < a.n_qg ? max(0, min(a.qg_size, nr * G - q0)) : 0;  // this wave's query vectors
  // A split's steps start at clo = s * kps: a committed split's keys do,
  // and the last split's in-round keys start at P + win >= clo.
  const int clo = s * a.kps;
  const int* bt = a.kv.bt + (size_t)sq * a.kv.bps;

  // (2): P, the block-table entries of the split, one per lane (two per
  // step), this lane's query vector (query mrow of the wave's group, vector
  // gq mapping to row r0 + gq % nr and head kvh*G + gq / nr) and its mask
  // (the pass's if it has them, else read from the query buffer and not
  // used: a load under a branch would make the compiler wait for every load
  // in flight where the branch joins).
  const int P = a.kv.P[sq];
  const int btreg = bt[min(clo / kBlock + lane, a.kv.bps - 1)];
  const int mrow = lane & 15, kq = lane >> 4;
  const bool qok = mrow < nq;
  const int gq = min(q0 + min(mrow, max(nq, 1) - 1), nr * G - 1);
  float4 qraw[KSQ][2];
  uint64_t mraw;
  {
    const float* src = a.q + ((size_t)(r0 + gq % nr) * a.H + kvh * G + gq / nr) * HD;
#pragma unroll
    for (int s2 = 0; s2 < KSQ; ++s2) {
      qraw[s2][0] = *reinterpret_cast<const float4*>(src + 32 * s2 + 8 * kq);
      qraw[s2][1] = *reinterpret_cast<const float4*>(src + 32 * s2 + 8 * kq + 4);
    }
    const uint64_t* const mbase =
        a.rows.mask != nullptr ? a.rows.mask + r0 : reinterpret_cast<const uint64_t*>(a.q);
    mraw = mbase[gq % nr];
  }
  // every request above is issued before the branch on P below
  asm volatile("" ::: "memory");

  const int ns = min(max(1, (P + a.kps - 1) / a.kps), ns_ub);  // this sequence's splits (P <= the host's bound)
  if (s >= ns) return;  // past what its context needs
  const bool last_split = s == ns - 1;
  const int wlo = P + a.rows.win, whi = wlo + a.rows.idx_off + nr;  // in-round keys
  const int chi = min(P, clo + a.kps);                             // committed keys of this split
  const int first = clo;
  const int last = last_split ? (whi + kStep - 1) / kStep * kStep : min(clo + a.kps, (P + kStep - 1) / kStep * kStep);
  // both ends are step-aligned; the host keeps a split within kAttnGroupSteps
  const int n_steps = min(last > first ? (last - first) / kStep : 0, kAttnGroupSteps);

  const uint16_t* const kpool = a.kv.k;
  const uint16_t* const vpool = a.kv.v;
  __builtin_assume(threadIdx.x < kThreads);

  // piece x of a step: K (x < 4 HD) or V, block (x / 2 HD) % 2, 16-byte
  // offset x % 2 HD inside that block's tile (K: [HD/8][16][8], V: [HD][16])
  auto load_step = [&](int t, u32x4(&r)[PPT]) {
    const int nb0 = __builtin_amdgcn_readlane(btreg, 2 * t);
    const int nb1 = __builtin_amdgcn_readlane(btreg, 2 * t + 1);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int x = threadIdx.x + j * kThreads;
      const int isv = x / (4 * HD), blk = (x / (2 * HD)) & 1, off = x % (2 * HD);
      const uint16_t* src = (isv ? vpool : kpool) + kv_tile(blk ? nb1 : nb0, kvh, a.Hkv, HD);
      r[j] = reinterpret_cast<const u32x4*>(src)[off];
    }
  };
  auto put_step = [&](const u32x4(&r)[PPT], int sb) {
    uint16_t* d = stg + sb * STAGE;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int x = threadIdx.x + j * kThreads;
      const int isv = x / (4 * HD), blk = (x / (2 * HD)) & 1, off = x % (2 * HD);
      uint16_t* dst = isv ? d + KPART + blk * kBlock * HD + off * 8
                          : d + (blk * kBlock + off % kBlock) * KROW + (off / kBlock) * 8;
      *reinterpret_cast<u32x4*>(dst) = r[j];
    }
  };

  // Every thread issues the same loads on every path (steps past the
  // split's end re-read its last step, a wave without queries reads a valid
  // query row), so that the compiler's wait counts stay exact and the ring's
  // steps remain in flight across iterations.
  const int t_end = max(n_steps - 1, 0);
  u32x4 ring[kDepth][PPT];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_step(min(d, t_end), ring[d]);

  // this lane's visibility mask over the in-round keys
  uint64_t qmask;
  {
    const int idx = a.rows.idx_off + gq % nr;
    const uint64_t mk = a.rows.mask != nullptr ? mraw : (idx >= 63 ? ~0ull : ((2ull << idx) - 1ull));
    qmask = qok ? mk : 0ull;
  }

  // query fragments (the B operand of S^T), pre-scaled into base-2 units and
  // split hi/lo
  const float qscale = a.scale * 1.4426950408889634f;
  u32x4 qh[KSQ], ql[KSQ];
#pragma unroll
  for (int s2 = 0; s2 < KSQ; ++s2) {
    const float4 u = qraw[s2][0], v = qraw[s2][1];
    const float x[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = qok ? x[k] * qscale : 0.f;
    split8(y, qh[s2], ql[s2]);
  }

  // Online softmax of this lane's query; O^T tile t3 holds dims
  // 16 t3 + 4 kq + r of it.
  float mrun = -INFINITY, lrun = 0.f;
  f32x4 oacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One step, computed transposed: S^T = K.Q^T puts keys 4 kq + r of block
  // t2 of the lane's query in its registers, so that the softmax reduces
  // eight values in the lane and then across the four lane groups, and the
  // probabilities are already the B operand of O^T += V^T.P^T (their k order
  // is block-major by lane group: k = 8 kq + j is key 4 kq + j % 4 of block
  // j / 4; V^T is read from LDS in the same order).
  auto compute = [&](int t, int sb) {
    const int base = first + t * kStep;
    const uint16_t* kst = stg + sb * STAGE;
    const uint16_t* vst = kst + KPART;
    f32x4 sacc[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < KSQ; ++s2) {
        const u32x4 kb = *reinterpret_cast<const u32x4*>(kst + (t2 * kBlock + mrow) * KROW + 32 * s2 + 8 * kq);
        c = mfma16(kb, qh[s2], c);
        c = mfma16(kb, ql[s2], c);
      }
      sacc[t2] = c;
    }
    // a step of committed keys only, all inside this split: no masking
    const bool full = base >= clo && base + kStep <= chi;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t2 = j >> 2, r = j & 3;
      if (full) {
        v[j] = sacc[t2][r];
      } else {
        // branch-free, and the shift count kept in 0..63: a count outside
        // it is undefined and lets the compiler drop the whole term
        const int slot = base + 16 * t2 + 4 * kq + r, wo = slot - wlo;
        const bool inwin = last_split & (wo >= 0) & (slot < whi);
        const bool vis = ((slot >= clo) & (slot < chi)) | (inwin & (((qmask >> (wo & 63)) & 1ull) != 0));
        v[j] = vis ? sacc[t2][r] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(mrun, mx);
    const float corr = (mrun == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun - mnew);
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = v[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(v[j] - mnew);
    // the four lanes of a query add the same values in the same pairs
    float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    lrun = lrun * corr + ps;
    mrun = mnew;
    // rescale the accumulators unless every factor is exactly 1 (no new max)
    if (!__all(corr == 1.f)) {
#pragma unroll
      for (int t3 = 0; t3 < NDT; ++t3) oacc[t3] *= corr;
    }
    u32x4 ph, pl;
    split8(p, ph, pl);
#pragma unroll
    for (int t3 = 0; t3 < NDT; ++t3) {
      const uint16_t* vr = vst + (16 * t3 + mrow) * kBlock + 4 * kq;
      const uint2 v0 = *reinterpret_cast<const uint2*>(vr);                   // block 0
      const uint2 v1 = *reinterpret_cast<const uint2*>(vr + kBlock * HD);     // block 1
      const u32x4 va = u32x4{v0.x, v0.y, v1.x, v1.y};
      oacc[t3] = mfma16(va, ph, oacc[t3]);
      oacc[t3] = mfma16(va, pl, oacc[t3]);
    }
  };

  // Step t is computed from LDS stage t % 2 while the ring holds steps
  // t+1 .. t+kDepth; after it, step t+1 moves into the other stage and its
  // ring slot takes step t+1+kDepth.  The loop is unrolled by kDepth so that
  // ring slots are registers.
  put_step(ring[0], 0);
  load_step(min(kDepth, t_end), ring[0]);
  lds_barrier();
  for (int t0 = 0; t0 < n_steps; t0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int t = t0 + u;
      if (t < n_steps && nq > 0) compute(t, u & 1);
      put_step(ring[(u + 1) % kDepth], (u + 1) & 1);
      load_step(min(t + 1 + kDepth, t_end), ring[(u + 1) % kDepth]);
      lds_barrier();
    }
  }
  if (!qok) return;

  const int unit = (i * a.Hkv + kvh) * a.n_qg + qg;
  if (ns == 1) {  // the only split: write the result
    const int m = r0 + gq % nr, h = kvh * G + gq / nr;
#pragma unroll
    for (int t3 = 0; t3 < NDT; ++t3)
#pragma unroll
      for (int r = 0; r < 4; ++r) xa_store(a.xa_o, h * HD + 16 * t3 + 4 * kq + r, m, a.M, oacc[t3][r] / lrun);
    return;
  }
  const size_t QG = a.qg_size;
  const size_t rec = (size_t)unit * a.n_split + s;
  float* po = a.part + (rec * QG + mrow) * HD + 4 * kq;
#pragma unroll
  for (int t3 = 0; t3 < NDT; ++t3) *reinterpret_cast<float4*>(po + 16 * t3) = make_float4(oacc[t3][0], oacc[t3][1], oacc[t3][2], oacc[t3][3]);
  if (kq == 0) reinterpret_cast<float2*>(a.part + a.ml_off)[rec * QG + mrow] = make_float2(mrun, lrun);
}

// Merge of the splits, for sequences with more than one.  A workgroup of 4
// waves takes 4 query vectors of one (sequence, KV head, query group); wave
// w merges vector w.  Its requests go out at once, beside P: the (max, sum)
// record of split `lane` and the lane's pair of dims of the first 16 splits,
// for every split of the host's bound (>= the device's count; the records
// past the device's are read but never used).  Lane j's weight
// exp2(m_j - max) reaches the other lanes by shuffles, and each lane sums
// its pair over the splits in split order.
template <int HD>
__global__ __launch_bounds__(256) void attn_group_combine(const AttnArgs a) {
  static_assert(kAttnGroupMaxSplits <= 64, "one split per lane");
  constexpr int HP = HD / 2;  // dim pairs
  static_assert(HP <= 64, "one pair per lane");
  constexpr int kB = 16;      // splits whose pairs are requested with the records
  const int quarters = (a.qg_size + 3) / 4;
  const int unit = blockIdx.x / quarters, v0 = (blockIdx.x % quarters) * 4;
  const int qg = unit % a.n_qg, ik = unit / a.n_qg, kvh = ik % a.Hkv, i = ik / a.Hkv;
  const int nsb = a.nsplit[i];
  if (nsb <= 1) return;  // one split: written by the main kernel
  const int r0 = a.rows.row_start[i];
  const int nr = a.rows.row_start[i + 1] - r0;
  const int G = a.H / a.Hkv;
  const int q0 = qg * a.qg_size;
  const int nq = max(0, min(a.qg_size, nr * G - q0));
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int v = v0 + wave;
  if (v >= nq) return;  // this wave's vector is past the group's
  const size_t QG = a.qg_size, rec0 = (size_t)unit * a.n_split;
  const int P = a.kv.P[a.rows.seq[i]];
  const float2 mlr = lane < nsb ? reinterpret_cast<const float2*>(a.part + a.ml_off)[(rec0 + lane) * QG + v]
                                : make_float2(-INFINITY, 0.f);
  const int c = min(lane, HP - 1);
  const float* base = a.part + __builtin_amdgcn_readfirstlane((int)((rec0 * QG + v) * HD));
  const float* src = base + 2 * c;
  const size_t stride = QG * HD;  // floats between consecutive splits
  // The first kB splits' pairs through a buffer resource whose extent ends at
  // split nsb: a load past it returns zeros without touching memory, so the
  // requests go out together, unbranched, and fetch only the bound's splits.
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, __builtin_amdgcn_readfirstlane((int)(nsb * stride * sizeof(float))), kRawBufferWord3);
  float2 x[kB];
#pragma unroll
  for (int e = 0; e < kB; ++e) {
    const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(rs, 8 * c + e * (int)(stride * sizeof(float)), 0, 0);
    x[e] = make_float2(__uint_as_float(w2[0]), __uint_as_float(w2[1]));
  }
  asm volatile("" ::: "memory");  // keep the requests above the P-dependent exit
  const int ns = min(max(1, (P + a.kps - 1) / a.kps), nsb);
  if (ns <= 1) return;  // one split on the device: written by the main kernel
  const float2 ml = lane < ns ? mlr : make_float2(-INFINITY, 0.f);
  const float mx = wave_max(ml.y > 0.f ? ml.x : -INFINITY);  // a split that saw no key has sum 0
  const float w = ml.y > 0.f ? __builtin_amdgcn_exp2f(ml.x - mx) : 0.f;
  const float t = wave_sum(w * ml.y);
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int e = 0; e < kB; ++e) {
    const float we = __shfl(w, e, 64);
    if (e < ns) {
      o0 += we * x[e].x;
      o1 += we * x[e].y;
    }
  }
  for (int j = kB; j < ns; ++j) {  // past the first kB splits (the tree's 17)
    const float2 xj = *reinterpret_cast<const float2*>(src + (size_t)j * stride);
    const float wj = __shfl(w, j, 64);
    o0 += wj * xj.x;
    o1 += wj * xj.y;
  }
  if (lane >= HP) return;
  const int gq = q0 + v;
  const int m = r0 + gq % nr, h = kvh * G + gq / nr;
  xa_store(a.xa_o, h * HD + 2 * c, m, a.M, o0 / t);
  xa_store(a.xa_o, h * HD + 2 * c + 1, m, a.M, o1 / t);
}

void launch_attention_group(const AttnArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const bool combine = a.n_split > 1;
  const dim3 grid(a.wg_start[a.rows.n_seq]), cgrid(a.rows.n_seq * a.Hkv * a.n_qg * ((a.qg_size + 3) / 4));
  hipEvent_t e1 = combine ? nullptr : ev1;
#define VS_GRP(HD, WV)                                                                                         \
  do {                                                                                                         \
    if (ev0 != nullptr || e1 != nullptr)                                                                       \
      hipExtLaunchKernelGGL((attn_group_kernel<HD, WV>), grid, dim3(WV * 64), 0, st, ev0, e1, 0, a);           \
    else                                                                                                       \
      hipLaunchKernelGGL((attn_group_kernel<HD, WV>), grid, dim3(WV * 64), 0, st, a);                          \
    if (combine) {                                                                                             \
      if (ev1 != nullptr)                                                                                      \
        hipExtLaunchKernelGGL((attn_group_combine<HD>), cgrid, dim3(256), 0, st, nullptr, ev1, 0, a);          \
      else                                                                                                     \
        hipLaunchKernelGGL((attn_group_combine<HD>), cgrid, dim3(256), 0, st, a);                              \
    }                                                                                                          \
  } while (0)
  if (a.hd == 128) VS_GRP(128, kAttnGroupWaves);
  else VS_GRP(64, kAttnGroupWaves);
#undef VS_GRP
}

}  // namespace vs
