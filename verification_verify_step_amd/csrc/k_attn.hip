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
// its own online softmax: no block barriers, no K/V staging.  Per 32-key
// step: S for two 16-key tiles (bf16 16x16x32 MFMA, the query split into bf16
// hi + lo parts so scores keep fp32 precision), masking, softmax update in
// fp32, P through a small per-wave LDS scratch into A-operand order (again
// split hi/lo), then O += P.V.  The next step's K/V loads are in flight while
// the current one computes.  Each split writes (max, sum, unnormalised o); a
// second kernel combines the splits in a fixed order and writes the result
// as split-bf16 activation fragments for the O projection.
#include "kernels.h"

namespace vs {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kStep = 32;           // keys per step
constexpr int kCombineMax = 1024;   // splits combined by one workgroup

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// 8 floats -> bf16 hi and lo parts, packed as two MFMA operand registers.
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h0 = f2bf(x[2 * e]), h1 = f2bf(x[2 * e + 1]);
    const uint16_t l0 = f2bf(x[2 * e] - bf2f(h0)), l1 = f2bf(x[2 * e + 1] - bf2f(h1));
    h[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

template <int MTQ, int HD>
__global__ __launch_bounds__(kThreads) void attn_kernel(const AttnArgs a) {
  constexpr int KSQ = HD / 32;  // k-steps of S over head dims
  constexpr int NDT = HD / 16;  // 16-dim output tiles
  constexpr int QR = MTQ * 16;
  constexpr int PS = kStep + 4;  // P scratch row stride (floats)
  __shared__ float Pl[kWaves][QR * PS];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_parts = a.n_split + 1;
  const int wpb = (n_parts + kWaves - 1) / kWaves;  // workgroups per (sequence, kv head, query group)
  const int i = blockIdx.x / wpb;
  const int split = (blockIdx.x % wpb) * kWaves + wave;
  if (split >= n_parts) return;  // whole wave; no block-level barriers below
  const int kvh = blockIdx.y, qg = blockIdx.z;
  const int sq = a.rows.seq[i];
  const int r0 = a.rows.row_start[i];
  const int nr = a.rows.row_start[i + 1] - r0;
  const int G = a.H / a.Hkv;
  const int q0 = qg * a.qg_size;
  const int nq = max(0, min(a.qg_size, nr * G - q0));
  const int P = a.kv.P[sq];
  const int W = a.rows.idx_off + nr;  // in-round keys present: window indices 0..W-1
  const bool window = split == a.n_split;
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

  // query fragments (A operand of S), pre-scaled and split hi/lo
  u32x4 qh[MTQ][KSQ], ql[MTQ][KSQ];
  uint64_t qmask[MTQ][4];  // visibility masks of the 4 rows this lane holds in S
#pragma unroll
  for (int mt = 0; mt < MTQ; ++mt) {
    const int qv = mt * 16 + mrow;
    const int gq = q0 + min(qv, max(nq - 1, 0));
    const float* src = a.q + ((size_t)(r0 + gq % nr) * a.H + kvh * G + gq / nr) * HD;
#pragma unroll
    for (int s = 0; s < KSQ; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = qv < nq ? src[32 * s + 8 * kq + e] * a.scale : 0.f;
      split8(x, qh[mt][s], ql[mt][s]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mt * 16 + 4 * kq + r;
      uint64_t mk = 0;
      if (row < nq) {
        const int rl = (q0 + row) % nr;
        const int idx = a.rows.idx_off + rl;
        mk = a.rows.mask ? a.rows.mask[r0 + rl] : (idx >= 63 ? ~0ull : ((2ull << idx) - 1ull));
      }
      qmask[mt][r] = mk;
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

  // Steps of 32 keys aligned to blocks: [base, base+32) covers slots of two
  // blocks.  A committed split's steps and block-table entries follow from
  // the split index alone (P only masks), so its first K/V loads do not wait
  // for P.  K of the next step is requested right after this step's S, V of
  // the next step right after this step's P.V.
  const int first = window ? (key_lo / kStep) * kStep : split * a.kps;
  const int last = window ? key_hi : split * a.kps + a.kps;  // exclusive
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
  float* pw = Pl[wave];
  blocks_of(first);
  load_k();
  load_v();
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
    // mask, online softmax update, P into the scratch (row, key) layout
#pragma unroll
    for (int mt = 0; mt < MTQ; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = mt * 16 + 4 * kq + r;
        float v[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int slot = base + 16 * t + mrow;
          bool vis = slot >= key_lo && slot < key_hi;
          if (vis && window) vis = (qmask[mt][r] >> (slot - key_lo)) & 1ull;
          v[t] = vis ? sacc[mt][t][r] : -INFINITY;
        }
        float mx = fmaxf(v[0], v[1]);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        const float mnew = fmaxf(mrun[mt][r], mx);
        const float corr = (mrun[mt][r] == -INFINITY) ? 0.f : expf(mrun[mt][r] - mnew);
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float p = v[t] == -INFINITY ? 0.f : expf(v[t] - mnew);
          pw[row * PS + 16 * t + mrow] = p;
          ps += p;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o, 64);
        lrun[mt][r] = lrun[mt][r] * corr + ps;
        mrun[mt][r] = mnew;
#pragma unroll
        for (int t = 0; t < NDT; ++t) oacc[mt][t][r] *= corr;
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

  // partials: lane holds rows 16mt + 4(lane/16) + r, dims 16t + lane%16
  const int unit = (i * a.Hkv + kvh) * a.n_qg + qg;
  const size_t rec = (size_t)HD + 2;
  float* part = a.part + ((size_t)unit * n_parts + split) * a.qg_size * rec;
#pragma unroll
  for (int mt = 0; mt < MTQ; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mt * 16 + 4 * kq + r;
      if (row < nq) {
        float* pp = part + (size_t)row * rec;
        if (mrow == 0) {
          pp[0] = mrun[mt][r];
          pp[1] = lrun[mt][r];
        }
#pragma unroll
        for (int t = 0; t < NDT; ++t) pp[2 + 16 * t + mrow] = oacc[mt][t][r];
      }
    }
}

// Combines the split partials of one query vector of one (sequence, KV head,
// query group): workgroup = (unit, query vector), thread = head dim.  The
// (max, sum) of every split go through LDS, then each thread sums its dim
// over the splits in split order with all loads issued up front.
constexpr int kCombineThreads = 128;
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(const AttnArgs a) {
  __shared__ float mls[kCombineMax], wts[kCombineMax];
  const int unit = blockIdx.x, qv = blockIdx.y;
  const int qg = unit % a.n_qg;
  const int kvh = (unit / a.n_qg) % a.Hkv;
  const int i = unit / (a.n_qg * a.Hkv);
  const int hd = a.hd, QG = a.qg_size;
  const int r0 = a.rows.row_start[i];
  const int nr = a.rows.row_start[i + 1] - r0;
  const int G = a.H / a.Hkv;
  const int q0 = qg * QG;
  const int nq = max(0, min(QG, nr * G - q0));
  if (qv >= nq) return;  // whole workgroup
  const int n_parts = a.n_split + 1;
  const size_t rec = (size_t)hd + 2, stride = (size_t)QG * rec;
  const float* base = a.part + (size_t)unit * n_parts * stride + (size_t)qv * rec;
  // the (max, sum) of every split and this thread's first block of o values
  // are requested in the same round
  constexpr int kB = 32;
  const int dd = threadIdx.x;
  const float* pp = base + 2 + min(dd, hd - 1);
  float x[kB];
#pragma unroll
  for (int e = 0; e < kB; ++e) x[e] = e < n_parts ? pp[(size_t)e * stride] : 0.f;
  for (int sp = threadIdx.x; sp < n_parts; sp += kCombineThreads) {
    mls[sp] = base[sp * stride];
    wts[sp] = base[sp * stride + 1];
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int sp = 0; sp < n_parts; ++sp)
    if (wts[sp] > 0.f) mx = fmaxf(mx, mls[sp]);
  float tot = 0.f;
  for (int sp = 0; sp < n_parts; ++sp)
    if (wts[sp] > 0.f) tot += wts[sp] * expf(mls[sp] - mx);
  float o = 0.f;
  for (int b = 0; b < n_parts; b += kB) {  // splits summed in order
    if (b > 0) {
#pragma unroll
      for (int e = 0; e < kB; ++e) x[e] = b + e < n_parts ? pp[(size_t)(b + e) * stride] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kB; ++e)
      if (b + e < n_parts && wts[b + e] > 0.f) o += x[e] * expf(mls[b + e] - mx);
  }
  if (dd < hd) {
    const int gq = q0 + qv;
    const int m = r0 + gq % nr, h = kvh * G + gq / nr;
    xa_store(a.xa_o, h * hd + dd, m, a.M, o / tot);
  }
}

hipError_t attn_init() { return hipSuccess; }

void launch_attention(const AttnArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const int n_parts = a.n_split + 1;
  const int wpb = (n_parts + kWaves - 1) / kWaves;
  dim3 grid(a.rows.n_seq * wpb, a.Hkv, a.n_qg);
  const int mtq = (a.qg_size + 15) / 16;  // at most 2 (query groups hold <= kAttnQG vectors)
#define VS_ATT(MTQ, HD)                                                                                     \
  do {                                                                                                      \
    if (ev0 != nullptr)                                                                                     \
      hipExtLaunchKernelGGL((attn_kernel<MTQ, HD>), grid, dim3(kThreads), 0, st, ev0, nullptr, 0, a);       \
    else                                                                                                    \
      hipLaunchKernelGGL((attn_kernel<MTQ, HD>), grid, dim3(kThreads), 0, st, a);                           \
  } while (0)
  if (a.hd == 128) {
    if (mtq <= 1) VS_ATT(1, 128);
    else VS_ATT(2, 128);
  } else {
    if (mtq <= 1) VS_ATT(1, 64);
    else VS_ATT(2, 64);
  }
#undef VS_ATT
  const dim3 cgrid(a.rows.n_seq * a.Hkv * a.n_qg, a.qg_size);
  if (ev1 != nullptr)
    hipExtLaunchKernelGGL(attn_combine_kernel, cgrid, dim3(kCombineThreads), 0, st, nullptr, ev1, 0, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel, cgrid, dim3(kCombineThreads), 0, st, a);
}

}  // namespace vs
