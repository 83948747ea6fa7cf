// Masked multi-query attention over the paged KV cache (gfx950).
//
// A verify pass has a few rows per sequence (k+1 chain positions or up to 64
// tree nodes); each row attends to every committed key of its sequence plus
// the in-round keys its ancestor mask selects ("FlashSpec" page,
// lnrk.cn/news/47842, §2.2: level-order tree batch with a parent mask; §5.2:
// nothing outside the mask may leak).  All query rows and grouped heads of a
// KV head share one read of each K/V tile.
//
// Work split: workgroup = (sequence, split of the committed keys or the
// in-round window, KV head, query group).  64-key tiles of K and V are staged
// in LDS with coalesced 16-byte loads; lane = key for the scores, lane =
// dimension pair for P.V; online softmax across tiles.  Each workgroup writes
// (max, sum, unnormalised o) partials; the last workgroup of a (sequence, KV
// head, query group) to finish combines the splits in a fixed order and
// writes the result as split-bf16 activation fragments for the O projection.
#include "kernels.h"

namespace vs {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void attn_kernel(const AttnArgs a) {
  extern __shared__ float smem[];
  const int hd = a.hd, hw = hd / 2;       // dims, 32-bit words per bf16 row
  const int ks = hw + 1;                  // padded K row stride in words
  const int QG = a.qg_size;
  float* Q = smem;                          // [QG][hd]
  float* Pm = Q + QG * hd;                  // [QG][64]
  uint32_t* Kl = reinterpret_cast<uint32_t*>(Pm + QG * kChunk);  // [64][ks]
  uint32_t* Vl = Kl + kChunk * ks;          // [64][hw]

  const int n_parts = a.n_split + 1;
  const int i = blockIdx.x / n_parts;
  const int split = blockIdx.x % n_parts;
  const int kvh = blockIdx.y, qg = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int sq = a.rows.seq[i];
  const int r0 = a.rows.row_start[i];
  const int nr = a.rows.row_start[i + 1] - r0;
  const int G = a.H / a.Hkv;
  const int nq_total = nr * G;
  const int q0 = qg * QG;
  const int nq = max(0, min(QG, nq_total - q0));
  const int P = a.kv.P[sq];
  const int W = a.rows.idx_off + nr;  // in-round keys present: indices 0..W-1

  int key_lo, key_hi;  // slot range of this split
  if (split < a.n_split) {
    key_lo = split * a.kps;
    key_hi = min(P, key_lo + a.kps);
  } else {
    key_lo = P + a.rows.win;
    key_hi = key_lo + W;
  }
  const bool window = split == a.n_split;

  // queries of this group, pre-scaled
  for (int e = tid; e < nq * hd; e += kThreads) {
    const int qv = e / hd, dd = e % hd;
    const int gq = q0 + qv;
    const int m = r0 + gq % nr, h = kvh * G + gq / nr;
    Q[qv * hd + dd] = a.q[((size_t)m * a.H + h) * hd + dd] * a.scale;
  }

  // per-wave online-softmax state for its query vectors qv = wave + 4j
  constexpr int kMaxQW = 16;
  float mrun[kMaxQW], lrun[kMaxQW], o0[kMaxQW], o1[kMaxQW];
#pragma unroll
  for (int j = 0; j < kMaxQW; ++j) {
    mrun[j] = -INFINITY;
    lrun[j] = 0.f;
    o0[j] = 0.f;
    o1[j] = 0.f;
  }
  uint64_t rowmask[kMaxQW];
#pragma unroll
  for (int j = 0; j < kMaxQW; ++j) {
    const int qv = wave + 4 * j;
    uint64_t mk = 0;
    if (qv < nq) {
      const int rl = (q0 + qv) % nr;
      const int idx = a.rows.idx_off + rl;
      mk = a.rows.mask ? a.rows.mask[r0 + rl] : (idx >= 63 ? ~0ull : ((2ull << idx) - 1ull));
    }
    rowmask[j] = mk;
  }

  const int pieces = hd / 8;  // 16-byte pieces per key row
  for (int k0 = key_lo; k0 < key_hi; k0 += kChunk) {
    const int nk = min(kChunk, key_hi - k0);
    __syncthreads();
    for (int pc = tid; pc < kChunk * pieces; pc += kThreads) {
      const int key = pc / pieces, part = pc % pieces;
      uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
      if (key < nk) {
        const int slot = k0 + key;
        const int blk = a.kv.bt[sq * a.kv.bps + slot / kBlock];
        const size_t off = (((size_t)blk * a.Hkv + kvh) * kBlock + (slot % kBlock)) * hd + part * 8;
        kv4 = *reinterpret_cast<const uint4*>(a.kv.k + off);
        vv4 = *reinterpret_cast<const uint4*>(a.kv.v + off);
      }
      uint32_t* kd = Kl + key * ks + part * 4;
      kd[0] = kv4.x; kd[1] = kv4.y; kd[2] = kv4.z; kd[3] = kv4.w;
      uint32_t* vd = Vl + key * hw + part * 4;
      vd[0] = vv4.x; vd[1] = vv4.y; vd[2] = vv4.z; vd[3] = vv4.w;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxQW; ++j) {
      const int qv = wave + 4 * j;
      if (qv >= nq) break;
      // scores: lane = key
      float s = -INFINITY;
      bool vis = lane < nk;
      if (vis && window) vis = (rowmask[j] >> (k0 - key_lo + lane)) & 1ull;
      if (vis) {
        const float* qq = Q + qv * hd;
        const uint32_t* kr = Kl + lane * ks;
        float acc = 0.f;
        for (int w2 = 0; w2 < hw; ++w2) {
          const uint32_t kw = kr[w2];
          acc = fmaf(qq[2 * w2], bf_lo(kw), acc);
          acc = fmaf(qq[2 * w2 + 1], bf_hi(kw), acc);
        }
        s = acc;
      }
      const float mt = wave_max(s);
      const float mnew = fmaxf(mrun[j], mt);
      float p = 0.f, corr = 1.f;
      if (mnew != -INFINITY) {
        p = vis ? expf(s - mnew) : 0.f;
        corr = (mrun[j] == -INFINITY) ? 0.f : expf(mrun[j] - mnew);
      }
      lrun[j] = lrun[j] * corr + wave_sum(p);
      mrun[j] = mnew;
      Pm[qv * kChunk + lane] = p;
      o0[j] *= corr;
      o1[j] *= corr;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxQW; ++j) {
      const int qv = wave + 4 * j;
      if (qv >= nq) break;
      if (lane < hw) {
        const float* pr = Pm + qv * kChunk;
        float a0 = o0[j], a1 = o1[j];
        for (int key = 0; key < nk; ++key) {
          const float pk = pr[key];
          const uint32_t vw = Vl[key * hw + lane];
          a0 = fmaf(pk, bf_lo(vw), a0);
          a1 = fmaf(pk, bf_hi(vw), a1);
        }
        o0[j] = a0;
        o1[j] = a1;
      }
    }
  }

  // ---- partials ----
  const int unit = (i * a.Hkv + kvh) * a.n_qg + qg;
  const size_t rec = (size_t)hd + 2;
  float* part = a.part + ((size_t)unit * n_parts + split) * QG * rec;
#pragma unroll
  for (int j = 0; j < kMaxQW; ++j) {
    const int qv = wave + 4 * j;
    if (qv >= nq) break;
    float* pp = part + (size_t)qv * rec;
    if (lane < hw) {
      pp[2 + 2 * lane] = o0[j];
      pp[3 + 2 * lane] = o1[j];
    }
    if (lane == 0) {
      pp[0] = mrun[j];
      pp[1] = lrun[j];
    }
  }
  __threadfence();
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) s_last = (atomicAdd(&a.counters[unit], 1) == n_parts - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- combine splits in order (last workgroup only) ----
  const float* base = a.part + (size_t)unit * n_parts * QG * rec;
  for (int e = tid; e < nq * hd; e += kThreads) {
    const int qv = e / hd, dd = e % hd;
    float mx = -INFINITY;
    for (int sp = 0; sp < n_parts; ++sp) {
      const float* pp = base + ((size_t)sp * QG + qv) * rec;
      if (pp[1] > 0.f) mx = fmaxf(mx, pp[0]);
    }
    float l = 0.f, o = 0.f;
    for (int sp = 0; sp < n_parts; ++sp) {
      const float* pp = base + ((size_t)sp * QG + qv) * rec;
      if (pp[1] > 0.f) {
        const float w = expf(pp[0] - mx);
        l += pp[1] * w;
        o += pp[2 + dd] * w;
      }
    }
    const int gq = q0 + qv;
    const int m = r0 + gq % nr, h = kvh * G + gq / nr;
    xa_store(a.xa_o, h * hd + dd, m, a.M, o / l);
  }
  if (tid == 0) a.counters[unit] = 0;
}

hipError_t attn_init() {
  // largest launch: 64 query vectors of 128 dims, ~81 KB
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             96 * 1024);
}

void launch_attention(const AttnArgs& a, hipStream_t st) {
  const int n_parts = a.n_split + 1;
  dim3 grid(a.rows.n_seq * n_parts, a.Hkv, a.n_qg);
  const int hw = a.hd / 2;
  const size_t lds = (size_t)a.qg_size * a.hd * 4 + (size_t)a.qg_size * kChunk * 4 + (size_t)kChunk * (hw + 1) * 4 +
                     (size_t)kChunk * hw * 4;
  hipLaunchKernelGGL(attn_kernel, grid, dim3(kThreads), lds, st, a);
}

}  // namespace vs
