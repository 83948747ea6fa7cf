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
// KV layout per layer: K [block][kv head][head_dim/8][16 keys][8 dims], V
// [block][kv head][head_dim][16 keys].  With that layout both MFMA operands
// come straight from HBM as 16-byte pieces: for S = Q.K^T a lane reads 8 dims
// of one key, and the 64 lanes of one k-step read 1 KiB of consecutive bytes
// (whole cache lines: a vector L1 miss costs one 128-byte request, and the
// number of misses a CU can keep in flight is what bounds its bandwidth);
// for O += P.V a lane reads 8 consecutive keys of one dim.
//
// Split structure, fixed by absolute key index and the sequence's own KV
// length P (read here on the device), so that a row's bits never depend on
// the other sequences of its pass or on how the work is spread:
//  * committed split j holds keys [32 j, 32 j + 32) below P (one step); the
//    in-round window is split ceil(P / 32);
//  * chunk c is splits [4 c, 4 c + 4), one per wave (4-wave workgroups, two
//    per CU: the loads of a workgroup go through its CU at a few tens of
//    GB/s, so a pass spreads them over every CU); its waves' (max, sum, o)
//    are merged in LDS in wave order into the chunk's partial;
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
// invalidate the whole L2.  When every unit of the pass is one workgroup's
// and the chunk partials fit (LP), they stay in LDS and the workgroup
// combines them there with the same arithmetic.
#include "attn_dev.h"

namespace vs {

namespace {

// LDS writes of this wave done, then the workgroup barrier; global loads
// stay in flight (unlike __syncthreads(), which waits for them too).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace

// Query vector v of a unit maps to row r0 + v % nr and head kvh*G + v / nr.
// LP: every unit of the pass is one workgroup's and its chunk partials fit
// kAttnLpRecords records in LDS, where they stay until the combine instead
// of making a round trip through memory.
// Two workgroups per CU where the LDS allows it (at most 256 registers per
// lane); the LP instance holds 128 KB of LDS and runs one.
template <int HD, int WV, bool LP>
__global__ __launch_bounds__(WV * 64, LP ? 1 : 2) void attn_kernel(const AttnArgs a) {
  constexpr int kThreads = WV * 64;
  constexpr int KSQ = HD / 32;  // k-steps of S over head dims
  constexpr int NDT = HD / 16;  // 16-dim output tiles
  constexpr int QR = 16;        // query vectors of the MFMA tile
  constexpr int PS = kStep + 4;  // P scratch row stride (floats)
  constexpr int HDP = HD + 4;    // merge row stride (floats): rows one lane group apart in other banks
  constexpr int PL_FLOATS = WV * QR * PS;                 // per-wave P scratch
  constexpr int MG_FLOATS = WV * QR * HDP + 2 * WV * QR;  // one merge buffer: o, then (max, sum)
  constexpr int SM_FLOATS = PL_FLOATS + 2 * MG_FLOATS;
  // P scratch, then two merge buffers used by alternate chunks, so that a
  // chunk's merge needs one barrier: the next chunk writes the other buffer,
  // and the one after that passes this chunk's barrier first.
  __shared__ float smem[SM_FLOATS];
  __shared__ int last_wg;
  // LP: chunk partial (chunk j, query v) at lpo[(j * nq + v) * HD], its
  // (max, sum) at lml[j * nq + v]
  __shared__ float lpo[LP ? kAttnLpRecords * HD : 1];
  __shared__ float2 lml[LP ? kAttnLpRecords : 1];

  // The wave index is made wave-uniform, so that every per-split decision is
  // a scalar branch and no K/V wait is merged with a branch's loads: the
  // compiler then waits for each K/V load alone instead of draining them all.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;  // the grid is exactly the pass's wg_start[n_seq] workgroups
  // Memory round trips before the first scores: (1) every per-sequence field
  // of the arguments at once, lane l holding sequence l's, the workgroup's
  // sequence being the last whose first workgroup is <= b; (2) P, the
  // block-table entries and the query vectors together; (3) K and V.
  const int ls = min(lane, kMaxSeq - 1);
  const int ws_l = a.wg_start[ls], sq_l = a.rows.seq[ls], r0_l = a.rows.row_start[ls];
  const int r1_l = a.rows.row_start[ls + 1], nsp_l = a.nsplit[ls], wb_l = a.wblk[ls];
  const int i = __popcll(__ballot(lane < a.rows.n_seq && ws_l <= b)) - 1;
  // Workgroups of a sequence in order of their chunks, KV heads fastest:
  // the ones past what the device's context needs (the host lays out its
  // upper bound) come last and exit as soon as P is known.
  const int local = b - __builtin_amdgcn_readlane(ws_l, i);
  const int wgi = local / a.Hkv, kvh = local - wgi * a.Hkv;
  const int sq = __builtin_amdgcn_readlane(sq_l, i);
  const int r0 = __builtin_amdgcn_readlane(r0_l, i);
  const int nr = __builtin_amdgcn_readlane(r1_l, i) - r0;
  const int wblk = __builtin_amdgcn_readlane(wb_l, i);
  const int G = a.H / a.Hkv;
  const int nq = min(QR, nr * G);
  const int c0 = wgi * a.cpw;
  const int* bt = a.kv.bt + (size_t)sq * a.kv.bps;
  const int mrow = lane & 15, kq = lane >> 4;
  // Round (2): P, the block-table entries of this wave's steps (read once
  // into lane-indexed registers so that no K/V load waits on a table load:
  // lane l of bt_c holds block 2 * (WV c + wave) + l % 2 of chunk c = c0 +
  // l / 2, its committed split, a workgroup running at most 32 chunks; lane
  // l of bt_w holds block wblk + l, the window's steps when P is within 64
  // blocks of the host's lower bound; entries are clamped to the table and
  // data outside a split is masked), the query vectors and the masks.
  const int P = a.kv.P[sq];
  const int bt_c = bt[min(2 * (WV * (c0 + (lane >> 1)) + wave) + (lane & 1), a.kv.bps - 1)];
  const int bt_w = bt[min(wblk + lane, a.kv.bps - 1)];
  float4 qraw[KSQ][2];
  // Visibility masks of the 4 rows this lane holds in S: the pass's masks
  // if it has them, else a chain's (row idx sees in-round keys 0..idx).  The
  // loads are unconditional (a pass without masks reads its query buffer
  // instead) and the choice is made where a mask is used: a branch here
  // would make the compiler wait for every load in flight at its join.
  uint64_t mraw[4];
  const uint64_t* const mbase =
      a.rows.mask != nullptr ? a.rows.mask + r0 : reinterpret_cast<const uint64_t*>(a.q);
  {
    const int gq = min(mrow, nq - 1);
    const float* src = a.q + ((size_t)(r0 + gq % nr) * a.H + kvh * G + gq / nr) * HD;
#pragma unroll
    for (int s = 0; s < KSQ; ++s) {
      qraw[s][0] = *reinterpret_cast<const float4*>(src + 32 * s + 8 * kq);
      qraw[s][1] = *reinterpret_cast<const float4*>(src + 32 * s + 8 * kq + 4);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) mraw[r] = mbase[min(4 * kq + r, nq - 1) % nr];
  }
  // every request above is issued before the branch on P below
  asm volatile("" ::: "memory");

  const int ns = (P + kStep - 1) / kStep;  // committed splits
  // + the in-round window; never past the host's layout (P <= its bound)
  const int n_chunks = min((ns + 1 + WV - 1) / WV, __builtin_amdgcn_readlane(nsp_l, i));
  if (c0 >= n_chunks) return;  // past what this sequence's context needs
  const int c1 = min(n_chunks, c0 + a.cpw);
  const int nwg = (n_chunks + a.cpw - 1) / a.cpw;  // workgroups of the unit with chunks
  const int unit = i * a.Hkv + kvh;
  const int wlo = P + a.rows.win, whi = wlo + a.rows.idx_off + nr;  // in-round keys

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
  auto blocks_of = [&](int c, int base) {  // step at key `base`, in chunk c
    if (c * WV + wave < ns) {
      const int l = 2 * (c - c0);
      nb0 = __builtin_amdgcn_readlane(bt_c, l);
      nb1 = __builtin_amdgcn_readlane(bt_c, l + 1);
    } else {
      const int l = base / kBlock - wblk;
      if (l >= 0 && l < 63) {
        nb0 = __builtin_amdgcn_readlane(bt_w, l);
        nb1 = __builtin_amdgcn_readlane(bt_w, l + 1);
      } else {  // P far from the host's lower bound: read the two entries
        // (scalar loads: the constant address space keeps them off the
        // vector memory counter that the K/V ring's waits count)
        const auto* cbt = (const __attribute__((address_space(4))) int*)(bt);
        nb0 = cbt[min(base / kBlock, a.kv.bps - 1)];
        nb1 = cbt[min(base / kBlock + 1, a.kv.bps - 1)];
      }
    }
  };
  using KBuf = u32x4[2][KSQ];
  using VBuf = u32x4[NDT];
  auto load_k = [&](KBuf& kbuf) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* kr = a.kv.k + kv_tile(t ? nb1 : nb0, kvh, a.Hkv, HD) + k_tile_off(mrow, 8 * kq);
#pragma unroll
      for (int s = 0; s < KSQ; ++s)
        kbuf[t][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + k_tile_off(0, 32 * s)));
    }
  };
  auto load_v = [&](VBuf& vbuf) {  // lane: keys 8*kq .. +8 of dim 16t + lane%16, i.e. block kq/2, keys 8*(kq%2) ..
    const uint16_t* vr = a.kv.v + kv_tile((kq >> 1) ? nb1 : nb0, kvh, a.Hkv, HD) + 8 * (kq & 1);
#pragma unroll
    for (int t = 0; t < NDT; ++t)
      vbuf[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vr + (size_t)(16 * t + mrow) * kBlock));
  };

  // Round (3): the first K/V step; the queries are split while it is in
  // flight.
  int first, last;
  split_steps(c0, first, last);
  if (first < last) {
    blocks_of(c0, first);
    load_k(kb);
    load_v(vb);
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

  // One step of 32 keys at `base` of this wave's split in chunk c, its K and
  // V in (kbuf, vbuf): S, then kload() (a later step's K into kbuf), the
  // masked online-softmax update, O += P.V, then vload().
  auto run_step = [&](KBuf& kbuf, VBuf& vbuf, const int c, const int base, float(&mrun)[4], float(&lrun)[4],
                      f32x4(&oacc)[NDT], auto&& kload, auto&& vload) {
    const int sp = c * WV + wave;
    const bool window = sp == ns;
    const int key_lo = window ? wlo : sp * kStep;
    const int key_hi = window ? whi : min(P, sp * kStep + kStep);
    // S = Q.K^T for the two 16-key tiles
    f32x4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSQ; ++s) {
        cc = mfma16(qh[s], kbuf[t][s], cc);
        cc = mfma16(ql[s], kbuf[t][s], cc);
      }
      sacc[t] = cc;
    }
    kload();
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
          if (vis && window) {
            const int rl = min(row, nq - 1) % nr, idx = a.rows.idx_off + rl;
            const uint64_t mk = a.rows.mask != nullptr ? mraw[r] : (idx >= 63 ? ~0ull : ((2ull << idx) - 1ull));
            vis = row < nq && ((mk >> ((slot - key_lo) & 63)) & 1ull);  // count kept in 0..63
          }
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
        oacc[t] = mfma16(ph, vbuf[t], oacc[t]);
        oacc[t] = mfma16(pl, vbuf[t], oacc[t]);
      }
    }
    vload();
  };
  auto merge_chunk = [&](const int c, const float(&mrun)[4], const float(&lrun)[4], const f32x4(&oacc)[NDT]) {
    // ---- merge the chunk's WV split partials: every wave puts its (max,
    // sum, o) for the rows below nq in the chunk's merge buffer; after one
    // barrier, wave w merges dims [w*DS, (w+1)*DS) of all WV partials in
    // wave order and writes that slice of the chunk's partial (or of the
    // result).  Each lane takes the weights exp2(m_j - max) of its row
    // itself (the same operations in the same order for every lane).
    float* xo = smem + PL_FLOATS + (c & 1) * MG_FLOATS;             // [WV][QR][HDP]
    float2* xml = reinterpret_cast<float2*>(xo + WV * QR * HDP);     // [WV][QR]
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
    const size_t rec = (size_t)unit * a.n_split + c;
    for (int e = lane; e < nq * DS; e += 64) {
      const int row = e / DS, d = wave * DS + e % DS;
      float2 ml[WV];
      float xv[WV];
#pragma unroll
      for (int j = 0; j < WV; ++j) {  // every LDS read first, one wait
        ml[j] = xml[j * QR + row];
        xv[j] = xo[(j * QR + row) * HDP + d];
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < WV; ++j)
        if (ml[j].y > 0.f) mx = fmaxf(mx, ml[j].x);  // a split that saw no key has sum 0
      float o = 0.f, l = 0.f;
#pragma unroll
      for (int j = 0; j < WV; ++j) {
        const float w = ml[j].y > 0.f ? __builtin_amdgcn_exp2f(ml[j].x - mx) : 0.f;
        l += w * ml[j].y;
        o += w * xv[j];
      }
      if (single) {
        xa_store(a.xa_o, (kvh * G + row / nr) * HD + d, r0 + row % nr, a.M, o / l);
      } else if constexpr (LP) {  // c0 = 0: one workgroup holds every chunk of the unit
        lpo[(c * nq + row) * HD + d] = o;
        if (d == 0) lml[c * nq + row] = make_float2(mx, l);
      } else {
        __hip_atomic_store(po + (rec * QG + row) * HD + d, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
          const uint64_t bits = (uint64_t)__float_as_uint(mx) | ((uint64_t)__float_as_uint(l) << 32);
          __hip_atomic_store(pml + rec * QG + row, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  };
  auto init_acc = [&](float(&mrun)[4], float(&lrun)[4], f32x4(&oacc)[NDT]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mrun[r] = -INFINITY;
      lrun[r] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < NDT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  for (int c = c0; c < c1; ++c) {
    float mrun[4], lrun[4];
    f32x4 oacc[NDT];
    init_acc(mrun, lrun, oacc);
    for (int base = first; base < last; base += kStep) {
      // the next step to load: this split's next one, else the first step
      // of this wave's split in the next chunk of the workgroup, else this
      // step again (an L2 hit): the loads are issued on every path, so that
      // the compiler's waits count them exactly and the next step stays in
      // flight while this one computes
      int nbase = base + kStep, nc = c;
      if (nbase >= last) {
        nbase = base;
        if (c + 1 < c1) {
          int nf, nl;
          split_steps(c + 1, nf, nl);
          if (nf < nl) {
            nbase = nf;
            nc = c + 1;
          }
        }
      }
      blocks_of(nc, nbase);
      run_step(kb, vb, c, base, mrun, lrun, oacc, [&] { load_k(kb); }, [&] { load_v(vb); });
    }
    merge_chunk(c, mrun, lrun, oacc);
    if (c + 1 < c1) split_steps(c + 1, first, last);
  }
  if (single) return;

  if constexpr (LP) {
    // The unit's combine from LDS, with the arithmetic of the combine
    // below: the largest chunk maximum over chunks that saw a key, then
    // the weights exp2(m_j - max) and the sums in chunk order.
    constexpr int HP = HD / 2;
    __syncthreads();
    for (int p = threadIdx.x; p < nq * HP; p += kThreads) {
      const int r = p / HP, cp = p - r * HP;
      float mx = -INFINITY;
      for (int j = 0; j < n_chunks; ++j) {
        const float2 ml = lml[j * nq + r];
        if (ml.y > 0.f) mx = fmaxf(mx, ml.x);
      }
      float tot = 0.f, o0 = 0.f, o1 = 0.f;
      for (int j = 0; j < n_chunks; ++j) {
        const float2 ml = lml[j * nq + r];
        const float w = ml.y > 0.f ? __builtin_amdgcn_exp2f(ml.x - mx) : 0.f;
        tot += w * ml.y;
        o0 += w * lpo[(j * nq + r) * HD + 2 * cp];
        o1 += w * lpo[(j * nq + r) * HD + 2 * cp + 1];
      }
      const int m = r0 + r % nr, h = kvh * G + r / nr;
      xa_store(a.xa_o, h * HD + 2 * cp, m, a.M, o0 / tot);
      xa_store(a.xa_o, h * HD + 2 * cp + 1, m, a.M, o1 / tot);
    }
    return;
  }

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
  // order.  A thread takes one or two pairs of dims of one query vector: it
  // requests every (max, sum) record of the vector's row and every partial
  // of its pairs at once (kCB chunks at a time), then forms the weights
  // exp2(m_j - max) and the sums in chunk order itself: one round trip to
  // memory, no barrier.
  constexpr int HP = HD / 2;   // dim pairs
  constexpr int kCB = 16;      // chunks requested per batch
  constexpr int kPairs = 2;    // pairs per thread per round
  // The loads go through buffer resources whose extents end at the unit's
  // last chunk: a load past it (the batch's chunks beyond nc, a thread's
  // pair beyond the vectors') returns zeros without a memory request, so
  // the CU fetches only the partials that exist.  They keep the
  // device-coherent cache policy (sc1) of agent-scope atomic loads.
  constexpr int kSc1 = 16;
  const int nc = n_chunks;
  const int S = (int)QG * HP;  // pairs between consecutive partials
  const int npair = nq * HP;
  const int xbytes = nc * S * 8, mlbytes = nc * (int)QG * 8;
  const size_t ubase = (size_t)__builtin_amdgcn_readfirstlane(unit) * a.n_split * QG;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)(reinterpret_cast<const uint64_t*>(po) + ubase * HP), 0, xbytes, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc((void*)(pml + ubase), 0, mlbytes, kRawBufferWord3);
  for (int p0 = threadIdx.x; p0 < npair; p0 += kPairs * kThreads) {
    int pr[kPairs], rr[kPairs], xo[kPairs], mo[kPairs];
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      const bool ok = p0 + q * kThreads < npair;
      pr[q] = min(p0 + q * kThreads, npair - 1);
      rr[q] = pr[q] / HP;
      xo[q] = ok ? pr[q] * 8 : xbytes;  // byte offsets in chunk 0, or out of range
      mo[q] = ok ? rr[q] * 8 : mlbytes;
    }
    float mx[kPairs], tot[kPairs], o0[kPairs], o1[kPairs];
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      mx[q] = -INFINITY;
      tot[q] = o0[q] = o1[q] = 0.f;
    }
    uint64_t mlv[kPairs][kCB], xv[kPairs][kCB];
    auto load = [&](int j0, bool with_x) {
#pragma unroll
      for (int q = 0; q < kPairs; ++q)
#pragma unroll
        for (int e = 0; e < kCB; ++e) {
          const int j = j0 + e;
          const auto m2 = __builtin_amdgcn_raw_buffer_load_b64(rm, j * (int)QG * 8 + mo[q], 0, kSc1);
          mlv[q][e] = (uint64_t)m2[0] | ((uint64_t)m2[1] << 32);
          if (with_x) {
            const auto x2 = __builtin_amdgcn_raw_buffer_load_b64(rx, j * S * 8 + xo[q], 0, kSc1);
            xv[q][e] = (uint64_t)x2[0] | ((uint64_t)x2[1] << 32);
          }
        }
    };
    auto take_max = [&](int j0) {  // a chunk that saw no key has sum 0
#pragma unroll
      for (int q = 0; q < kPairs; ++q)
#pragma unroll
        for (int e = 0; e < kCB; ++e) {
          const float m = __uint_as_float((uint32_t)mlv[q][e]), l = __uint_as_float((uint32_t)(mlv[q][e] >> 32));
          if (j0 + e < nc && l > 0.f) mx[q] = fmaxf(mx[q], m);
        }
    };
    auto add = [&](int j0) {  // weights exp2(m_j - max), sums in chunk order
#pragma unroll
      for (int q = 0; q < kPairs; ++q)
#pragma unroll
        for (int e = 0; e < kCB; ++e) {
          const float m = __uint_as_float((uint32_t)mlv[q][e]), l = __uint_as_float((uint32_t)(mlv[q][e] >> 32));
          const float w = (j0 + e < nc && l > 0.f) ? __builtin_amdgcn_exp2f(m - mx[q]) : 0.f;
          tot[q] += w * l;
          o0[q] += w * __uint_as_float((uint32_t)xv[q][e]);
          o1[q] += w * __uint_as_float((uint32_t)(xv[q][e] >> 32));
        }
    };
    if (nc <= kCB) {  // one batch: every load in flight at once
      load(0, true);
      take_max(0);
      add(0);
    } else {  // the maxima over every chunk first, then the sums
      for (int j0 = 0; j0 < nc; j0 += kCB) {
        load(j0, false);
        take_max(j0);
      }
      for (int j0 = 0; j0 < nc; j0 += kCB) {
        load(j0, true);
        add(j0);
      }
    }
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      if (p0 + q * kThreads >= npair) continue;
      const int r = rr[q], cp = pr[q] - r * HP;
      const int m = r0 + r % nr, h = kvh * G + r / nr;
      xa_store(a.xa_o, h * HD + 2 * cp, m, a.M, o0[q] / tot[q]);
      xa_store(a.xa_o, h * HD + 2 * cp + 1, m, a.M, o1[q] / tot[q]);
    }
  }
}

hipError_t attn_init() { return hipSuccess; }

void launch_attention(const AttnArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid(a.wg_start[a.rows.n_seq]);
#define VS_ATT(HD, LP)                                                                                    \
  do {                                                                                                    \
    if (ev0 != nullptr || ev1 != nullptr)                                                                 \
      hipExtLaunchKernelGGL((attn_kernel<HD, kAttnWaves, LP>), grid, dim3(kAttnWaves * 64), 0, st, ev0, ev1, 0, a); \
    else                                                                                                  \
      hipLaunchKernelGGL((attn_kernel<HD, kAttnWaves, LP>), grid, dim3(kAttnWaves * 64), 0, st, a);      \
  } while (0)
  if (a.hd == 128) {
    if (a.lp) VS_ATT(128, true);
    else VS_ATT(128, false);
  } else {
    if (a.lp) VS_ATT(64, true);
    else VS_ATT(64, false);
  }
#undef VS_ATT
}

}  // namespace vs
