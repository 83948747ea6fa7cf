// C ABI of the verify-step library: argument validation, buffer layout and
// the order of kernel launches for prefill, draft, verify, accept and commit.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <vector>

#include "attn_group.h"
#include "kernels.h"
#include "gemm_dev.h"
#include "misc.h"

using namespace vs;

namespace {

thread_local std::string g_err;

vs_status fail(vs_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Mat {
  uint16_t* w = nullptr;
  int n_tiles = 0, k_steps = 0;
  size_t bytes() const { return (size_t)n_tiles * k_steps * 1024; }
};

// Layout of the packed weight buffer (offsets in bytes, 256-aligned).
struct WeightLayout {
  size_t embed, g_final, head, total;
  std::vector<size_t> qkv, o, gu, down, g_attn, g_ffn;
};

bool shape_ok(const vs_model_cfg* c, std::string* why) {
  auto bad = [&](const char* s) {
    if (why) *why = s;
    return false;
  };
  if (c->n_layers < 1 || c->d_model < 32 || c->n_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 16 ||
      c->d_ffn < 32 || c->vocab < 16)
    return bad("sizes must be positive (d_model, d_ffn >= 32, head_dim >= 16, vocab >= 16)");
  if (c->exit_layer < 0 || c->exit_layer > c->n_layers) return bad("exit_layer must lie in [0, n_layers]");
  if (c->d_model % 256 != 0) return bad("d_model must be a multiple of 256");
  if (c->d_ffn % 32 != 0) return bad("d_ffn must be a multiple of 32");
  if (c->head_dim != 64 && c->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (c->n_heads % c->n_kv_heads != 0) return bad("n_heads must be a multiple of n_kv_heads");
  if ((c->n_heads * c->head_dim) % 32 != 0) return bad("n_heads*head_dim must be a multiple of 32");
  if (c->vocab % 16 != 0 || c->vocab > 32768) return bad("vocab must be a multiple of 16, at most 32768");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 1.f)) return bad("rms_eps > 0 and rope_theta > 1 required");
  return true;
}

WeightLayout weight_layout(const vs_model_cfg* c) {
  WeightLayout L;
  const size_t d = c->d_model, hd = c->head_dim, H = c->n_heads, Hkv = c->n_kv_heads, F = c->d_ffn, V = c->vocab;
  size_t off = 0;
  auto take = [&](size_t b) {
    size_t o = off;
    off = align256(off + b);
    return o;
  };
  L.embed = take(V * d * 2);
  for (int l = 0; l < c->n_layers; ++l) {
    L.qkv.push_back(take((H + 2 * Hkv) * hd * d * 2));
    L.o.push_back(take(d * H * hd * 2));
    L.gu.push_back(take(2 * F * d * 2));
    L.down.push_back(take(d * F * 2));
    L.g_attn.push_back(take(d * 4));
    L.g_ffn.push_back(take(d * 4));
  }
  L.g_final = take(d * 4);
  L.head = take(V * d * 2);
  L.total = off;
  return L;
}

constexpr size_t kAttnPartFloats = size_t(128) << 20;  // 512 MB of attention partials
// tree drafting state: node arrays (4 int + 1 double per node), meta, row arrays
constexpr size_t kTreeBytes = (size_t)kTreeNodes * 24 + 256 + (size_t)kMaxRows * 24;

struct WsLayout {
  size_t h, xa_h, xa_o, xa_act, ss, q, rope, kvrow, part, attn_cnt, tree, amax_val, amax_idx, logits, dlogits, hidden, tokens, st_mx, st_amax,
      st_second, st_sum, dst_mx, dst_amax, dst_sum, result, conf, tp_key, tp_id, tp_mass, rs, kpart, kcnt, total;
};

WsLayout ws_layout(const vs_model_cfg* c, int R, int S) {
  WsLayout w;
  const size_t d = c->d_model, hd = c->head_dim, H = c->n_heads, F = c->d_ffn, V = c->vocab;
  size_t off = 0;
  auto take = [&](size_t b) {
    size_t o = off;
    off = align256(off + b);
    return o;
  };
  w.h = take(R * d * 4);
  w.xa_h = take(R * d * 4);
  w.xa_o = take(R * H * hd * 4);
  w.xa_act = take(R * F * 4);
  w.ss = take(R * (d / 16) * 4);
  w.q = take(R * H * hd * 4);
  w.rope = take(R * (hd / 2) * 8);
  w.kvrow = take(R * 4);
  w.part = take(kAttnPartFloats * 4);
  w.attn_cnt = take(kAttnMaxUnits * 4);
  w.tree = take(kTreeBytes);
  w.amax_val = take(R * (V / 16) * 4);
  w.amax_idx = take(R * (V / 16) * 4);
  w.logits = take(R * V * 4);
  w.dlogits = take(R * V * 4);
  w.hidden = take(R * d * 4);
  w.tokens = take(R * 4);
  w.st_mx = take(R * 4);
  w.st_amax = take(R * 4);
  w.st_second = take(R * 4);
  w.st_sum = take(R * 8);
  w.dst_mx = take(R * 4);
  w.dst_amax = take(R * 4);
  w.dst_sum = take(R * 8);
  w.result = take((size_t)S * VS_RESULT_INTS * 4);
  w.conf = take((size_t)kMaxSeq * 2 * 8);
  w.tp_key = take(R * 4);
  w.tp_id = take(R * 4);
  w.tp_mass = take(R * 8);
  w.rs = take(R * 4);
  w.kpart = take(kGemmSplitFloats * 4);
  w.kcnt = take((size_t)kGemmSplitCells * 4);
  w.total = off;
  return w;
}

// Longest committed split of the grouped attention kernel: 29 steps, so that
// with up to 64 in-round keys a split stays within kAttnGroupSteps steps.
constexpr int kAttnGroupMaxKps = (kAttnGroupSteps - 3) * kAttnStepKeys;

// Default split length of the grouped kernel for a model: the splits of one
// sequence cut about 4 MiB of K/V (all its KV heads) each, within
// [32, kAttnGroupMaxKps] keys: 256 keys at the 7B shape (32 KV heads x 128),
// the longest split at the 70B shape (8 x 128).
int default_attn_split(const vs_model_cfg& c) {
  const long per_key = (long)c.n_kv_heads * c.head_dim * 4;
  const long keys = (4L << 20) / per_key / kAttnStepKeys * kAttnStepKeys;
  return (int)std::min<long>(kAttnGroupMaxKps, std::max<long>(kAttnStepKeys, keys));
}

enum Family { F_QKV = 0, F_O, F_GU, F_DOWN, F_HEAD, F_ATTN, F_SMALL, F_COUNT };
const char* kFamilyNames[F_COUNT] = {"gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "gemm_head",
                                     "attention", "small"};

struct Timed {
  int fam;
  hipEvent_t prev, a, b;  // previous launch's end; this kernel's start and end (a may be null)
  double bytes;
};

}  // namespace

struct vs_model {
  vs_model_cfg c;
  WeightLayout wl;
  char* wbase = nullptr;
  std::vector<Mat> qkv, o, gu, down;
  std::vector<float*> g_attn, g_ffn;
  uint16_t* embed = nullptr;
  float* g_final = nullptr;
  Mat head;
  int max_rows = 0, max_seqs = 0, max_ctx = 0;
  WsLayout wsl;
  char* ws = nullptr;
  unsigned* attn_cnt;
  TreeArgs tree;          // device pointers of the tree drafting state
  float *h, *ss, *rs, *kpart, *q, *part, *logits, *dlogits, *hidden, *st_mx, *st_second, *dst_mx, *amax_val;
  unsigned* kcnt = nullptr;
  int n_cu = 256;        // compute units of the device
  int attn_split = 256;  // keys per committed split of the grouped attention kernel
  uint16_t *xa_h, *xa_o, *xa_act;
  float2* rope;
  int* kvrow;
  int *amax_idx, *tokens, *st_amax, *dst_amax, *result;
  double *st_sum, *dst_sum, *conf, *tp_mass;
  unsigned* tp_key;
  int* tp_id;
  int ss_groups = 0;       // groups of the last producer of ss
  int head_groups = 0;     // groups of the last head pass
  int head_rows = 0;
  // timing
  int stats_mask = 0;  // families timed with events (bit f)
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  hipEvent_t prev_end = nullptr;  // end event of the last timed launch
  std::vector<Timed> timed;
  double acc_ms[F_COUNT] = {0};
  double acc_bytes[F_COUNT] = {0};
  int64_t acc_n[F_COUNT] = {0};
};

struct vs_kv {
  vs_model* m = nullptr;
  char* base = nullptr;
  int n_blocks = 0, max_seqs = 0, bps = 0;
  std::vector<uint16_t*> k, v;
  uint16_t** d_kptr = nullptr;
  uint16_t** d_vptr = nullptr;
  int *P = nullptr, *pending = nullptr, *committed = nullptr, *bt = nullptr;
  std::vector<int> free_blocks;
  std::vector<std::vector<int>> blocks;
  std::vector<int> open, cap, P_ub, prefilled;
  // The host's bound P_ub of each sequence's KV length: the exact value at
  // the last host-side setting (open, prefill, assume, rewind, sync) plus the
  // rows of every commit since.  Commits are numbered per sequence and the
  // commit kernel stores (number << 32 | new P) into a pinned host mirror,
  // so once the host sees a commit there the bound becomes that exact P plus
  // the rows of the later commits only.  No host wait is involved.
  uint64_t* mirror = nullptr;  // pinned [max_seqs]
  std::vector<unsigned> commit_no, base_no;
  std::vector<int> P_base;
  std::vector<int> P_known;  // the exact P the bound starts from (last landed commit, else P_base)
  std::vector<std::deque<std::pair<unsigned, int>>> in_flight;  // (commit number, rows) not yet seen
};

namespace {

hipStream_t S(void* st) { return reinterpret_cast<hipStream_t>(st); }

// The bound becomes exact: P is known on the host (in stream order after
// every earlier commit of the sequence).
void kv_set_exact(vs_kv* kv, int s, int P) {
  kv->P_ub[s] = kv->P_base[s] = kv->P_known[s] = P;
  kv->base_no[s] = kv->commit_no[s] + 1;
  kv->in_flight[s].clear();
}

// Tightens P_ub[s] from the mirror.
void kv_refresh(vs_kv* kv, int s) {
  if (kv->mirror == nullptr) return;
  const uint64_t m = __atomic_load_n(kv->mirror + s, __ATOMIC_ACQUIRE);
  const unsigned no = (unsigned)(m >> 32);
  auto& q = kv->in_flight[s];
  int bound;
  if (no >= kv->base_no[s] && no <= kv->commit_no[s]) {  // a commit since the exact setting has landed
    while (!q.empty() && q.front().first <= no) q.pop_front();
    bound = (int)(uint32_t)m;
  } else {
    bound = kv->P_base[s];
  }
  kv->P_known[s] = bound;
  for (const auto& c : q) bound += c.second;
  kv->P_ub[s] = bound;
}

// A lower bound of P: the exact value the upper bound starts from plus one
// per commit still in flight (a commit advances P by a + 1 >= 1).  With no
// commit in flight the upper bound is exact.
int kv_lower(const vs_kv* kv, int s) {
  const auto& q = kv->in_flight[s];
  return q.empty() ? kv->P_ub[s] : std::min(kv->P_ub[s], kv->P_known[s] + (int)q.size());
}

vs_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VS_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return VS_OK;
}

hipEvent_t next_event(vs_model* m) {
  if (m->ev_used == m->ev_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    m->ev_pool.push_back(e);
  }
  return m->ev_pool[m->ev_used++];
}

// Launch timing while a stats mask is set: every launch gets an end event
// timestamped by the kernel itself (GEMM and attention launches take their
// start and end events through hipExtLaunchKernelGGL; other launches get a
// marker right after), and a launch of a selected family is charged from the
// later of the previous launch's end and its own start event to its end.
// Back to back, the start event can be stamped before the previous kernel
// has drained, so the previous end bounds it; with idle time between
// launches, the start event does.
template <typename F>
void timed(vs_model* m, int fam, double bytes, hipStream_t st, F launch) {
  if (m->stats_mask == 0) {
    launch(nullptr, nullptr);
    return;
  }
  const bool sel = (m->stats_mask >> fam & 1) && fam != F_SMALL && m->prev_end != nullptr;
  hipEvent_t a = sel ? next_event(m) : nullptr;
  hipEvent_t b = next_event(m);
  if (!b || (sel && !a)) {
    launch(nullptr, nullptr);
    return;
  }
  if (fam == F_SMALL) {
    launch(nullptr, nullptr);
    (void)hipEventRecord(b, st);
  } else {
    launch(a, b);
  }
  if ((m->stats_mask >> fam & 1) && m->prev_end != nullptr) m->timed.push_back(Timed{fam, m->prev_end, a, b, bytes});
  m->prev_end = b;
}

KvView kv_view(vs_kv* kv, int layer) {
  KvView v;
  v.k = kv->k[layer];
  v.v = kv->v[layer];
  v.P = kv->P;
  v.bt = kv->bt;
  v.bps = kv->bps;
  return v;
}

GemmArgs gemm_base(vs_model* m, const Mat& W, const uint16_t* xa, int M) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.W = W.w;
  g.n_tiles = W.n_tiles;
  g.k_steps = W.k_steps;
  g.xa = xa;
  g.M = M;
  g.m0 = 0;
  g.ld = M;
  g.inv_d = 1.0f / (float)m->c.d_model;
  g.eps = m->c.rms_eps;
  g.d = m->c.d_model;
  g.out_row_identity = 1;
  g.rs_buf = m->rs;
  g.kpart = m->kpart;
  g.kcnt = m->kcnt;
  return g;
}

double gemm_bytes(const Mat& W, int M) {
  return (double)W.bytes() + (double)M * W.k_steps * 32 * 4 + (double)M * W.n_tiles * 16 * 4;
}

// One GEMM of a pass.  The row-tiled form takes the whole pass in one launch
// unless rows are redirected (out_rows).  Otherwise a pass of more than
// kMaxRows rows runs as launches of kMaxRows rows (row offset m0, row stride
// = the pass's rows) that all use one launch configuration, so the
// per-workgroup norm sums of an EPI_RESID product keep one layout (every
// form writes one sum per 16 columns).  out_rows (optional): destination row
// of each pass row (h_copy / logits).  Returns the number of norm / argmax
// groups a launch writes.
int run_gemm(vs_model* m, GemmArgs g, int epi, int fam, const Mat& W, hipStream_t st, const int* out_rows) {
  const int M = g.M;
  g.m0 = 0;
  g.ld = M;
  if (out_rows == nullptr && gemm_uses_tile(W.n_tiles, W.k_steps, M, g.cfg)) {
    int groups = 0;
    timed(m, fam, gemm_bytes(W, M), st, [&](hipEvent_t e0, hipEvent_t e1) { groups = launch_gemm(g, epi, st, e0, e1); });
    return groups;
  }
  if (M > kMaxRows && !gemm_uses_tile(W.n_tiles, W.k_steps, kMaxRows, g.cfg)) g.cfg = gemm_pick(W.n_tiles, W.k_steps, kMaxRows);
  int groups = 0;
  for (int m0 = 0; m0 < M; m0 += kMaxRows) {
    GemmArgs c = g;
    c.m0 = m0;
    c.M = std::min(kMaxRows, M - m0);
    if (out_rows != nullptr) {
      c.out_row_identity = 0;
      for (int i = 0; i < c.M; ++i) c.out_row[i] = out_rows[m0 + i];
    }
    timed(m, fam, gemm_bytes(W, c.M), st,
          [&](hipEvent_t e0, hipEvent_t e1) { groups = launch_gemm(c, epi, st, e0, e1); });
  }
  return groups;
}

// Loads rows (embedding of token ids, or hidden rows) into the residual
// stream with the next consumer's gain g.
void load_rows(vs_model* m, int M, const int* tokens, const float* hidden, const int* src_rows, const float* g,
               hipStream_t st, const RowMap* rows = nullptr, const vs_kv* kv = nullptr) {
  LoadArgs a;
  memset(&a, 0, sizeof(a));
  a.M = M;
  a.d = m->c.d_model;
  a.V = m->c.vocab;
  a.tokens = tokens;
  a.embed = m->embed;
  a.hidden = hidden;
  a.src_identity = src_rows == nullptr;
  if (src_rows)  // row gathers come from draft steps: one row per sequence
    for (int i = 0; i < M && i < kMaxRows; ++i) a.src_row[i] = src_rows[i];
  a.h = m->h;
  a.xa = m->xa_h;
  a.g = g;
  a.ss = m->ss;
  if (rows != nullptr) {  // the pass runs layers: build its RoPE table
    a.rope = m->rope;
    a.P = kv->P;
    a.bt = kv->bt;
    a.bps = kv->bps;
    a.kvrow = m->kvrow;
    a.rows = *rows;
    a.half = m->c.head_dim / 2;
    a.theta = m->c.rope_theta;
  }
  timed(m, F_SMALL, (double)M * m->c.d_model * 10, st, [&](hipEvent_t, hipEvent_t) { launch_load_rows(a, st); });
  m->ss_groups = (m->c.d_model + 255) / 256;
}

// Split plan of a pass's attention (the same for every layer of the pass).
// The split structure itself is fixed (see AttnArgs): the plan lays out the
// workgroups from the host's upper bound P_ub of each sequence's KV length,
// and the kernels skip what the device's P does not need.  The kernel class
// is a property of the sequence alone: a sequence whose KV heads carry more
// than one query group (a GQA model, or more than 16 rows of an MHA model)
// takes the grouped kernel, which reads each K/V step once for all of a
// head's query groups; the others take the one-group kernel.  A pass that
// holds both runs both launches, each over its own sequences (the other
// sequences get no workgroups and nsplit 0).  Fails when a launch does not
// fit the partials workspace, the counters or the combine.
struct AttnPlan {
  AttnArgs one, grp;  // split fields, workgroup layout, query groups
  bool has_one = false, has_grp = false;
  double bytes_one = 0, bytes_grp = 0;  // algorithmic K/V bytes of one layer
};

bool attn_seq_grouped(const vs_model_cfg& c, int nr) {
  const int G = c.n_heads / c.n_kv_heads;
  return G > 1 || nr * G > kAttnQG;
}

vs_status attn_plan(vs_model* m, vs_kv* kv, const RowMap& rm, AttnPlan* pl) {
  const vs_model_cfg& c = m->c;
  const int G = c.n_heads / c.n_kv_heads;
  auto base = [&](AttnArgs& a) {
    memset(&a, 0, sizeof(a));
    a.rows = rm;
    a.H = c.n_heads;
    a.Hkv = c.n_kv_heads;
    a.hd = c.head_dim;
    a.scale = 1.0f / std::sqrt((float)c.head_dim);
    a.part = m->part;
    a.cnt = m->attn_cnt;
    a.xa_o = m->xa_o;
    a.M = rm.M;
  };
  base(pl->one);
  base(pl->grp);
  pl->has_one = pl->has_grp = false;
  pl->bytes_one = pl->bytes_grp = 0;
  int nr_one = 0, nr_grp = 0;
  bool grp[kMaxSeq];
  for (int i = 0; i < rm.n_seq; ++i) {
    const int nr = rm.row_start[i + 1] - rm.row_start[i];
    grp[i] = attn_seq_grouped(c, nr);
    const double b = (double)(kv->P_ub[rm.seq[i]] + rm.idx_off + nr) * c.n_kv_heads * c.head_dim * 4;
    if (grp[i]) {
      nr_grp = std::max(nr_grp, nr);
      pl->bytes_grp += b;
    } else {
      nr_one = std::max(nr_one, nr);
      pl->bytes_one += b;
    }
  }
  const size_t rec_floats = (size_t)c.head_dim + 2;
  auto finish = [&](AttnArgs& a, size_t units) -> vs_status {
    if (units > (size_t)kAttnMaxUnits)
      return fail(VS_E_SHAPE, "attention: %zu units exceed the %d counters", units, kAttnMaxUnits);
    if (units * a.n_split * a.qg_size * rec_floats > kAttnPartFloats)
      return fail(VS_E_SHAPE, "attention: pass too wide for the partials workspace");
    a.ml_off = units * a.n_split * a.qg_size * c.head_dim;
    a.ml_off += a.ml_off & 1;
    return VS_OK;
  };
  if (nr_grp > 0) {
    AttnArgs& a = pl->grp;
    pl->has_grp = true;
    const int nq = nr_grp * G;
    a.n_qg = (nq + kAttnQG - 1) / kAttnQG;
    a.qg_size = (nq + a.n_qg - 1) / a.n_qg;
    const int wv = kAttnGroupWaves;
    a.kps = m->attn_split;
    long wgs = 0;
    int nmax = 1;
    for (int i = 0; i < rm.n_seq; ++i) {
      a.wg_start[i] = (int)wgs;
      a.nsplit[i] = 0;
      if (!grp[i]) continue;
      const int nr = rm.row_start[i + 1] - rm.row_start[i];
      const int nqb = ((nr * G + a.qg_size - 1) / a.qg_size + wv - 1) / wv;
      const int ns = std::max(1, (kv->P_ub[rm.seq[i]] + a.kps - 1) / a.kps);
      if (ns > kAttnGroupMaxSplits)
        return fail(VS_E_SHAPE, "attention: a context of %d keys needs more than %d splits of %d keys",
                    kv->P_ub[rm.seq[i]], kAttnGroupMaxSplits, a.kps);
      const long groups = ((long)c.n_kv_heads * ns + kAttnXcds - 1) / kAttnXcds * kAttnXcds;
      a.nsplit[i] = ns;
      wgs += groups * nqb;
      nmax = std::max(nmax, ns);
      if (wgs > (1L << 30)) return fail(VS_E_SHAPE, "attention: pass too large");
    }
    a.wg_start[rm.n_seq] = (int)wgs;
    a.n_split = nmax;
    vs_status rc = finish(a, (size_t)rm.n_seq * c.n_kv_heads * a.n_qg);
    if (rc != VS_OK) return rc;
  }
  if (nr_one > 0) {
    AttnArgs& a = pl->one;
    pl->has_one = true;
    a.n_qg = 1;
    a.qg_size = nr_one * G;
    // Chunks of each sequence (4 one-step splits and the window), then the
    // chunks per workgroup (cpw, at most kAttnMaxCpw) that minimise a
    // launch-time model: a workgroup starts in about kStart, runs its chunks
    // one after another at about kChunk each (one step, the merge; the next
    // chunk's loads in flight meanwhile), two workgroups per CU, plus the
    // cross-workgroup combine when a unit has several workgroups.  One sequence at a short context takes one chunk per
    // workgroup (parallel over the chip); many sequences or long contexts
    // take several (fewer starts and combines).
    int chunks[kMaxSeq];
    int cmax = 1;
    for (int i = 0; i < rm.n_seq; ++i) {
      chunks[i] = 0;
      if (grp[i]) continue;
      const int ns = (kv->P_ub[rm.seq[i]] + kAttnStepKeys - 1) / kAttnStepKeys;
      chunks[i] = (ns + 1 + kAttnWaves - 1) / kAttnWaves;
      cmax = std::max(cmax, chunks[i]);
    }
    // Once the units alone give every CU one (one workgroup per unit), a
    // second workgroup per unit costs more than it hides: at 8 sequences x
    // 2048 keys (256 units) one workgroup per unit took 71.6 us against 78.0
    // us at two (each CU then streams two workgroups' keys, and every unit
    // pays the combine).
    long units_one = 0;
    for (int i = 0; i < rm.n_seq; ++i)
      if (!grp[i]) units_one += c.n_kv_heads;
    constexpr double kStart = 5.0, kChunk = 3.0, kCombine = 5.0;  // us
    const int ncu = 2 * std::max(1, m->n_cu);  // workgroup slots
    double best = 1e30;
    int best_cpw = units_one >= m->n_cu ? std::min(cmax, kAttnMaxCpw) : 1;
    for (int cpw = 1; units_one < m->n_cu && cpw <= std::min(cmax, kAttnMaxCpw); ++cpw) {
      if (cpw > 1 && (cmax + cpw - 1) / cpw == (cmax + cpw - 2) / (cpw - 1)) continue;  // same split of the longest
      long wgs = 0;
      bool multi = false;
      for (int i = 0; i < rm.n_seq; ++i) {
        wgs += (long)c.n_kv_heads * ((chunks[i] + cpw - 1) / cpw);
        multi |= chunks[i] > cpw;
      }
      const double t = std::ceil((double)wgs / ncu) * (kStart + cpw * kChunk) + (multi ? kCombine : 0.0);
      if (t < best) {
        best = t;
        best_cpw = cpw;
      }
    }
    a.cpw = best_cpw;
    // One workgroup per unit and one per CU (the LDS records leave room for
    // one workgroup per CU), and each unit's chunk partials (chunks x query
    // vectors) fit the records: they stay in LDS for the combine.
    a.lp = 0;
    if (units_one == m->n_cu && cmax <= kAttnMaxCpw) {
      a.lp = 1;
      for (int i = 0; i < rm.n_seq; ++i) {
        const int nq = std::min(kAttnQG, (rm.row_start[i + 1] - rm.row_start[i]) * G);
        if (!grp[i] && chunks[i] * nq > kAttnLpRecords) a.lp = 0;
      }
    }
    a.kps = kAttnStepKeys;
    long wgs = 0;
    for (int i = 0; i < rm.n_seq; ++i) {
      a.wg_start[i] = (int)wgs;
      a.nsplit[i] = chunks[i];
      a.wblk[i] = (kv_lower(kv, rm.seq[i]) + rm.win) / kAttnStepKeys * kAttnStepKeys / kBlock;
      wgs += (long)c.n_kv_heads * ((chunks[i] + a.cpw - 1) / a.cpw);
    }
    a.wg_start[rm.n_seq] = (int)wgs;
    a.n_split = cmax;
    vs_status rc = finish(a, (size_t)rm.n_seq * c.n_kv_heads);
    if (rc != VS_OK) return rc;
  }
  return VS_OK;
}

void attention(vs_model* m, vs_kv* kv, const AttnPlan& pl, int layer, hipStream_t st) {
  if (pl.has_one) {
    AttnArgs a = pl.one;
    a.kv = kv_view(kv, layer);
    a.q = m->q;
    timed(m, F_ATTN, pl.bytes_one, st, [&](hipEvent_t e0, hipEvent_t e1) { launch_attention(a, st, e0, e1); });
  }
  if (pl.has_grp) {
    AttnArgs a = pl.grp;
    a.kv = kv_view(kv, layer);
    a.q = m->q;
    timed(m, F_ATTN, pl.bytes_grp, st, [&](hipEvent_t e0, hipEvent_t e1) { launch_attention_group(a, st, e0, e1); });
  }
}

// Layers [start, end) over rows already loaded into h / xa_h / ss.
void run_layers(vs_model* m, vs_kv* kv, const RowMap& rm, int start, int end, hipStream_t st, float* h_copy,
                const int* copy_rows) {
  const vs_model_cfg& c = m->c;
  const int M = rm.M;
  AttnPlan plan;
  if (start < end) (void)attn_plan(m, kv, rm, &plan);  // checked before the pass was enqueued
  for (int l = start; l < end; ++l) {
    {
      GemmArgs g = gemm_base(m, m->qkv[l], m->xa_h, M);
      g.ss = m->ss;
      g.ss_groups = m->ss_groups;
      g.rows = rm;
      g.kv = kv_view(kv, l);
      g.q = m->q;
      g.H = c.n_heads;
      g.Hkv = c.n_kv_heads;
      g.hd = c.head_dim;
      g.rope = m->rope;
      g.kvrow = m->kvrow;
      run_gemm(m, g, EPI_QKV, F_QKV, m->qkv[l], st, nullptr);
    }
    attention(m, kv, plan, l, st);
    {
      GemmArgs g = gemm_base(m, m->o[l], m->xa_o, M);
      g.h = m->h;
      g.xa_next = m->xa_h;
      g.g_next = m->g_ffn[l];
      g.ss_out = m->ss;
      m->ss_groups = run_gemm(m, g, EPI_RESID, F_O, m->o[l], st, nullptr);
    }
    {
      GemmArgs g = gemm_base(m, m->gu[l], m->xa_h, M);
      g.ss = m->ss;
      g.ss_groups = m->ss_groups;
      g.xa_act = m->xa_act;
      run_gemm(m, g, EPI_SWIGLU, F_GU, m->gu[l], st, nullptr);
    }
    {
      GemmArgs g = gemm_base(m, m->down[l], m->xa_act, M);
      g.h = m->h;
      g.xa_next = m->xa_h;
      g.g_next = (l + 1 < end) ? m->g_attn[l + 1] : m->g_final;
      g.ss_out = m->ss;
      const bool copy = l + 1 == end && h_copy != nullptr;
      std::vector<int> rows;
      if (copy) {
        g.h_copy = h_copy;
        rows.resize(M);
        for (int i = 0; i < M; ++i) rows[i] = copy_rows ? copy_rows[i] : i;
      }
      m->ss_groups = run_gemm(m, g, EPI_RESID, F_DOWN, m->down[l], st, copy ? rows.data() : nullptr);
    }
  }
}

// Final norm + head over the rows in h (xa_h already carries g_final).
void run_head(vs_model* m, int M, float* logits, const int* out_rows, hipStream_t st) {
  GemmArgs g = gemm_base(m, m->head, m->xa_h, M);
  g.ss = m->ss;
  g.ss_groups = m->ss_groups;
  g.logits = logits;
  g.V = m->c.vocab;
  g.amax_val = m->amax_val;
  g.amax_idx = m->amax_idx;
  m->head_groups = run_gemm(m, g, EPI_LOGITS, F_HEAD, m->head, st, out_rows);
  m->head_rows = M;
}

vs_status batch_rowmap(vs_kv* kv, const vs_batch* b, RowMap* rm) {
  if (b == nullptr || b->seq == nullptr || b->n_rows == nullptr) return fail(VS_E_INVAL, "batch: null pointer");
  if (b->n_seq < 1 || b->n_seq > kMaxSeq) return fail(VS_E_SHAPE, "batch: n_seq %d not in [1, %d]", b->n_seq, kMaxSeq);
  memset(rm, 0, sizeof(*rm));
  rm->n_seq = b->n_seq;
  int M = 0;
  for (int i = 0; i < b->n_seq; ++i) {
    const int s = b->seq[i];
    if (s < 0 || s >= kv->max_seqs || !kv->open[s]) return fail(VS_E_STATE, "batch: sequence %d is not open", s);
    kv_refresh(kv, s);
    for (int j = 0; j < i; ++j)
      if (b->seq[j] == s) return fail(VS_E_INVAL, "batch: sequence %d listed twice", s);
    if (b->n_rows[i] < 1 || b->n_rows[i] > kMaxRows)
      return fail(VS_E_SHAPE, "batch: %d rows for sequence %d (1..%d allowed)", b->n_rows[i], s, kMaxRows);
    rm->seq[i] = s;
    rm->row_start[i] = M;
    M += b->n_rows[i];
  }
  rm->row_start[b->n_seq] = M;
  if (M > kv->m->max_rows) return fail(VS_E_SHAPE, "batch: %d rows exceed the model's max_rows %d", M, kv->m->max_rows);
  if (M > kMaxPassRows) return fail(VS_E_SHAPE, "batch: %d rows in one pass exceed %d", M, kMaxPassRows);
  rm->M = M;
  rm->depth = b->d_depth;
  rm->mask = b->d_mask;
  return VS_OK;
}

// The pass's attention plan must fit the workspace (attn_plan).
vs_status check_attn_budget(vs_model* m, vs_kv* kv, const RowMap& rm) {
  AttnPlan pl;
  return attn_plan(m, kv, rm, &pl);
}

vs_status check_capacity(vs_kv* kv, const RowMap& rm) {
  vs_status rc = check_attn_budget(kv->m, kv, rm);
  if (rc != VS_OK) return rc;
  for (int i = 0; i < rm.n_seq; ++i) {
    const int s = rm.seq[i];
    const int last = kv->P_ub[s] + rm.win + rm.idx_off + (rm.row_start[i + 1] - rm.row_start[i]) - 1;
    if (last >= kv->cap[s])
      return fail(VS_E_NOKV, "sequence %d: slot %d beyond its capacity %d", s, last, kv->cap[s]);
  }
  return VS_OK;
}

}  // namespace

// ===========================================================================
extern "C" {

const char* vs_last_error(void) { return g_err.c_str(); }

size_t vs_weight_bytes(const vs_model_cfg* cfg) {
  if (cfg == nullptr || !shape_ok(cfg, nullptr)) return 0;
  return weight_layout(cfg).total;
}

size_t vs_workspace_bytes(const vs_model_cfg* cfg, int32_t max_rows, int32_t max_seqs, int32_t max_ctx) {
  if (cfg == nullptr || !shape_ok(cfg, nullptr) || max_rows < 1 || max_seqs < 1 || max_ctx < 1) return 0;
  return ws_layout(cfg, max_rows, max_seqs).total;
}

size_t vs_kv_bytes(const vs_model_cfg* cfg, int32_t n_blocks, int32_t max_seqs, int32_t max_blocks_per_seq) {
  if (cfg == nullptr || !shape_ok(cfg, nullptr) || n_blocks < 1 || max_seqs < 1 || max_blocks_per_seq < 1) return 0;
  const size_t pool = align256((size_t)n_blocks * cfg->n_kv_heads * kBlock * cfg->head_dim * 2);
  return pool * 2 * cfg->n_layers + align256((size_t)cfg->n_layers * 2 * sizeof(void*)) +
         align256((size_t)max_seqs * 4) * 3 + align256((size_t)max_seqs * max_blocks_per_seq * 4);
}

vs_status vs_model_create(const vs_model_cfg* cfg, void* d_weights, void* d_workspace, int32_t max_rows,
                          int32_t max_seqs, int32_t max_ctx, void* stream, vs_model** out) {
  if (cfg == nullptr || out == nullptr || d_weights == nullptr || d_workspace == nullptr)
    return fail(VS_E_INVAL, "vs_model_create: null argument");
  std::string why;
  if (!shape_ok(cfg, &why)) return fail(VS_E_SHAPE, "vs_model_create: %s", why.c_str());
  if (max_rows < 1 || max_rows > kMaxPassRows || max_seqs < 1 || max_seqs > kMaxSeq || max_ctx < 1)
    return fail(VS_E_SHAPE, "vs_model_create: limits out of range");
  vs_model* m = new vs_model();
  m->c = *cfg;
  m->wl = weight_layout(cfg);
  m->wbase = static_cast<char*>(d_weights);
  const int d = cfg->d_model, hd = cfg->head_dim, H = cfg->n_heads, Hkv = cfg->n_kv_heads, F = cfg->d_ffn;
  auto mat = [&](size_t off, int N, int K) {
    Mat w;
    w.w = reinterpret_cast<uint16_t*>(m->wbase + off);
    w.n_tiles = N / 16;
    w.k_steps = K / 32;
    return w;
  };
  for (int l = 0; l < cfg->n_layers; ++l) {
    m->qkv.push_back(mat(m->wl.qkv[l], (H + 2 * Hkv) * hd, d));
    m->o.push_back(mat(m->wl.o[l], d, H * hd));
    m->gu.push_back(mat(m->wl.gu[l], 2 * F, d));
    m->down.push_back(mat(m->wl.down[l], d, F));
    m->g_attn.push_back(reinterpret_cast<float*>(m->wbase + m->wl.g_attn[l]));
    m->g_ffn.push_back(reinterpret_cast<float*>(m->wbase + m->wl.g_ffn[l]));
  }
  m->embed = reinterpret_cast<uint16_t*>(m->wbase + m->wl.embed);
  m->g_final = reinterpret_cast<float*>(m->wbase + m->wl.g_final);
  m->head = mat(m->wl.head, cfg->vocab, d);
  m->max_rows = max_rows;
  m->max_seqs = max_seqs;
  m->max_ctx = max_ctx;
  m->wsl = ws_layout(cfg, max_rows, max_seqs);
  m->ws = static_cast<char*>(d_workspace);
  char* w = m->ws;
  m->h = reinterpret_cast<float*>(w + m->wsl.h);
  m->xa_h = reinterpret_cast<uint16_t*>(w + m->wsl.xa_h);
  m->xa_o = reinterpret_cast<uint16_t*>(w + m->wsl.xa_o);
  m->xa_act = reinterpret_cast<uint16_t*>(w + m->wsl.xa_act);
  m->ss = reinterpret_cast<float*>(w + m->wsl.ss);
  m->rs = reinterpret_cast<float*>(w + m->wsl.rs);
  m->kpart = reinterpret_cast<float*>(w + m->wsl.kpart);
  m->kcnt = reinterpret_cast<unsigned*>(w + m->wsl.kcnt);
  m->q = reinterpret_cast<float*>(w + m->wsl.q);
  m->rope = reinterpret_cast<float2*>(w + m->wsl.rope);
  m->kvrow = reinterpret_cast<int*>(w + m->wsl.kvrow);
  m->part = reinterpret_cast<float*>(w + m->wsl.part);
  m->attn_cnt = reinterpret_cast<unsigned*>(w + m->wsl.attn_cnt);
  {
    char* t = w + m->wsl.tree;
    memset(&m->tree, 0, sizeof(m->tree));
    m->tree.score = reinterpret_cast<double*>(t);
    t += (size_t)kTreeNodes * 8;
    m->tree.tok = reinterpret_cast<int*>(t);
    m->tree.parent = m->tree.tok + kTreeNodes;
    m->tree.depth = m->tree.parent + kTreeNodes;
    m->tree.rank = m->tree.depth + kTreeNodes;
    m->tree.meta = m->tree.rank + kTreeNodes;
    m->tree.row_mask = reinterpret_cast<uint64_t*>(m->tree.meta + 64);
    m->tree.row_tok = reinterpret_cast<int*>(m->tree.row_mask + kMaxRows);
    m->tree.row_depth = m->tree.row_tok + kMaxRows;
    m->tree.row_node = m->tree.row_depth + kMaxRows;
    m->tree.row_parent = m->tree.row_node + kMaxRows;
  }
  m->amax_val = reinterpret_cast<float*>(w + m->wsl.amax_val);
  m->amax_idx = reinterpret_cast<int*>(w + m->wsl.amax_idx);
  m->logits = reinterpret_cast<float*>(w + m->wsl.logits);
  m->dlogits = reinterpret_cast<float*>(w + m->wsl.dlogits);
  m->hidden = reinterpret_cast<float*>(w + m->wsl.hidden);
  m->tokens = reinterpret_cast<int*>(w + m->wsl.tokens);
  m->st_mx = reinterpret_cast<float*>(w + m->wsl.st_mx);
  m->st_amax = reinterpret_cast<int*>(w + m->wsl.st_amax);
  m->st_second = reinterpret_cast<float*>(w + m->wsl.st_second);
  m->st_sum = reinterpret_cast<double*>(w + m->wsl.st_sum);
  m->dst_mx = reinterpret_cast<float*>(w + m->wsl.dst_mx);
  m->dst_amax = reinterpret_cast<int*>(w + m->wsl.dst_amax);
  m->dst_sum = reinterpret_cast<double*>(w + m->wsl.dst_sum);
  m->result = reinterpret_cast<int*>(w + m->wsl.result);
  m->conf = reinterpret_cast<double*>(w + m->wsl.conf);
  m->tp_key = reinterpret_cast<unsigned*>(w + m->wsl.tp_key);
  m->tp_id = reinterpret_cast<int*>(w + m->wsl.tp_id);
  m->tp_mass = reinterpret_cast<double*>(w + m->wsl.tp_mass);
  // the attention kernel's arrival counters start at zero and every launch
  // leaves them at zero
  hipError_t ae = hipMemset(m->attn_cnt, 0, kAttnMaxUnits * sizeof(unsigned));
  // so do the K-split GEMM's arrival counters
  if (ae == hipSuccess) ae = hipMemset(m->kcnt, 0, kGemmSplitCells * sizeof(unsigned));
  if (ae == hipSuccess) {
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n_cu > 0)
      m->n_cu = n_cu;
  }
  m->attn_split = default_attn_split(*cfg);
  if (ae == hipSuccess) ae = attn_init();
  if (ae != hipSuccess) {
    vs_model_destroy(m);
    (void)hipGetLastError();
    return fail(VS_E_DEVICE, "vs_model_create: attention set-up: %s", hipGetErrorString(ae));
  }
  vs_status rc = check_launch("vs_model_create");
  if (rc != VS_OK) {
    vs_model_destroy(m);
    return rc;
  }
  *out = m;
  return VS_OK;
}

vs_status vs_model_set_tensor(vs_model* m, int32_t tensor, int32_t layer, const void* d_src, void* stream) {
  if (m == nullptr || d_src == nullptr) return fail(VS_E_INVAL, "vs_model_set_tensor: null argument");
  if (tensor < 0 || tensor >= VS_T_COUNT) return fail(VS_E_INVAL, "vs_model_set_tensor: bad tensor id %d", tensor);
  const vs_model_cfg& c = m->c;
  const bool per_layer = !(tensor == VS_T_EMBED || tensor == VS_T_FINAL_NORM || tensor == VS_T_HEAD);
  if (per_layer && (layer < 0 || layer >= c.n_layers))
    return fail(VS_E_INVAL, "vs_model_set_tensor: layer %d out of range", layer);
  const int d = c.d_model, hd = c.head_dim, H = c.n_heads, Hkv = c.n_kv_heads, F = c.d_ffn, V = c.vocab;
  const uint16_t* src = static_cast<const uint16_t*>(d_src);
  hipStream_t st = S(stream);
  PackArgs p;
  memset(&p, 0, sizeof(p));
  p.src = src;
  p.hd = hd;
  auto pack = [&](const Mat& W, int rows, int K, int row_off, int map) {
    p.dst = W.w;
    p.rows = rows;
    p.K = K;
    p.k_steps = K / 32;
    p.row_off = row_off;
    p.map = map;
    p.wide32 = gemm_wide32(W.n_tiles, W.k_steps) ? 1 : 0;
    launch_pack(p, st);
  };
  switch (tensor) {
    case VS_T_EMBED: {
      const hipError_t e = hipMemcpyAsync(m->embed, src, (size_t)V * d * 2, hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return fail(VS_E_DEVICE, "vs_model_set_tensor: %s", hipGetErrorString(e));
      break;
    }
    case VS_T_ATTN_NORM: launch_bf16_to_f32(src, m->g_attn[layer], d, st); break;
    case VS_T_FFN_NORM: launch_bf16_to_f32(src, m->g_ffn[layer], d, st); break;
    case VS_T_FINAL_NORM: launch_bf16_to_f32(src, m->g_final, d, st); break;
    case VS_T_WQ: pack(m->qkv[layer], H * hd, d, 0, PACK_HEADS); break;
    case VS_T_WK: pack(m->qkv[layer], Hkv * hd, d, H * hd, PACK_HEADS); break;
    case VS_T_WV: pack(m->qkv[layer], Hkv * hd, d, (H + Hkv) * hd, PACK_HEADS); break;
    case VS_T_WO: pack(m->o[layer], d, H * hd, 0, PACK_IDENTITY); break;
    case VS_T_W_GATE: pack(m->gu[layer], F, d, 0, PACK_EVEN); break;
    case VS_T_W_UP: pack(m->gu[layer], F, d, 0, PACK_ODD); break;
    case VS_T_W_DOWN: pack(m->down[layer], d, F, 0, PACK_IDENTITY); break;
    case VS_T_HEAD: pack(m->head, V, d, 0, PACK_IDENTITY); break;
  }
  return check_launch("vs_model_set_tensor");
}

void vs_model_destroy(vs_model* m) {
  if (!m) return;
  for (auto e : m->ev_pool) (void)hipEventDestroy(e);  // nothing to report from a destructor
  delete m;
}

vs_status vs_model_set_attn_split(vs_model* m, int32_t keys) {
  if (m == nullptr) return fail(VS_E_INVAL, "vs_model_set_attn_split: null model");
  if (keys < kAttnStepKeys || keys > kAttnGroupMaxKps || keys % kAttnStepKeys != 0)
    return fail(VS_E_INVAL, "vs_model_set_attn_split: %d keys (a multiple of %d in [%d, %d])", keys, kAttnStepKeys,
                kAttnStepKeys, kAttnGroupMaxKps);
  m->attn_split = keys;
  return VS_OK;
}

int32_t vs_model_attn_split(const vs_model* m) { return m == nullptr ? 0 : m->attn_split; }

vs_status vs_kv_create(vs_model* m, void* d_kv, int32_t n_blocks, int32_t max_seqs, int32_t max_blocks_per_seq,
                       void* stream, vs_kv** out) {
  if (m == nullptr || d_kv == nullptr || out == nullptr) return fail(VS_E_INVAL, "vs_kv_create: null argument");
  if (n_blocks < 1 || max_seqs < 1 || max_seqs > 4096 || max_blocks_per_seq < 1)
    return fail(VS_E_SHAPE, "vs_kv_create: limits out of range");
  const vs_model_cfg& c = m->c;
  vs_kv* kv = new vs_kv();
  kv->m = m;
  kv->base = static_cast<char*>(d_kv);
  kv->n_blocks = n_blocks;
  kv->max_seqs = max_seqs;
  kv->bps = max_blocks_per_seq;
  const size_t pool = align256((size_t)n_blocks * c.n_kv_heads * kBlock * c.head_dim * 2);
  size_t off = 0;
  for (int l = 0; l < c.n_layers; ++l) {
    kv->k.push_back(reinterpret_cast<uint16_t*>(kv->base + off));
    off += pool;
    kv->v.push_back(reinterpret_cast<uint16_t*>(kv->base + off));
    off += pool;
  }
  kv->d_kptr = reinterpret_cast<uint16_t**>(kv->base + off);
  kv->d_vptr = kv->d_kptr + c.n_layers;
  off += align256((size_t)c.n_layers * 2 * sizeof(void*));
  kv->P = reinterpret_cast<int*>(kv->base + off);
  off += align256((size_t)max_seqs * 4);
  kv->pending = reinterpret_cast<int*>(kv->base + off);
  off += align256((size_t)max_seqs * 4);
  kv->committed = reinterpret_cast<int*>(kv->base + off);
  off += align256((size_t)max_seqs * 4);
  kv->bt = reinterpret_cast<int*>(kv->base + off);
  std::vector<uint16_t*> ptrs(kv->k);
  ptrs.insert(ptrs.end(), kv->v.begin(), kv->v.end());
  hipStream_t st = S(stream);
  hipError_t e = hipMemcpyAsync(kv->d_kptr, ptrs.data(), ptrs.size() * sizeof(void*), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);  // the host vector goes out of scope
  if (e != hipSuccess) {
    delete kv;
    return fail(VS_E_DEVICE, "vs_kv_create: %s", hipGetErrorString(e));
  }
  launch_fill_i32(kv->P, 0, max_seqs, st);
  launch_fill_i32(kv->pending, -1, max_seqs, st);
  launch_fill_i32(kv->committed, 0, max_seqs, st);
  launch_fill_i32(kv->bt, 0, (size_t)max_seqs * max_blocks_per_seq, st);
  for (int b = n_blocks - 1; b >= 0; --b) kv->free_blocks.push_back(b);
  kv->blocks.resize(max_seqs);
  kv->open.assign(max_seqs, 0);
  kv->cap.assign(max_seqs, 0);
  kv->P_ub.assign(max_seqs, 0);
  kv->prefilled.assign(max_seqs, 0);
  kv->commit_no.assign(max_seqs, 0);
  kv->base_no.assign(max_seqs, 1);
  kv->P_base.assign(max_seqs, 0);
  kv->P_known.assign(max_seqs, 0);
  kv->in_flight.resize(max_seqs);
  if (hipHostMalloc(reinterpret_cast<void**>(&kv->mirror), (size_t)max_seqs * 8, hipHostMallocCoherent) != hipSuccess) {
    (void)hipGetLastError();
    delete kv;
    return fail(VS_E_DEVICE, "vs_kv_create: pinned host mirror of the KV lengths");
  }
  memset(kv->mirror, 0, (size_t)max_seqs * 8);
  vs_status rc = check_launch("vs_kv_create");
  if (rc != VS_OK) {
    delete kv;
    return rc;
  }
  *out = kv;
  return VS_OK;
}

void vs_kv_destroy(vs_kv* kv) {
  if (kv == nullptr) return;
  if (kv->mirror != nullptr) {
    (void)hipDeviceSynchronize();  // no commit kernel may still write it
    (void)hipHostFree(kv->mirror);
  }
  delete kv;
}

vs_status vs_seq_open(vs_kv* kv, int32_t max_len, void* stream, int32_t* seq_id) {
  if (kv == nullptr || seq_id == nullptr) return fail(VS_E_INVAL, "vs_seq_open: null argument");
  if (max_len < 1) return fail(VS_E_INVAL, "vs_seq_open: max_len %d", max_len);
  const int nb = (max_len + kBlock - 1) / kBlock;
  if (nb > kv->bps) return fail(VS_E_NOKV, "vs_seq_open: %d blocks exceed %d per sequence", nb, kv->bps);
  if ((int)kv->free_blocks.size() < nb) return fail(VS_E_NOKV, "vs_seq_open: pool has %zu free blocks, %d needed",
                                                    kv->free_blocks.size(), nb);
  int s = -1;
  for (int i = 0; i < kv->max_seqs; ++i)
    if (!kv->open[i]) {
      s = i;
      break;
    }
  if (s < 0) return fail(VS_E_NOKV, "vs_seq_open: all %d sequence slots in use", kv->max_seqs);
  std::vector<int>& bl = kv->blocks[s];
  bl.clear();
  for (int i = 0; i < nb; ++i) {
    bl.push_back(kv->free_blocks.back());
    kv->free_blocks.pop_back();
  }
  hipStream_t st = S(stream);
  for (int first = 0; first < nb; first += 256) {
    BlockSetArgs a;
    memset(&a, 0, sizeof(a));
    a.bt = kv->bt;
    a.bps = kv->bps;
    a.seq = s;
    a.first = first;
    a.n = std::min(256, nb - first);
    a.reset_state = first == 0;
    a.P = kv->P;
    a.pending = kv->pending;
    a.committed = kv->committed;
    for (int i = 0; i < a.n; ++i) a.ids[i] = bl[first + i];
    launch_set_blocks(a, st);
  }
  vs_status rc = check_launch("vs_seq_open");
  if (rc != VS_OK) return rc;
  kv->open[s] = 1;
  kv->cap[s] = nb * kBlock;
  kv_set_exact(kv, s, 0);
  kv->prefilled[s] = 0;
  *seq_id = s;
  return VS_OK;
}

vs_status vs_seq_assume(vs_kv* kv, int32_t seq, int32_t P, int32_t pending, void* stream) {
  if (kv == nullptr) return fail(VS_E_INVAL, "vs_seq_assume: null argument");
  if (seq < 0 || seq >= kv->max_seqs || !kv->open[seq]) return fail(VS_E_STATE, "vs_seq_assume: sequence %d is not open", seq);
  if (kv->prefilled[seq]) return fail(VS_E_STATE, "vs_seq_assume: sequence %d already holds a context", seq);
  if (P < 0 || P >= kv->cap[seq]) return fail(VS_E_NOKV, "vs_seq_assume: length %d outside the capacity %d", P, kv->cap[seq]);
  if (pending < 0 || pending >= kv->m->c.vocab) return fail(VS_E_INVAL, "vs_seq_assume: pending token %d", pending);
  launch_set_state(kv->P, kv->pending, kv->committed, seq, P, pending, S(stream));
  vs_status rc = check_launch("vs_seq_assume");
  if (rc != VS_OK) return rc;
  kv_set_exact(kv, seq, P);
  kv->prefilled[seq] = 1;
  return VS_OK;
}

vs_status vs_seq_rewind(vs_kv* kv, int32_t seq, int32_t P, int32_t pending, void* stream) {
  if (kv == nullptr) return fail(VS_E_INVAL, "vs_seq_rewind: null argument");
  if (seq < 0 || seq >= kv->max_seqs || !kv->open[seq]) return fail(VS_E_STATE, "vs_seq_rewind: sequence %d is not open", seq);
  if (!kv->prefilled[seq]) return fail(VS_E_STATE, "vs_seq_rewind: sequence %d holds no context", seq);
  if (pending < 0 || pending >= kv->m->c.vocab) return fail(VS_E_INVAL, "vs_seq_rewind: pending token %d", pending);
  // the KV length lives on the device: read it back to check P exactly
  hipStream_t st = S(stream);
  int P_now = 0;
  hipError_t e = hipMemcpyAsync(&P_now, kv->P + seq, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(VS_E_DEVICE, "vs_seq_rewind: %s", hipGetErrorString(e));
  if (P < 0 || P > P_now) return fail(VS_E_NOKV, "vs_seq_rewind: length %d beyond the sequence's %d", P, P_now);
  launch_set_state(kv->P, kv->pending, kv->committed, seq, P, pending, st);
  vs_status rc = check_launch("vs_seq_rewind");
  if (rc != VS_OK) return rc;
  kv_set_exact(kv, seq, P);
  return VS_OK;
}

vs_status vs_seq_close(vs_kv* kv, int32_t seq_id) {
  if (kv == nullptr) return fail(VS_E_INVAL, "vs_seq_close: null argument");
  if (seq_id < 0 || seq_id >= kv->max_seqs || !kv->open[seq_id])
    return fail(VS_E_STATE, "vs_seq_close: sequence %d is not open", seq_id);
  for (int b : kv->blocks[seq_id]) kv->free_blocks.push_back(b);
  kv->blocks[seq_id].clear();
  kv->open[seq_id] = 0;
  return VS_OK;
}

vs_status vs_kv_state(vs_kv* kv, int32_t** d_P, int32_t** d_pending, int32_t** d_committed) {
  if (kv == nullptr) return fail(VS_E_INVAL, "vs_kv_state: null argument");
  if (d_P) *d_P = kv->P;
  if (d_pending) *d_pending = kv->pending;
  if (d_committed) *d_committed = kv->committed;
  return VS_OK;
}

vs_status vs_kv_layer(vs_kv* kv, int32_t layer, void** d_k, void** d_v, int32_t** d_block_table) {
  if (kv == nullptr) return fail(VS_E_INVAL, "vs_kv_layer: null argument");
  if (layer < 0 || layer >= kv->m->c.n_layers) return fail(VS_E_INVAL, "vs_kv_layer: layer %d", layer);
  if (d_k) *d_k = kv->k[layer];
  if (d_v) *d_v = kv->v[layer];
  if (d_block_table) *d_block_table = kv->bt;
  return VS_OK;
}

vs_status vs_kv_sync(vs_kv* kv, void* stream) {
  if (kv == nullptr) return fail(VS_E_INVAL, "vs_kv_sync: null argument");
  std::vector<int> P(kv->max_seqs);
  hipError_t e = hipMemcpyAsync(P.data(), kv->P, kv->max_seqs * 4, hipMemcpyDeviceToHost, S(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(S(stream));
  if (e != hipSuccess) return fail(VS_E_DEVICE, "vs_kv_sync: %s", hipGetErrorString(e));
  for (int s = 0; s < kv->max_seqs; ++s)
    if (kv->open[s]) kv_set_exact(kv, s, P[s]);
  return VS_OK;
}

vs_status vs_forward_layers(vs_model* m, vs_kv* kv, const vs_batch* b, int32_t start, int32_t end,
                            const int32_t* d_tokens, const float* d_hidden_in, float* d_hidden_out, void* stream) {
  if (m == nullptr || kv == nullptr) return fail(VS_E_INVAL, "vs_forward_layers: null handle");
  if (start < 0 || end > m->c.n_layers || start > end) return fail(VS_E_INVAL, "vs_forward_layers: bad layer range");
  if (start == 0 && d_tokens == nullptr) return fail(VS_E_INVAL, "vs_forward_layers: tokens needed at start 0");
  if (start > 0 && d_hidden_in == nullptr) return fail(VS_E_INVAL, "vs_forward_layers: hidden rows needed");
  RowMap rm;
  vs_status rc = batch_rowmap(kv, b, &rm);
  if (rc != VS_OK) return rc;
  if ((rc = check_capacity(kv, rm)) != VS_OK) return rc;
  hipStream_t st = S(stream);
  const float* g0 = start < end ? m->g_attn[start] : m->g_final;
  load_rows(m, rm.M, start == 0 ? d_tokens : nullptr, d_hidden_in, nullptr, g0, st, &rm, kv);
  run_layers(m, kv, rm, start, end, st, nullptr, nullptr);
  if (d_hidden_out) launch_copy_rows(m->h, d_hidden_out, rm.M, m->c.d_model, st);
  return check_launch("vs_forward_layers");
}

vs_status vs_head(vs_model* m, int32_t M, const float* d_hidden, float* d_logits, void* stream) {
  if (m == nullptr || d_hidden == nullptr || d_logits == nullptr) return fail(VS_E_INVAL, "vs_head: null argument");
  if (M < 1 || M > m->max_rows) return fail(VS_E_SHAPE, "vs_head: %d rows", M);
  hipStream_t st = S(stream);
  load_rows(m, M, nullptr, d_hidden, nullptr, m->g_final, st);
  run_head(m, M, d_logits, nullptr, st);
  return check_launch("vs_head");
}

vs_status vs_prefill(vs_model* m, vs_kv* kv, int32_t seq, const int32_t* d_tokens, int32_t n, int32_t mode,
                     float temp, const double* d_u, float* d_logits_last, void* stream) {
  if (m == nullptr || kv == nullptr || d_tokens == nullptr) return fail(VS_E_INVAL, "vs_prefill: null argument");
  if (seq < 0 || seq >= kv->max_seqs || !kv->open[seq]) return fail(VS_E_STATE, "vs_prefill: sequence not open");
  if (kv->prefilled[seq]) return fail(VS_E_STATE, "vs_prefill: sequence %d already prefilled", seq);
  if (n < 1) return fail(VS_E_INVAL, "vs_prefill: n = %d", n);
  if (mode != VS_GREEDY && mode != VS_SAMPLE) return fail(VS_E_INVAL, "vs_prefill: mode %d", mode);
  if (mode == VS_SAMPLE && (d_u == nullptr || !(temp > 0.f))) return fail(VS_E_INVAL, "vs_prefill: sampling needs u, T>0");
  if (n + 1 > kv->cap[seq]) return fail(VS_E_NOKV, "vs_prefill: %d tokens exceed capacity %d", n, kv->cap[seq]);
  const int chunk = std::min(kMaxRows, m->max_rows);
  {  // the last chunk's attention plan bounds the others' (same rows or fewer, shorter contexts)
    const int nc = n - (n - 1) / chunk * chunk;
    RowMap rm;
    memset(&rm, 0, sizeof(rm));
    rm.n_seq = 1;
    rm.M = chunk;
    rm.seq[0] = seq;
    rm.row_start[1] = chunk;
    const int saved = kv->P_ub[seq];
    kv->P_ub[seq] = n - nc;
    vs_status rc = check_attn_budget(m, kv, rm);
    kv->P_ub[seq] = saved;
    if (rc != VS_OK) return rc;
  }
  hipStream_t st = S(stream);
  for (int c0 = 0; c0 < n; c0 += chunk) {
    const int nc = std::min(chunk, n - c0);
    RowMap rm;
    memset(&rm, 0, sizeof(rm));
    rm.n_seq = 1;
    rm.M = nc;
    rm.seq[0] = seq;
    rm.row_start[1] = nc;
    load_rows(m, nc, d_tokens + c0, nullptr, nullptr, m->g_attn[0], st, &rm, kv);
    run_layers(m, kv, rm, 0, m->c.n_layers, st, nullptr, nullptr);
    const bool last = c0 + nc == n;
    if (last) run_head(m, nc, m->logits, nullptr, st);
    launch_advance(kv->P, kv->committed, seq, nc, nc + (last ? 1 : 0), st);
    kv->P_ub[seq] += nc;
    if (last) {
      PickArgs p;
      memset(&p, 0, sizeof(p));
      p.n = 1;
      p.mode = mode;
      p.temp = temp;
      p.slot = 32;
      p.pending = kv->pending;
      p.amax_val = m->amax_val;
      p.amax_idx = m->amax_idx;
      p.groups = m->head_groups;
      p.Mprev = nc;
      p.logits = m->logits;
      p.V = m->c.vocab;
      p.u = d_u;
      p.tokens = kv->pending;
      p.seq[0] = seq;
      p.src[0] = nc - 1;
      p.lrow[0] = nc - 1;
      p.uidx[0] = 0;
      p.dst[0] = seq;
      launch_pick(p, st);
      if (d_logits_last) {
        const hipError_t e = hipMemcpyAsync(d_logits_last, m->logits + (size_t)(nc - 1) * m->c.vocab,
                                            (size_t)m->c.vocab * 4, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return fail(VS_E_DEVICE, "vs_prefill: %s", hipGetErrorString(e));
      }
    }
  }
  kv->prefilled[seq] = 1;
  kv_set_exact(kv, seq, kv->P_ub[seq]);  // the prompt's length, exactly
  return check_launch("vs_prefill");
}

}  // extern "C"

namespace {

vs_status validate_chain(vs_model* m, vs_kv* kv, int n_seq, const int32_t* seq, const int32_t* k, int mode,
                         float temp, const double* d_u, int* M_out) {
  if (n_seq < 1 || n_seq > kMaxSeq) return fail(VS_E_SHAPE, "n_seq %d not in [1, %d]", n_seq, kMaxSeq);
  if (seq == nullptr || k == nullptr) return fail(VS_E_INVAL, "null seq or k");
  if (mode != VS_GREEDY && mode != VS_SAMPLE) return fail(VS_E_INVAL, "mode %d", mode);
  if (mode == VS_SAMPLE && (d_u == nullptr || !(temp > 0.f))) return fail(VS_E_INVAL, "sampling needs u and T > 0");
  int M = 0;
  for (int i = 0; i < n_seq; ++i) {
    const int s = seq[i];
    if (s < 0 || s >= kv->max_seqs || !kv->open[s]) return fail(VS_E_STATE, "sequence %d is not open", s);
    if (!kv->prefilled[s]) return fail(VS_E_STATE, "sequence %d has no prefill", s);
    kv_refresh(kv, s);
    for (int j = 0; j < i; ++j)
      if (seq[j] == s) return fail(VS_E_INVAL, "sequence %d listed twice", s);
    if (k[i] < 0 || k[i] > VS_MAX_K) return fail(VS_E_INVAL, "k = %d not in [0, %d]", k[i], VS_MAX_K);
    if (kv->P_ub[s] + k[i] + 1 > kv->cap[s]) return fail(VS_E_NOKV, "sequence %d: capacity %d reached", s, kv->cap[s]);
    M += k[i] + 1;
  }
  if (M > m->max_rows || M > kMaxPassRows) return fail(VS_E_SHAPE, "%d verify rows exceed max_rows %d", M, m->max_rows);
  // the verify pass's attention plan bounds the draft steps' (fewer rows,
  // the same contexts)
  RowMap rm;
  memset(&rm, 0, sizeof(rm));
  rm.n_seq = n_seq;
  for (int i = 0; i < n_seq; ++i) {
    rm.seq[i] = seq[i];
    rm.row_start[i + 1] = rm.row_start[i] + k[i] + 1;
  }
  rm.M = M;
  vs_status rc = check_attn_budget(m, kv, rm);
  if (rc != VS_OK) return rc;
  *M_out = M;
  return VS_OK;
}

void chain_batch_rowmap(const int n_seq, const int32_t* seq, const int32_t* k, RowMap* rm) {
  memset(rm, 0, sizeof(*rm));
  rm->n_seq = n_seq;
  int M = 0;
  for (int i = 0; i < n_seq; ++i) {
    rm->seq[i] = seq[i];
    rm->row_start[i] = M;
    M += k[i] + 1;
  }
  rm->row_start[n_seq] = M;
  rm->M = M;
}

void draft_impl(vs_model* m, vs_kv* kv, int n_seq, const int32_t* seq, const int32_t* k, int mode, float temp,
                const double* d_u, int32_t* d_tokens, float* d_hidden_L, float* d_draft_logits, hipStream_t st) {
  const int L = m->c.exit_layer;
  std::vector<int> vstart(n_seq);
  int kmax = 0, M = 0;
  for (int i = 0; i < n_seq; ++i) {
    vstart[i] = M;
    M += k[i] + 1;
    kmax = std::max(kmax, (int)k[i]);
  }
  std::vector<int> prev;  // active sequences (indices) of the previous step
  for (int s = 0; s <= kmax; ++s) {
    std::vector<int> act;
    for (int i = 0; i < n_seq; ++i)
      if (k[i] >= s) act.push_back(i);
    const int Ma = (int)act.size();
    PickArgs p;
    memset(&p, 0, sizeof(p));
    p.n = Ma;
    p.mode = mode;
    p.temp = temp;
    p.slot = s - 1;
    p.pending = kv->pending;
    p.amax_val = m->amax_val;
    p.amax_idx = m->amax_idx;
    p.groups = m->head_groups;
    p.Mprev = (int)prev.size();
    p.logits = d_draft_logits;
    p.V = m->c.vocab;
    p.u = d_u;
    p.tokens = d_tokens;
    std::vector<int> rows_src(Ma), rows_out(Ma), logit_rows(Ma);
    for (int a = 0; a < Ma; ++a) {
      const int i = act[a];
      p.seq[a] = seq[i];
      p.src[a] = -1;
      if (s > 0)
        for (int b = 0; b < (int)prev.size(); ++b)
          if (prev[b] == i) p.src[a] = b;
      p.lrow[a] = vstart[i] + s - 1;
      p.uidx[a] = i;
      p.dst[a] = vstart[i] + s;
      rows_src[a] = vstart[i] + s;
      logit_rows[a] = k[i] > s ? vstart[i] + s : -1;
    }
    timed(m, F_SMALL, 0, st, [&](hipEvent_t, hipEvent_t) { launch_pick(p, st); });
    RowMap rm;
    memset(&rm, 0, sizeof(rm));
    rm.n_seq = Ma;
    rm.M = Ma;
    rm.idx_off = s;
    for (int a = 0; a < Ma; ++a) {
      rm.seq[a] = seq[act[a]];
      rm.row_start[a] = a;
    }
    rm.row_start[Ma] = Ma;
    load_rows(m, Ma, d_tokens, nullptr, rows_src.data(), L > 0 ? m->g_attn[0] : m->g_final, st, &rm, kv);
    if (L > 0) {
      run_layers(m, kv, rm, 0, L, st, d_hidden_L, rows_src.data());
    } else {
      // with L = 0 the layer-L input is the embedding itself; a failed copy
      // is reported by the caller's check_launch (hipGetLastError returns
      // the last failing call's code)
      for (int a = 0; a < Ma; ++a)
        (void)hipMemcpyAsync(d_hidden_L + (size_t)rows_src[a] * m->c.d_model, m->h + (size_t)a * m->c.d_model,
                             (size_t)m->c.d_model * 4, hipMemcpyDeviceToDevice, st);
    }
    bool need_head = false;
    for (int a = 0; a < Ma; ++a) need_head |= k[act[a]] > s;
    if (need_head) run_head(m, Ma, d_draft_logits, logit_rows.data(), st);
    prev = act;
  }
}

// Tree draft of one sequence: level passes (layers 0..L-1 + head over the
// root and the kept nodes) grow the tree; a final first-L pass over the
// final rows writes their KV at slots P + row and their layer-L inputs.
void draft_tree_impl(vs_model* m, vs_kv* kv, int seq, int topk, int depth, int keep, float temp, int32_t* d_tokens,
                     int32_t* d_depth, uint64_t* d_mask, int32_t* d_parent, float* d_hidden_L, float* d_level_logits,
                     hipStream_t st) {
  const int L = m->c.exit_layer, V = m->c.vocab, R = 1 + keep;
  TreeArgs ta = m->tree;
  ta.R = R;
  ta.max_depth = depth;
  ta.topk = topk;
  ta.keep = keep;
  ta.pending = kv->pending;
  ta.seq = seq;
  ta.V = V;
  ta.temp = temp;
  RowMap rm;
  memset(&rm, 0, sizeof(rm));
  rm.n_seq = 1;
  rm.M = R;
  rm.seq[0] = seq;
  rm.row_start[1] = R;
  rm.depth = ta.row_depth;
  rm.mask = ta.row_mask;
  const float* g0 = L > 0 ? m->g_attn[0] : m->g_final;
  for (int lev = 0; lev <= depth; ++lev) {
    ta.level = lev;
    const bool last = lev == depth;
    if (last) {
      ta.out_tok = d_tokens;
      ta.out_depth = d_depth;
      ta.out_mask = d_mask;
      ta.out_parent = d_parent;
    }
    timed(m, F_SMALL, 0, st, [&](hipEvent_t, hipEvent_t) { launch_tree_select(ta, st); });
    load_rows(m, R, ta.row_tok, nullptr, nullptr, g0, st, &rm, kv);
    if (L > 0) run_layers(m, kv, rm, 0, L, st, last ? d_hidden_L : nullptr, nullptr);
    if (last) {
      if (L == 0) launch_copy_rows(m->h, d_hidden_L, R, m->c.d_model, st);
      break;
    }
    float* z = d_level_logits != nullptr ? d_level_logits + (size_t)lev * R * V : m->dlogits;
    run_head(m, R, z, nullptr, st);
    ta.logits = z;
    timed(m, F_SMALL, 0, st, [&](hipEvent_t, hipEvent_t) { launch_tree_expand(ta, st); });
  }
}

}  // namespace

extern "C" {

vs_status vs_draft_tree(vs_model* m, vs_kv* kv, int32_t seq, int32_t topk, int32_t depth, int32_t keep, float temp,
                        int32_t* d_tokens, int32_t* d_depth, uint64_t* d_mask, int32_t* d_parent, float* d_hidden_L,
                        float* d_level_logits, void* stream) {
  if (m == nullptr || kv == nullptr || d_tokens == nullptr || d_depth == nullptr || d_mask == nullptr ||
      d_parent == nullptr || d_hidden_L == nullptr)
    return fail(VS_E_INVAL, "vs_draft_tree: null argument");
  if (seq < 0 || seq >= kv->max_seqs || !kv->open[seq]) return fail(VS_E_STATE, "vs_draft_tree: sequence %d is not open", seq);
  if (!kv->prefilled[seq]) return fail(VS_E_STATE, "vs_draft_tree: sequence %d has no prefill", seq);
  kv_refresh(kv, seq);
  if (topk < 1 || topk > kTreeMaxTopk) return fail(VS_E_INVAL, "vs_draft_tree: topk %d not in [1, %d]", topk, kTreeMaxTopk);
  if (depth < 1 || depth > kTreeMaxDepth)
    return fail(VS_E_INVAL, "vs_draft_tree: depth %d not in [1, %d]", depth, kTreeMaxDepth);
  if (keep < 1 || 1 + keep > kMaxRows || 1 + keep > m->max_rows)
    return fail(VS_E_SHAPE, "vs_draft_tree: %d kept nodes need %d rows (max_rows %d)", keep, 1 + keep, m->max_rows);
  if (1 + (size_t)topk * (1 + (size_t)(depth - 1) * keep) > (size_t)kTreeNodes)
    return fail(VS_E_SHAPE, "vs_draft_tree: expansion may exceed %d nodes", kTreeNodes);
  if (!(temp > 0.f)) return fail(VS_E_INVAL, "vs_draft_tree: temperature must be positive");
  RowMap rm;
  memset(&rm, 0, sizeof(rm));
  rm.n_seq = 1;
  rm.M = 1 + keep;
  rm.seq[0] = seq;
  rm.row_start[1] = 1 + keep;
  vs_status rc = check_capacity(kv, rm);
  if (rc != VS_OK) return rc;
  draft_tree_impl(m, kv, seq, topk, depth, keep, temp, d_tokens, d_depth, d_mask, d_parent, d_hidden_L, d_level_logits,
                  S(stream));
  return check_launch("vs_draft_tree");
}

vs_status vs_draft(vs_model* m, vs_kv* kv, int32_t n_seq, const int32_t* seq, const int32_t* k, int32_t mode,
                   float temp, const double* d_u, int32_t* d_tokens, float* d_hidden_L, float* d_draft_logits,
                   void* stream) {
  if (m == nullptr || kv == nullptr || d_tokens == nullptr || d_hidden_L == nullptr)
    return fail(VS_E_INVAL, "vs_draft: null argument");
  int M = 0;
  vs_status rc = validate_chain(m, kv, n_seq, seq, k, mode, temp, d_u, &M);
  if (rc != VS_OK) return rc;
  if (mode == VS_SAMPLE && d_draft_logits == nullptr) return fail(VS_E_INVAL, "vs_draft: sampling needs draft logits");
  draft_impl(m, kv, n_seq, seq, k, mode, temp, d_u, d_tokens, d_hidden_L, d_draft_logits, S(stream));
  return check_launch("vs_draft");
}

vs_status vs_verify(vs_model* m, vs_kv* kv, const vs_batch* b, int32_t start_layer, const int32_t* d_tokens,
                    const float* d_hidden_in, float* d_logits, void* stream) {
  if (m == nullptr || kv == nullptr || d_logits == nullptr) return fail(VS_E_INVAL, "vs_verify: null argument");
  if (start_layer < 0 || start_layer > m->c.n_layers) return fail(VS_E_INVAL, "vs_verify: start_layer %d", start_layer);
  if (start_layer == 0 && d_tokens == nullptr) return fail(VS_E_INVAL, "vs_verify: tokens needed at start 0");
  if (start_layer > 0 && d_hidden_in == nullptr) return fail(VS_E_INVAL, "vs_verify: hidden rows needed");
  RowMap rm;
  vs_status rc = batch_rowmap(kv, b, &rm);
  if (rc != VS_OK) return rc;
  if ((rc = check_capacity(kv, rm)) != VS_OK) return rc;
  hipStream_t st = S(stream);
  const int N = m->c.n_layers;
  load_rows(m, rm.M, start_layer == 0 ? d_tokens : nullptr, d_hidden_in, nullptr,
            start_layer < N ? m->g_attn[start_layer] : m->g_final, st, &rm, kv);
  run_layers(m, kv, rm, start_layer, N, st, nullptr, nullptr);
  run_head(m, rm.M, d_logits, nullptr, st);
  return check_launch("vs_verify");
}

}  // extern "C"

namespace {

// Per-row statistics the accept kernels use (target, draft, top-p set).
struct AcceptBufs {
  float *mx, *second, *dmx;
  int *amax, *damax;
  double *sum, *dsum, *tp_mass;
  unsigned* tp_key;
  int* tp_id;
};

// The accept step over a batch's rows: vocabulary statistics of the target
// (and of the draft when sampling), the top-p set when top_p < 1, then the
// acceptance kernel.  m (optional) times the launches.
vs_status accept_core(vs_model* m, const AcceptBufs& bf, int V, int max_rows, const char* name, const vs_batch* b,
                      int32_t mode, float temp, double top_p, const int32_t* d_tokens, const float* d_logits,
                      const float* d_draft_logits, const double* d_u, int32_t* d_result, hipStream_t st) {
  if (d_tokens == nullptr || d_logits == nullptr || d_result == nullptr || b == nullptr || b->seq == nullptr ||
      b->n_rows == nullptr)
    return fail(VS_E_INVAL, "%s: null argument", name);
  if (mode != VS_GREEDY && mode != VS_SAMPLE) return fail(VS_E_INVAL, "%s: mode %d", name, mode);
  if (b->n_seq < 1 || b->n_seq > kMaxSeq) return fail(VS_E_SHAPE, "%s: n_seq %d", name, b->n_seq);
  if (mode == VS_SAMPLE) {
    if (d_draft_logits == nullptr || d_u == nullptr || !(temp > 0.f))
      return fail(VS_E_INVAL, "%s: sampling needs draft logits, u and T > 0", name);
    if (b->d_mask != nullptr || b->d_depth != nullptr) return fail(VS_E_INVAL, "%s: sampling is chain-only", name);
  }
  RowMap rm;
  memset(&rm, 0, sizeof(rm));
  rm.n_seq = b->n_seq;
  int M = 0;
  for (int i = 0; i < b->n_seq; ++i) {
    if (b->n_rows[i] < 1 || b->n_rows[i] > kMaxRows) return fail(VS_E_SHAPE, "%s: rows %d", name, b->n_rows[i]);
    rm.seq[i] = b->seq[i];
    rm.row_start[i] = M;
    M += b->n_rows[i];
  }
  rm.row_start[b->n_seq] = M;
  rm.M = M;
  rm.mask = b->d_mask;
  rm.depth = b->d_depth;
  if (M > max_rows) return fail(VS_E_SHAPE, "%s: %d rows exceed the limit of %d", name, M, max_rows);
  auto run = [&](double bytes, auto launch) {
    if (m != nullptr) timed(m, F_SMALL, bytes, st, [&](hipEvent_t, hipEvent_t) { launch(); });
    else launch();
  };
  StatsArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.logits = d_logits;
  sa.V = V;
  sa.temp = mode == VS_SAMPLE ? temp : 1.0f;
  sa.mx = bf.mx;
  sa.amax = bf.amax;
  sa.second = bf.second;
  sa.sumexp = mode == VS_SAMPLE ? bf.sum : nullptr;
  if (mode == VS_SAMPLE) {  // the target's and the draft's statistics in one launch
    StatsArgs da = sa;
    da.logits = d_draft_logits;
    da.mx = bf.dmx;
    da.amax = bf.damax;
    da.second = nullptr;
    da.sumexp = bf.dsum;
    run((double)M * V * 8, [&]() { launch_row_stats2(sa, da, M, st); });
  } else {
    run((double)M * V * 4, [&]() { launch_row_stats(sa, M, st); });
  }
  const bool tp = top_p < 1.0;
  if (tp) {
    TopPArgs ta;
    ta.logits = d_logits;
    ta.V = V;
    ta.temp = temp;
    ta.top_p = top_p;
    ta.mx = bf.mx;
    ta.key = bf.tp_key;
    ta.id = bf.tp_id;
    ta.mass = bf.tp_mass;
    run((double)M * V * 4, [&]() { launch_top_p(ta, M, st); });
  }
  AcceptArgs a;
  memset(&a, 0, sizeof(a));
  if (tp) {
    a.tp_key = bf.tp_key;
    a.tp_id = bf.tp_id;
    a.tp_mass = bf.tp_mass;
  }
  a.rows = rm;
  a.mode = mode;
  a.temp = temp;
  a.tokens = d_tokens;
  a.logits = d_logits;
  a.dlogits = d_draft_logits;
  a.mx = bf.mx;
  a.amax = bf.amax;
  a.second = bf.second;
  a.sumexp = bf.sum;
  a.dmx = bf.dmx;
  a.dsumexp = bf.dsum;
  a.V = V;
  a.u = d_u;
  a.result = d_result;
  run(0, [&]() { launch_accept(a, st); });
  return check_launch(name);
}

AcceptBufs model_accept_bufs(vs_model* m) {
  AcceptBufs bf;
  bf.mx = m->st_mx;
  bf.amax = m->st_amax;
  bf.second = m->st_second;
  bf.sum = m->st_sum;
  bf.dmx = m->dst_mx;
  bf.damax = m->dst_amax;
  bf.dsum = m->dst_sum;
  bf.tp_key = m->tp_key;
  bf.tp_id = m->tp_id;
  bf.tp_mass = m->tp_mass;
  return bf;
}

vs_status accept_impl(vs_model* m, const vs_batch* b, int32_t mode, float temp, double top_p, const int32_t* d_tokens,
                      const float* d_logits, const float* d_draft_logits, const double* d_u, int32_t* d_result,
                      void* stream) {
  const char* name = top_p < 1.0 ? "vs_accept_top_p" : "vs_accept";
  if (m == nullptr) return fail(VS_E_INVAL, "%s: null model", name);
  return accept_core(m, model_accept_bufs(m), m->c.vocab, m->max_rows, name, b, mode, temp, top_p, d_tokens, d_logits,
                     d_draft_logits, d_u, d_result, S(stream));
}

}  // namespace

extern "C" {

}  // extern "C"

// ---- allocation-free accept ----------------------------------------------
// vs_accept_noalloc keeps the per-row statistics of the accept kernels in a
// file-scope device array instead of a model workspace, for up to
// kNoAllocRows rows.  In host code the array's name is only a stand-in: its
// device address, one per GPU, comes from hipGetSymbolAddress on the first
// call on that GPU, and only that address is handed to kernels.  Every
// field is written by the statistics kernels before it is read, so nothing
// needs clearing; calls that overlap on one GPU share the array and race.
namespace {

constexpr int kNoAllocRows = VS_MAX_PASS_ROWS;
constexpr size_t kNaSlot4 = (size_t(kNoAllocRows) * 4 + 255) / 256 * 256;  // one 4-byte field per row
constexpr size_t kNaSlot8 = (size_t(kNoAllocRows) * 8 + 255) / 256 * 256;  // one 8-byte field per row
constexpr size_t kNoAllocBytes = 7 * kNaSlot4 + 3 * kNaSlot8;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

std::mutex g_scratch_mu;
unsigned char* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch`, per GPU

// Device address of `scratch` on the current GPU, looked up once per GPU.
vs_status scratch_address(unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VS_E_DEVICE, "vs_accept_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(VS_E_DEVICE, "vs_accept_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(VS_E_DEVICE, "vs_accept_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_dev[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch_dev[dev];
  return VS_OK;
}

}  // namespace

extern "C" {

vs_status vs_accept_noalloc(int32_t vocab, const vs_batch* b, int32_t mode, float temp, const int32_t* d_tokens,
                            const float* d_logits, const float* d_draft_logits, const double* d_u, int32_t* d_result,
                            void* stream) {
  if (vocab < 16 || vocab > 32768 || vocab % 16 != 0)
    return fail(VS_E_SHAPE, "vs_accept_noalloc: vocab %d (a multiple of 16 in [16, 32768])", vocab);
  unsigned char* base = nullptr;
  vs_status rc = scratch_address(&base);
  if (rc != VS_OK) return rc;
  AcceptBufs bf;
  unsigned char* p = base;
  auto take4 = [&]() {
    unsigned char* q = p;
    p += kNaSlot4;
    return q;
  };
  auto take8 = [&]() {
    unsigned char* q = p;
    p += kNaSlot8;
    return q;
  };
  bf.mx = reinterpret_cast<float*>(take4());
  bf.amax = reinterpret_cast<int*>(take4());
  bf.second = reinterpret_cast<float*>(take4());
  bf.dmx = reinterpret_cast<float*>(take4());
  bf.damax = reinterpret_cast<int*>(take4());
  bf.tp_key = reinterpret_cast<unsigned*>(take4());
  bf.tp_id = reinterpret_cast<int*>(take4());
  bf.sum = reinterpret_cast<double*>(take8());
  bf.dsum = reinterpret_cast<double*>(take8());
  bf.tp_mass = reinterpret_cast<double*>(take8());
  return accept_core(nullptr, bf, vocab, kNoAllocRows, "vs_accept_noalloc", b, mode, temp, 1.0, d_tokens, d_logits,
                     d_draft_logits, d_u, d_result, S(stream));
}

vs_status vs_accept(vs_model* m, const vs_batch* b, int32_t mode, float temp, const int32_t* d_tokens,
                    const float* d_logits, const float* d_draft_logits, const double* d_u, int32_t* d_result,
                    void* stream) {
  return accept_impl(m, b, mode, temp, 1.0, d_tokens, d_logits, d_draft_logits, d_u, d_result, stream);
}

vs_status vs_accept_top_p(vs_model* m, const vs_batch* b, float temp, double top_p, const int32_t* d_tokens,
                          const float* d_logits, const float* d_draft_logits, const double* d_u, int32_t* d_result,
                          void* stream) {
  if (!(top_p > 0.0 && top_p <= 1.0)) return fail(VS_E_INVAL, "vs_accept_top_p: top_p %g outside (0, 1]", top_p);
  return accept_impl(m, b, VS_SAMPLE, temp, top_p, d_tokens, d_logits, d_draft_logits, d_u, d_result, stream);
}

vs_status vs_commit(vs_model* m, vs_kv* kv, const vs_batch* b, const int32_t* d_result, void* stream) {
  if (m == nullptr || kv == nullptr || d_result == nullptr) return fail(VS_E_INVAL, "vs_commit: null argument");
  RowMap rm;
  vs_status rc = batch_rowmap(kv, b, &rm);
  if (rc != VS_OK) return rc;
  hipStream_t st = S(stream);
  CommitArgs a;
  memset(&a, 0, sizeof(a));
  a.rows = rm;
  a.result = d_result;
  a.P = kv->P;
  a.pending = kv->pending;
  a.committed = kv->committed;
  a.bt = kv->bt;
  a.bps = kv->bps;
  a.kpool = kv->d_kptr;
  a.vpool = kv->d_vptr;
  a.n_layers = m->c.n_layers;
  a.Hkv = m->c.n_kv_heads;
  a.hd = m->c.head_dim;
  a.mirror = kv->mirror;
  for (int i = 0; i < rm.n_seq; ++i) a.commit_no[i] = kv->commit_no[rm.seq[i]] + 1;
  if (b->d_mask != nullptr) timed(m, F_SMALL, 0, st, [&](hipEvent_t, hipEvent_t) { launch_compact(a, st); });
  timed(m, F_SMALL, 0, st, [&](hipEvent_t, hipEvent_t) { launch_commit(a, st); });
  for (int i = 0; i < rm.n_seq; ++i) {  // the bound counts every row until the mirror shows the commit
    const int s = rm.seq[i], rows = rm.row_start[i + 1] - rm.row_start[i];
    kv->commit_no[s] += 1;
    kv->in_flight[s].emplace_back(kv->commit_no[s], rows);
    kv->P_ub[s] += rows;
  }
  return check_launch("vs_commit");
}

vs_status vs_step(vs_model* m, vs_kv* kv, int32_t n_seq, const int32_t* seq, const int32_t* k, int32_t mode,
                  float temp, const double* d_u, int32_t* d_tokens, int32_t* d_result, void* stream) {
  if (m == nullptr || kv == nullptr || d_tokens == nullptr || d_result == nullptr)
    return fail(VS_E_INVAL, "vs_step: null argument");
  int M = 0;
  vs_status rc = validate_chain(m, kv, n_seq, seq, k, mode, temp, d_u, &M);
  if (rc != VS_OK) return rc;
  hipStream_t st = S(stream);
  draft_impl(m, kv, n_seq, seq, k, mode, temp, d_u, d_tokens, m->hidden, m->dlogits, st);
  std::vector<int> rows(n_seq);
  for (int i = 0; i < n_seq; ++i) rows[i] = k[i] + 1;
  vs_batch b{n_seq, seq, rows.data(), nullptr, nullptr};
  const int L = m->c.exit_layer;
  if ((rc = vs_verify(m, kv, &b, L, d_tokens, m->hidden, m->logits, stream)) != VS_OK) return rc;
  if ((rc = vs_accept(m, &b, mode, temp, d_tokens, m->logits, m->dlogits, d_u, d_result, stream)) != VS_OK) return rc;
  return vs_commit(m, kv, &b, d_result, stream);
}

// Row map of a chain or tree batch for the per-row kernels (accept, stats).
static vs_status batch_rows(vs_model* m, const vs_batch* b, const char* name, RowMap* rm) {
  if (b == nullptr || b->seq == nullptr || b->n_rows == nullptr) return fail(VS_E_INVAL, "%s: null batch", name);
  if (b->n_seq < 1 || b->n_seq > kMaxSeq) return fail(VS_E_SHAPE, "%s: n_seq %d", name, b->n_seq);
  memset(rm, 0, sizeof(*rm));
  rm->n_seq = b->n_seq;
  int M = 0;
  for (int i = 0; i < b->n_seq; ++i) {
    if (b->n_rows[i] < 1 || b->n_rows[i] > kMaxRows) return fail(VS_E_SHAPE, "%s: rows %d", name, b->n_rows[i]);
    rm->seq[i] = b->seq[i];
    rm->row_start[i] = M;
    M += b->n_rows[i];
  }
  rm->row_start[b->n_seq] = M;
  rm->M = M;
  rm->mask = b->d_mask;
  rm->depth = b->d_depth;
  if (M > m->max_rows) return fail(VS_E_SHAPE, "%s: %d rows exceed max_rows", name, M);
  return VS_OK;
}

vs_status vs_confidence(vs_model* m, const vs_batch* b, float temp, const float* d_logits, double* d_conf,
                        void* stream) {
  if (m == nullptr || d_logits == nullptr || d_conf == nullptr) return fail(VS_E_INVAL, "vs_confidence: null argument");
  if (!(temp > 0.f)) return fail(VS_E_INVAL, "vs_confidence: temperature %g", (double)temp);
  RowMap rm;
  vs_status rc = batch_rows(m, b, "vs_confidence", &rm);
  if (rc != VS_OK) return rc;
  hipStream_t st = S(stream);
  StatsArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.logits = d_logits;
  sa.V = m->c.vocab;
  sa.temp = temp;
  sa.mx = m->st_mx;
  sa.amax = m->st_amax;
  sa.second = m->st_second;
  sa.sumexp = m->st_sum;
  timed(m, F_SMALL, (double)rm.M * m->c.vocab * 4, st, [&](hipEvent_t, hipEvent_t) { launch_row_stats(sa, rm.M, st); });
  ConfArgs ca;
  ca.rows = rm;
  ca.mx = m->st_mx;
  ca.second = m->st_second;
  ca.sumexp = m->st_sum;
  ca.temp = temp;
  ca.conf = d_conf;
  timed(m, F_SMALL, 0, st, [&](hipEvent_t, hipEvent_t) { launch_confidence(ca, st); });
  return check_launch("vs_confidence");
}

static vs_status check_sched(const vs_sched_cfg* c) {
  if (c == nullptr) return fail(VS_E_INVAL, "schedule: null config");
  if (c->min_k < 1 || c->max_k < c->min_k || c->max_k > VS_MAX_K)
    return fail(VS_E_INVAL, "schedule: draft lengths [%d, %d] outside [1, %d]", c->min_k, c->max_k, VS_MAX_K);
  if (!(c->low < c->high)) return fail(VS_E_INVAL, "schedule: thresholds %g >= %g", c->low, c->high);
  return VS_OK;
}

vs_status vs_sched_init(const vs_sched_cfg* c, int32_t k0, vs_spec_state* s) {
  vs_status rc = check_sched(c);
  if (rc != VS_OK) return rc;
  if (s == nullptr) return fail(VS_E_INVAL, "vs_sched_init: null state");
  s->ema = 0.5;
  s->k = std::min(c->max_k, std::max(c->min_k, k0));
  s->rounds = 0;
  s->last_a = -1;
  return VS_OK;
}

vs_status vs_sched_update(const vs_sched_cfg* c, vs_spec_state* s, int32_t a, double avg_top1, double avg_gap) {
#pragma clang fp contract(off)
  vs_status rc = check_sched(c);
  if (rc != VS_OK) return rc;
  if (s == nullptr) return fail(VS_E_INVAL, "vs_sched_update: null state");
  if (a < 0 || a > s->k) return fail(VS_E_INVAL, "vs_sched_update: %d accepted of %d drafts", a, s->k);
  if (!std::isfinite(avg_top1) || !std::isfinite(avg_gap))
    return fail(VS_E_INVAL, "vs_sched_update: confidence inputs not finite");
  const double acc = (double)a / (double)s->k;
  s->ema = 0.2 * acc + 0.8 * s->ema;
  const double C = 0.4 * avg_top1 + 0.3 * std::fmin(avg_gap * 5.0, 1.0) + 0.3 * s->ema;
  const double x = c->min_k + (c->max_k - c->min_k) * (C - c->low) / (c->high - c->low);
  int nk = x >= (double)c->max_k ? c->max_k : x <= (double)c->min_k ? c->min_k : (int)x;
  if (a == 0) nk = c->min_k;  // the first draft was rejected: back to the shortest block at once
  s->k = nk;
  s->last_a = a;
  s->rounds += 1;
  return VS_OK;
}

static vs_status check_dynk(const vs_dynk_cfg* c) {
  if (c == nullptr) return fail(VS_E_INVAL, "dynamic k: null config");
  if (c->window < 1 || c->window > VS_DYNK_MAX_WINDOW)
    return fail(VS_E_INVAL, "dynamic k: window %d outside [1, %d]", c->window, VS_DYNK_MAX_WINDOW);
  if (c->min_k < 1 || c->max_k < c->min_k || c->max_k > VS_MAX_K)
    return fail(VS_E_INVAL, "dynamic k: draft lengths [%d, %d] outside [1, %d]", c->min_k, c->max_k, VS_MAX_K);
  if (!(c->down <= c->up)) return fail(VS_E_INVAL, "dynamic k: thresholds %g > %g", c->down, c->up);
  return VS_OK;
}

vs_status vs_dynk_init(const vs_dynk_cfg* c, int32_t k0, vs_dynk_state* s) {
  vs_status rc = check_dynk(c);
  if (rc != VS_OK) return rc;
  if (s == nullptr) return fail(VS_E_INVAL, "vs_dynk_init: null state");
  memset(s, 0, sizeof(*s));
  s->k = std::min(c->max_k, std::max(c->min_k, k0));
  s->alpha = 1.0;
  return VS_OK;
}

vs_status vs_dynk_update(const vs_dynk_cfg* c, vs_dynk_state* s, int32_t a, int32_t k_used, double c_draft,
                         int32_t* k_next) {
#pragma clang fp contract(off)
  vs_status rc = check_dynk(c);
  if (rc != VS_OK) return rc;
  if (s == nullptr || k_next == nullptr) return fail(VS_E_INVAL, "vs_dynk_update: null argument");
  if (k_used < 0 || a < 0 || a > k_used)
    return fail(VS_E_INVAL, "vs_dynk_update: %d accepted of %d drafts", a, k_used);
  if (k_used > 0) {  // a speculative round: slide the window, then step k
    s->a[s->head] = a;
    s->drafted[s->head] = k_used;
    s->head = (s->head + 1) % c->window;
    s->n = std::min(s->n + 1, c->window);
    int64_t sa = 0, sk = 0;
    for (int j = 0; j < s->n; ++j) {  // the n most recent rounds, oldest first
      const int slot = (s->head - s->n + j + 2 * c->window) % c->window;
      sa += s->a[slot];
      sk += s->drafted[slot];
    }
    s->alpha = (double)sa / (double)sk;
    if (s->alpha > c->up) s->k = std::min(c->max_k, s->k + 1);
    else if (s->alpha < c->down) s->k = std::max(c->min_k, s->k - 1);
  }
  int kn = s->k;
  if (c_draft > 0.0) {
    // k maximising E(k) / (c k + 1), E(k) = (1 - alpha^(k+1)) / (1 - alpha)
    int best_k = 1;
    double best = -1.0;
    for (int k = 1; k <= c->max_k; ++k) {
      const double e = s->alpha == 1.0 ? (double)(k + 1) : (1.0 - std::pow(s->alpha, k + 1)) / (1.0 - s->alpha);
      const double sp = e / (c_draft * k + 1.0);
      if (sp > best) {
        best = sp;
        best_k = k;
      }
    }
    kn = (best <= 1.0 || best_k < c->min_k) ? 0 : std::min(kn, best_k);
  }
  *k_next = kn;
  return VS_OK;
}

vs_status vs_ngram_propose(const int32_t* tokens, int32_t n, int32_t search_len, int32_t min_ngram,
                           int32_t max_ngram, int32_t k_max, int32_t* out, int32_t* n_out) {
  if (tokens == nullptr || out == nullptr || n_out == nullptr) return fail(VS_E_INVAL, "vs_ngram_propose: null argument");
  if (n < 1 || min_ngram < 1 || max_ngram < min_ngram || k_max < 0 || k_max > VS_MAX_K)
    return fail(VS_E_INVAL, "vs_ngram_propose: n %d, n-gram [%d, %d], k_max %d", n, min_ngram, max_ngram, k_max);
  *n_out = 0;
  if (k_max == 0) return VS_OK;
  const int limit = std::min(n, std::max(0, search_len));
  for (int g = std::min(max_ngram, n - 1); g >= min_ngram; --g) {
    const int32_t* suf = tokens + n - g;
    for (int i = limit - g - 1; i >= 0; --i) {  // latest start with i + g < limit
      if (std::memcmp(tokens + i, suf, (size_t)g * sizeof(int32_t)) != 0) continue;
      const int end = std::min(i + g + k_max, limit);
      for (int j = i + g; j < end; ++j) out[(*n_out)++] = tokens[j];
      return VS_OK;
    }
  }
  return VS_OK;
}

vs_status vs_step_ngram(vs_model* m, vs_kv* kv, int32_t seq, const int32_t* h_history, int32_t n_hist,
                        int32_t search_len, int32_t min_ngram, int32_t max_ngram, int32_t k_max, int32_t* d_tokens,
                        int32_t* d_result, int32_t* h_result, int32_t* k_out, void* stream) {
  if (m == nullptr || kv == nullptr || h_history == nullptr || d_tokens == nullptr || d_result == nullptr ||
      h_result == nullptr || k_out == nullptr)
    return fail(VS_E_INVAL, "vs_step_ngram: null argument");
  int32_t rows[VS_MAX_K + 1];
  int32_t k = 0;
  vs_status rc = vs_ngram_propose(h_history, n_hist, search_len, min_ngram, max_ngram, k_max, rows + 1, &k);
  if (rc != VS_OK) return rc;
  rows[0] = h_history[n_hist - 1];
  hipStream_t st = S(stream);
  hipError_t e = hipMemcpyAsync(d_tokens, rows, (size_t)(k + 1) * sizeof(int32_t), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return fail(VS_E_DEVICE, "vs_step_ngram: %s", hipGetErrorString(e));
  const int32_t n_rows = k + 1;
  vs_batch b{1, &seq, &n_rows, nullptr, nullptr};
  if ((rc = vs_verify(m, kv, &b, 0, d_tokens, nullptr, m->logits, stream)) != VS_OK) return rc;
  if ((rc = vs_accept(m, &b, VS_GREEDY, 1.0f, d_tokens, m->logits, nullptr, nullptr, d_result, stream)) != VS_OK)
    return rc;
  if ((rc = vs_commit(m, kv, &b, d_result, stream)) != VS_OK) return rc;
  e = hipMemcpyAsync(h_result, d_result, VS_RESULT_INTS * sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(VS_E_DEVICE, "vs_step_ngram: %s", hipGetErrorString(e));
  *k_out = k;
  return VS_OK;
}

vs_status vs_step_sched(vs_model* m, vs_kv* kv, int32_t n_seq, const int32_t* seq, const vs_sched_cfg* c,
                        vs_spec_state* states, int32_t* d_tokens, int32_t* d_result, int32_t* h_result, double* h_conf,
                        void* stream) {
  if (m == nullptr || kv == nullptr || seq == nullptr || states == nullptr || h_result == nullptr)
    return fail(VS_E_INVAL, "vs_step_sched: null argument");
  vs_status rc = check_sched(c);
  if (rc != VS_OK) return rc;
  if (n_seq < 1 || n_seq > kMaxSeq) return fail(VS_E_SHAPE, "vs_step_sched: n_seq %d", n_seq);
  std::vector<int> k(n_seq), rows(n_seq);
  for (int i = 0; i < n_seq; ++i) {
    if (states[i].k < c->min_k || states[i].k > c->max_k)
      return fail(VS_E_STATE, "vs_step_sched: sequence %d has draft length %d outside the schedule", i, states[i].k);
    k[i] = states[i].k;
    rows[i] = k[i] + 1;
  }
  if ((rc = vs_step(m, kv, n_seq, seq, k.data(), VS_GREEDY, 1.0f, nullptr, d_tokens, d_result, stream)) != VS_OK)
    return rc;
  vs_batch b{n_seq, seq, rows.data(), nullptr, nullptr};
  if ((rc = vs_confidence(m, &b, 1.0f, m->logits, m->conf, stream)) != VS_OK) return rc;
  hipStream_t st = S(stream);
  std::vector<double> conf(2 * n_seq);
  hipError_t e = hipMemcpyAsync(h_result, d_result, (size_t)n_seq * VS_RESULT_INTS * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipMemcpyAsync(conf.data(), m->conf, conf.size() * 8, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(VS_E_DEVICE, "vs_step_sched: %s", hipGetErrorString(e));
  for (int i = 0; i < n_seq; ++i) {
    if ((rc = vs_sched_update(c, &states[i], h_result[i * VS_RESULT_INTS], conf[2 * i], conf[2 * i + 1])) != VS_OK)
      return rc;
    if (h_conf != nullptr) {
      h_conf[2 * i] = conf[2 * i];
      h_conf[2 * i + 1] = conf[2 * i + 1];
    }
  }
  return VS_OK;
}

vs_status vs_read_probe(const void* d_src, size_t bytes, uint32_t* d_sink, void* stream) {
  if (d_src == nullptr || d_sink == nullptr) return fail(VS_E_INVAL, "vs_read_probe: null argument");
  if (bytes < 16 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(d_src) & 15) != 0)
    return fail(VS_E_INVAL, "vs_read_probe: %zu bytes (a positive multiple of 16, 16-byte aligned)", bytes);
  launch_read_probe(static_cast<const u32x4*>(d_src), bytes / 16, d_sink, S(stream));
  return check_launch("vs_read_probe");
}

vs_status vs_stats_enable(vs_model* m, int32_t on) {
  if (m == nullptr) return fail(VS_E_INVAL, "vs_stats_enable: null model");
  m->stats_mask = on;
  m->prev_end = nullptr;
  return VS_OK;
}

vs_status vs_stats_reset(vs_model* m) {
  if (m == nullptr) return fail(VS_E_INVAL, "vs_stats_reset: null model");
  for (const Timed& t : m->timed) {
    const hipError_t e = hipEventSynchronize(t.b);
    if (e != hipSuccess) return fail(VS_E_DEVICE, "vs_stats_reset: %s", hipGetErrorString(e));
  }
  m->timed.clear();
  m->ev_used = 0;
  m->prev_end = nullptr;
  for (int f = 0; f < F_COUNT; ++f) m->acc_ms[f] = m->acc_bytes[f] = 0, m->acc_n[f] = 0;
  return VS_OK;
}

vs_status vs_stats_read(vs_model* m, vs_kernel_stat* out, int32_t max, int32_t* n_out) {
  if (m == nullptr || out == nullptr || n_out == nullptr) return fail(VS_E_INVAL, "vs_stats_read: null argument");
  for (const Timed& t : m->timed) {
    if (hipEventSynchronize(t.b) != hipSuccess) return fail(VS_E_DEVICE, "vs_stats_read: event sync failed");
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, t.prev, t.b);
    float own = 0.f;
    if (t.a != nullptr && hipEventElapsedTime(&own, t.a, t.b) == hipSuccess) ms = std::min(ms, own);
    m->acc_ms[t.fam] += ms;
    m->acc_bytes[t.fam] += t.bytes;
    m->acc_n[t.fam] += 1;
  }
  m->timed.clear();
  m->ev_used = 0;
  m->prev_end = nullptr;
  int n = 0;
  for (int f = 0; f < F_COUNT && n < max; ++f) {
    memset(&out[n], 0, sizeof(out[n]));
    snprintf(out[n].name, sizeof(out[n].name), "%s", kFamilyNames[f]);
    out[n].launches = m->acc_n[f];
    out[n].total_ms = m->acc_ms[f];
    out[n].bytes = m->acc_bytes[f];
    ++n;
  }
  *n_out = n;
  return VS_OK;
}

}  // extern "C"
