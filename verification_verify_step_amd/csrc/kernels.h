// Launch interfaces of the library's kernels (internal).
#pragma once
#include <hip/hip_ext.h>

#include "common.h"

namespace vs {

enum Epi { EPI_RESID = 0, EPI_QKV = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

// Y[M][N] = X[M][K] . W[N][K]^T over packed bf16 weights and split-bf16
// activations, then one of four fused epilogues.
struct GemmArgs {
  const uint16_t* W;     // packed fragments [n_tiles][k_steps][64 lanes][8]
  int n_tiles, k_steps;
  const uint16_t* xa;    // activation fragments, see xa_index()
  int M;                 // rows computed by this launch: pass rows m0 .. m0+M-1
  int m0, ld;            // first row; rows of the whole pass (row stride of every row-indexed array)
  // RMSNorm scale of the input rows: rs[m] = 1/sqrt(sum_g ss[g*M+m] / d + eps)
  const float* ss;       // null: no norm scale
  int ss_groups;
  float inv_d, eps;
  // EPI_RESID: h += Y; next consumer's activation (h * g_next) -> xa_next,
  // per-group sum of squares -> ss_out[blockIdx][M]; optional copy of the
  // new h rows to h_copy[out_row[m]].
  float* h;
  int d;
  uint16_t* xa_next;
  const float* g_next;
  float* ss_out;
  float* h_copy;
  // EPI_QKV
  RowMap rows;
  KvView kv;
  float* q;
  int H, Hkv, hd;
  const float2* rope;    // [M][hd/2] (cos, sin) of each row's position
  const int* kvrow;      // [M] KV destination: block * 16 + slot % 16

  // EPI_SWIGLU
  uint16_t* xa_act;
  // EPI_LOGITS: logits[out_row[m]][V] (out_row relative to m0); per-group argmax partials
  float* logits;
  int V;
  float* amax_val;
  int* amax_idx;
  int out_row_identity;
  int out_row[kMaxRows];
  int cfg;               // launch configuration (0: chosen from the shape), see gemm_cfg()
  // Row-tiled form: per-row norm scales, computed into rs_buf[m0 .. m0+M)
  // (a workspace of the pass's rows) before the product when ss is set.
  float* rs_buf;
  const float* rs;
  // Row-tiled form with K split: chunk sums [cell][chunk][wave][...] and one
  // arrival counter per (n-range, row block) cell, zero between launches.
  float* kpart;
  unsigned* kcnt;
};

// Launch configurations: n-tiles per workgroup (NTW) x waves per workgroup
// (NW, splitting K).  Returns the number of workgroups launched (= the ss
// groups an EPI_RESID launch writes).
struct GemmCfg {
  int ntw, nw;
};
constexpr int kGemmCfgs = 5;
GemmCfg gemm_cfg(int id);
int gemm_pick(int n_tiles, int k_steps, int M);
// ev0/ev1 (optional): events timestamped at the kernel's own start and end.
// Passes of more than 8 rows go to the row-tiled form (cfg 0 or
// kGemmCfgTile) when its K chunks fit (gemm_tile_fits): the wide matrices
// (>= 512 n-tiles) at any row count, the narrow ones with long K chunks at
// up to 64 rows with K split over workgroups; cfg 1..4 force the skinny
// form.
int launch_gemm(const GemmArgs& a, int epi, hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
constexpr int kGemmCfgTile = 8;  // row-tiled form, n-tiles per wave chosen from the shape (+1, +2, +4: forced)
bool gemm_uses_tile(int n_tiles, int k_steps, int M, int cfg);

// Row-tiled form: row blocks of 16*mw rows (n_mblk of them), 4*ntw n-tiles
// per workgroup.  Returns the number of 16-column groups (= n_tiles).
struct TileShape {
  int mw, ntw, n_mblk;
  bool split;  // K split over workgroups (gemm_tile_split)
};
TileShape gemm_tile_shape(int n_tiles, int M, int ntw);
int launch_gemm_tile(const GemmArgs& a, int epi, int ntw, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
// The row-tiled form's per-row norm scales (a.ss -> a.rs_buf), launched
// before the product; `start` (optional) is stamped at its start.
void launch_row_scale(const GemmArgs& a, hipStream_t st, hipEvent_t start);
// The wide matrices (gemm_wide32): 32x32x16 MFMA forms, skinny (up to 8 rows)
// and row-tiled (tiles of 32 columns, ntw of them per wave).  Both return the
// number of 16-column groups (= n_tiles).
int launch_gemm32(const GemmArgs& a, int epi, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
TileShape gemm_tile32_shape(int n_tiles, int M, int ntw);
int launch_gemm_tile32(const GemmArgs& a, int epi, int ntw, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

struct AttnArgs {
  RowMap rows;
  KvView kv;
  const float* q;   // [M][H][hd]
  int H, Hkv, hd;
  float scale;
  int qg_size;      // query vectors per query group (<= 16)
  int n_qg;         // query groups per (sequence, KV head) at the pass's longest sequence
  // Split structure.  Keys are cut at fixed absolute indices, and every
  // count a kernel acts on follows from the sequence's own KV length P (read
  // on the device), so a row's result depends neither on the other
  // sequences of the pass nor on the host's bound of P.
  //  * one-group kernel: committed splits of one 32-key step, the in-round
  //    window as one more split, chunks of WV consecutive splits (one per
  //    wave); a workgroup runs cpw consecutive chunks of its unit;
  //  * grouped kernel: committed splits of kps keys (a multiple of 32), the
  //    last one also taking the in-round window.
  int kps;
  int cpw;
  int lp;           // one-group kernel: every unit one workgroup's, chunk partials kept in LDS
  // Workgroups of sequence i: [wg_start[i], wg_start[i+1]), laid out from
  // the host's upper bound of P; workgroups the device's P does not need
  // exit at once.  nsplit[i]: the bound's split (grouped) or chunk
  // (one-group) count of sequence i.
  int wg_start[kMaxSeq + 1];
  int nsplit[kMaxSeq];
  // One-group kernel: the block-table row of the first step of sequence i's
  // in-round window at the host's lower bound of P, so that the window's
  // table entries are requested with P itself (a device P outside the 64
  // entries read from there takes two scalar loads instead).
  int wblk[kMaxSeq];
  int n_split;      // largest nsplit: the partials' records per unit
  // Partials of a unit (sequence, KV head, query group), record j (split or
  // chunk): o at part[((unit * n_split + j) * qg_size + v) * hd + dim],
  // (max, sum) as a float pair at part[ml_off + 2 * ((unit * n_split + j) *
  // qg_size + v)].
  float* part;
  size_t ml_off;    // floats; even
  unsigned* cnt;    // per-unit arrival counters, zero between launches
  uint16_t* xa_o;
  int M;
};
constexpr int kGemmSplitCells = 4096;    // K-split arrival counters
constexpr size_t kGemmSplitFloats = size_t(8) * 8192 * 64;  // K-split chunk sums: 8 chunks x 8192 columns x 64 rows
// One launch: splits, in-workgroup merge per chunk, and the last
// workgroup's combine over the chunks of its unit.
void launch_attention(const AttnArgs& a, hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
constexpr int kAttnQG = 16;              // query vectors per query group
constexpr int kAttnWaves = 4;            // one-group kernel: waves (splits) per chunk
constexpr int kAttnMaxCpw = 32;          // one-group kernel: chunks per workgroup at most
constexpr int kAttnLpRecords = 96;       // one-group kernel: chunk partials one workgroup keeps in LDS
constexpr int kAttnMaxUnits = 16384;     // arrival counters
hipError_t attn_init();

}  // namespace vs
