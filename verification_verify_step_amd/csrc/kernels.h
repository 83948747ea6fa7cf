// Launch interfaces of the library's kernels (internal).
#pragma once
#include "common.h"

namespace vs {

enum Epi { EPI_RESID = 0, EPI_QKV = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

// Y[M][N] = X[M][K] . W[N][K]^T over packed bf16 weights and split-bf16
// activations, then one of four fused epilogues.
struct GemmArgs {
  const uint16_t* W;     // packed fragments [n_tiles][k_steps][64 lanes][8]
  int n_tiles, k_steps;
  const uint16_t* xa;    // activation fragments, see xa_index()
  int M;
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
  float theta;
  // EPI_SWIGLU
  uint16_t* xa_act;
  // EPI_LOGITS: logits[out_row[m]][V]; per-group argmax partials
  float* logits;
  int V;
  float* amax_val;
  int* amax_idx;
  int out_row_identity;
  int out_row[kMaxRows];
};

// Returns the number of workgroups launched (= ss groups for EPI_RESID).
int launch_gemm(const GemmArgs& a, int epi, hipStream_t st);
int gemm_groups(int n_tiles);

struct AttnArgs {
  RowMap rows;
  KvView kv;
  const float* q;   // [M][H][hd]
  int H, Hkv, hd;
  float scale;
  int n_split;      // committed-key splits; split n_split is the in-round window
  int kps;          // keys per committed split (multiple of kChunk)
  int qg_size;      // query vectors per workgroup
  int n_qg;
  float* part;      // partials: per (i, kvh, qg, split): qg_size x (hd + 2) floats
  int* counters;    // per (i, kvh, qg)
  uint16_t* xa_o;
  int M;
};
void launch_attention(const AttnArgs& a, hipStream_t st);
hipError_t attn_init();  // lets the attention kernel use more than 64 KB of LDS

}  // namespace vs
