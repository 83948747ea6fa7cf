// Argument structs and launchers of the round's small kernels (internal).
#pragma once
#include "common.h"

namespace vs {

enum PackMap { PACK_IDENTITY = 0, PACK_HEADS = 1, PACK_EVEN = 2, PACK_ODD = 3 };

struct PackArgs {
  const uint16_t* src;  // canonical [rows][K]
  uint16_t* dst;        // packed matrix
  int rows, K, k_steps, row_off, map, hd;
  int wide32;           // fragments of 32 columns x 16 inputs (gemm_wide32)
};

struct BlockSetArgs {
  int* bt;
  int bps, seq, first, n, reset_state;
  int* P;
  int* pending;
  int* committed;
  int ids[256];
};

struct LoadArgs {
  int M, d, V;
  const int* tokens;      // token ids (embedding) or null
  const uint16_t* embed;  // [V][d] bf16
  const float* hidden;    // hidden rows when tokens == null
  int src_identity;
  int src_row[kMaxRows];
  float* h;
  uint16_t* xa;
  const float* g;
  float* ss;              // [ceil(d/256)][M]
  // RoPE table of the pass rows: rope[m][i] = (cos, sin) of pos_m * theta^(-2i/hd)
  float2* rope;           // null: not needed
  const int* P;           // sequence KV lengths
  RowMap rows;
  int half;
  float theta;
  // KV destination of each row (block * 16 + slot % 16), the same in every
  // layer's pool; written with the RoPE table
  const int* bt;
  int bps;
  int* kvrow;
};

struct StatsArgs {
  const float* logits;
  int V;
  float temp;
  float* mx;
  int* amax;
  float* second;
  double* sumexp;         // null: skip
};

// Draft-token selection for one draft step: sequence i writes
// tokens[dst[i]] = pending (src == -1), the argmax of row src[i] of the head
// partials (greedy) or a draw from softmax(logits row / T) with
// u[i * 48 + slot] (sample).
struct PickArgs {
  int n;
  int mode;
  float temp;
  int slot;
  const int* pending;
  const float* amax_val;
  const int* amax_idx;
  int groups, Mprev;
  const float* logits;    // sample: rows of the previous head pass
  int V;
  const double* u;
  int* tokens;
  int seq[kMaxSeq];
  int src[kMaxSeq];       // previous-pass row, or -1 for the pending token
  int lrow[kMaxSeq];      // logits row (sample)
  int uidx[kMaxSeq];      // index of the sequence in the uniforms array
  int dst[kMaxSeq];
};

struct AcceptArgs {
  RowMap rows;            // rows of the verify pass (masks define parents)
  int mode;
  float temp;
  const int* tokens;
  const float* logits;    // target logits [M][V]
  const float* dlogits;   // draft logits [M][V] (sample)
  const float* mx;        // target row stats
  const int* amax;
  const float* second;
  const double* sumexp;
  const float* dmx;       // draft row stats
  const double* dsumexp;
  int V;
  const double* u;        // [n_seq][48]
  int* result;            // [n_seq][24]
  // top-p truncation of the target (null: none): token j of row r is kept
  // iff key(z_j) > tp_key[r], or key(z_j) == tp_key[r] and j <= tp_id[r];
  // tp_mass[r] = sum over the kept tokens of exp((z_j - max) / temp)
  const unsigned* tp_key;
  const int* tp_id;
  const double* tp_mass;
};

// Top-p boundary of each row (see top_p_kernel).
struct TopPArgs {
  const float* logits;
  int V;
  float temp;
  double top_p;
  const float* mx;        // row maxima
  unsigned* key;
  int* id;
  double* mass;
};

struct CommitArgs {
  RowMap rows;
  const int* result;
  int* P;
  int* pending;
  int* committed;
  const int* bt;
  int bps;
  uint16_t** kpool;       // [n_layers] device array of layer K pools
  uint16_t** vpool;
  int n_layers, Hkv, hd;
  // host-visible record of each committed sequence's new KV length:
  // mirror[seq] = (commit number << 32) | P, one 64-bit store (optional)
  uint64_t* mirror;
  unsigned commit_no[kMaxSeq];
};

// Target-model confidence of each sequence's verify rows: the mean over its
// rows of p_top1 and of p_top1 - p_top2 under softmax(z / temp), from the
// row statistics (max, second largest value, sum of exp((z - max) / temp)).
struct ConfArgs {
  RowMap rows;
  const float* mx;
  const float* second;
  const double* sumexp;
  float temp;
  double* conf;           // [n_seq][2]
};

// Tree drafting state (one sequence).  Nodes are numbered in creation order
// (root = 0); the verify rows are the root and the kept nodes in level order.
constexpr int kTreeNodes = 1024;
constexpr int kTreeMaxDepth = 8;
constexpr int kTreeMaxTopk = 8;
struct TreeArgs {
  int* tok;               // node arrays [kTreeNodes]
  int* parent;
  int* depth;
  int* rank;
  double* score;          // product of the draft probabilities along the path
  int* meta;              // [0] nodes, [1] frontier rows, [2] first frontier row, [3] real rows
  int* row_tok;           // pass rows [R]
  int* row_depth;
  uint64_t* row_mask;
  int* row_node;
  int* row_parent;
  int R;                  // rows of every pass (1 + keep)
  int level;              // select: rows for expanding this depth (== max_depth: final layout)
  int max_depth, topk, keep;
  const int* pending;     // root token = pending[seq]
  int seq;
  // expand
  const float* logits;    // head output of the pass [R][V]
  int V;
  float temp;
  // final layout copies (optional)
  int* out_tok;
  int* out_depth;
  uint64_t* out_mask;
  int* out_parent;
};

void launch_tree_select(const TreeArgs& a, hipStream_t st);
void launch_tree_expand(const TreeArgs& a, hipStream_t st);

void launch_pack(const PackArgs& a, hipStream_t st);
void launch_bf16_to_f32(const uint16_t* src, float* dst, int n, hipStream_t st);
void launch_fill_i32(int* p, int v, size_t n, hipStream_t st);
// Streaming read of n16 16-byte units by kReadProbeBlocks workgroups, each a
// contiguous range; one checksum word per workgroup into sink.
constexpr int kReadProbeBlocks = 2048;
void launch_read_probe(const u32x4* src, size_t n16, uint32_t* sink, hipStream_t st);
void launch_set_blocks(const BlockSetArgs& a, hipStream_t st);
void launch_set_state(int* P, int* pending, int* committed, int seq, int p, int pend, hipStream_t st);
void launch_load_rows(const LoadArgs& a, hipStream_t st);
void launch_copy_rows(const float* src, float* dst, int M, int d, hipStream_t st);
void launch_row_stats(const StatsArgs& a, int M, hipStream_t st);
// the rows of a, then the same rows of b, in one launch
void launch_row_stats2(const StatsArgs& a, const StatsArgs& b, int M, hipStream_t st);
void launch_pick(const PickArgs& a, hipStream_t st);
void launch_accept(const AcceptArgs& a, hipStream_t st);
void launch_compact(const CommitArgs& a, hipStream_t st);
void launch_commit(const CommitArgs& a, hipStream_t st);
void launch_advance(int* P, int* committed, int seq, int dP, int dC, hipStream_t st);
void launch_confidence(const ConfArgs& a, hipStream_t st);
void launch_top_p(const TopPArgs& a, int M, hipStream_t st);

}  // namespace vs
