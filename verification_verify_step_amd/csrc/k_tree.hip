// Tree drafting on the device ("FlashSpec" page, lnrk.cn/news/47842): the
// candidate tokens form a tree that one forward pass verifies, laid out in
// level order with each node seeing its ancestors (§2.2), positions by
// depth (§3.2).  Shape as read for the 63-node tree: every expanded node
// gets its top-k children by draft probability, a path's score is the
// product of the draft probabilities along it, and the kept set is the
// global top `keep` non-root nodes by (score, then shallower, then earlier
// created).  It is built level by level, expanding at depth d only the kept
// nodes of depth d; a child never scores above its parent, so this equals
// the selection over the full expansion.
//
// Each level pass recomputes the first layers over the root and every kept
// node (at most 1 + keep rows, weight-bound like a pass over the frontier
// alone), so every mask fits in 64 bits and no host round trip is needed:
// tree_select_kernel lays out the rows, the pass runs, the head scores them,
// tree_expand_kernel appends the frontier's children.
#include "misc.h"

namespace vs {

constexpr int kSelThreads = 1024;
constexpr int kExpThreads = 256;

// kept order: higher score first, then shallower, then created earlier
__device__ __forceinline__ bool kept_before(double sa, int da, int ia, double sb, int db, int ib) {
  if (sa != sb) return sa > sb;
  if (da != db) return da < db;
  return ia < ib;
}

__global__ __launch_bounds__(kSelThreads) void tree_select_kernel(TreeArgs a) {
  __shared__ double s_score[kTreeNodes];
  __shared__ int s_depth[kTreeNodes], s_parent[kTreeNodes], s_rank[kTreeNodes], s_tok[kTreeNodes];
  __shared__ int s_row[kTreeNodes];      // row of a kept node, -1 otherwise
  __shared__ unsigned char s_kept[kTreeNodes];
  __shared__ int s_node_of_row[kMaxRows];
  __shared__ uint64_t s_mask[kMaxRows];
  __shared__ int s_count[kTreeMaxDepth + 2], s_base[kTreeMaxDepth + 2];
  __shared__ int s_n;
  const int t = threadIdx.x;
  if (t == 0) {
    // nodes appended by the previous level's expansion
    const int n = a.level == 0 ? 1 : min(kTreeNodes, a.meta[0] + a.topk * a.meta[1]);
    s_n = n;
  }
  if (t < kTreeMaxDepth + 2) s_count[t] = 0;
  __syncthreads();
  const int n = s_n;
  for (int i = t; i < n; i += kSelThreads) {
    if (i == 0 && a.level == 0) {
      s_tok[0] = a.pending[a.seq];
      s_parent[0] = -1;
      s_depth[0] = 0;
      s_rank[0] = 0;
      s_score[0] = 1.0;
    } else {
      s_tok[i] = a.tok[i];
      s_parent[i] = a.parent[i];
      s_depth[i] = a.depth[i];
      s_rank[i] = a.rank[i];
      s_score[i] = a.score[i];
    }
    s_row[i] = -1;
  }
  __syncthreads();
  // kept set: the root and the top `keep` other nodes
  for (int i = t; i < n; i += kSelThreads) {
    int kept = i == 0;
    if (i > 0) {
      int r = 0;
      for (int j = 1; j < n && r < a.keep; ++j)
        r += kept_before(s_score[j], s_depth[j], j, s_score[i], s_depth[i], i);
      kept = r < a.keep;
    }
    s_kept[i] = (unsigned char)kept;
    if (kept && i > 0) atomicAdd(&s_count[s_depth[i]], 1);
  }
  __syncthreads();
  if (t == 0) {
    s_base[0] = 0;
    s_base[1] = 1;
    for (int d = 1; d <= kTreeMaxDepth; ++d) s_base[d + 1] = s_base[d] + s_count[d];
    s_row[0] = 0;
    s_node_of_row[0] = 0;
    s_mask[0] = 1ull;
  }
  // level order: depth, then the parent's row, then child rank
  for (int d = 1; d <= a.max_depth; ++d) {
    __syncthreads();
    for (int i = t; i < n; i += kSelThreads) {
      if (!s_kept[i] || i == 0 || s_depth[i] != d) continue;
      const int pr = s_row[s_parent[i]];
      if (pr < 0) continue;  // cannot happen: the kept set holds every kept node's parent
      int pos = 0;
      for (int j = 1; j < n; ++j) {
        if (!s_kept[j] || s_depth[j] != d) continue;
        const int pj = s_row[s_parent[j]];
        pos += (pj < pr) || (pj == pr && s_rank[j] < s_rank[i]);
      }
      const int row = s_base[d] + pos;
      if (row >= kMaxRows) continue;
      s_row[i] = row;
      s_node_of_row[row] = i;
      s_mask[row] = s_mask[pr] | (1ull << row);
    }
  }
  __syncthreads();
  const int real = min(s_base[a.max_depth + 1], a.R);  // 1 + kept nodes
  for (int r = t; r < a.R; r += kSelThreads) {
    int tok, dep, par, node;
    uint64_t mk;
    if (r < real) {
      node = s_node_of_row[r];
      tok = s_tok[node];
      dep = s_depth[node];
      par = node == 0 ? -1 : s_row[s_parent[node]];
      mk = s_mask[r];
    } else {  // padding: sees only itself and is seen by no real row
      node = -1;
      tok = s_tok[0];
      dep = 0;
      par = -1;
      mk = 1ull << r;
    }
    a.row_tok[r] = tok;
    a.row_depth[r] = dep;
    a.row_mask[r] = mk;
    a.row_node[r] = node;
    a.row_parent[r] = par;
    if (a.out_tok != nullptr) {
      a.out_tok[r] = tok;
      a.out_depth[r] = dep;
      a.out_mask[r] = mk;
      a.out_parent[r] = par;
    }
  }
  if (t == 0) {
    // frontier: the kept rows of depth `level` (the root at level 0); the
    // final layout expands nothing
    int n_front = 0, first = 0;
    if (a.level < a.max_depth) {
      n_front = a.level == 0 ? 1 : s_count[a.level];
      first = a.level == 0 ? 0 : s_base[a.level];
    }
    a.meta[0] = n;
    a.meta[1] = n_front;
    a.meta[2] = first;
    a.meta[3] = real;
  }
  if (t == 0 && n == 1) {  // the root lives in the node arrays from here on
    a.tok[0] = s_tok[0];
    a.parent[0] = -1;
    a.depth[0] = 0;
    a.rank[0] = 0;
    a.score[0] = 1.0;
  }
}

// Block reductions over kExpThreads threads in a fixed order.
__device__ double block_sum_f64(double v, double* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int o = kExpThreads / 2; o > 0; o >>= 1) {
    if (t < o) sh[t] += sh[t + o];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

// (value, id) maximum with ties to the lower id
__device__ void block_argmax(float& v, int& id, float* sv, int* si) {
  const int t = threadIdx.x;
  sv[t] = v;
  si[t] = id;
  __syncthreads();
  for (int o = kExpThreads / 2; o > 0; o >>= 1) {
    if (t < o) {
      const float v2 = sv[t + o];
      const int i2 = si[t + o];
      if (v2 > sv[t] || (v2 == sv[t] && i2 < si[t])) {
        sv[t] = v2;
        si[t] = i2;
      }
    }
    __syncthreads();
  }
  v = sv[0];
  id = si[0];
  __syncthreads();
}

// One workgroup per pass row; frontier rows append their top-k children.
__global__ __launch_bounds__(kExpThreads) void tree_expand_kernel(TreeArgs a) {
  __shared__ double sh_d[kExpThreads];
  __shared__ float sh_v[kExpThreads];
  __shared__ int sh_i[kExpThreads];
  const int r = blockIdx.x;
  const int n_front = a.meta[1], first = a.meta[2], n_base = a.meta[0];
  const int f = r - first;
  if (f < 0 || f >= n_front) return;  // whole workgroup
  const int node = a.row_node[r];
  if (node < 0) return;
  const float* z = a.logits + (size_t)r * a.V;
  const double T = (double)a.temp;
  // top-k ids by logit (= by softmax probability), ties to the lower id
  int ids[kTreeMaxTopk];
#pragma unroll
  for (int c = 0; c < kTreeMaxTopk; ++c) ids[c] = -1;
  float zmax = -INFINITY;
#pragma unroll
  for (int c = 0; c < kTreeMaxTopk; ++c) {
    if (c < a.topk) {  // uniform over the workgroup
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int v = threadIdx.x; v < a.V; v += kExpThreads) {
        bool taken = false;
#pragma unroll
        for (int e = 0; e < kTreeMaxTopk; ++e) taken |= e < c && ids[e] == v;
        const float x = z[v];
        if (!taken && (x > bv || (x == bv && v < bi))) {
          bv = x;
          bi = v;
        }
      }
      block_argmax(bv, bi, sh_v, sh_i);
      ids[c] = min(bi, a.V - 1);  // no candidate (non-finite logits) leaves bi at INT_MAX: keep it an index
      if (c == 0) zmax = bv;
    }
  }
  // softmax(z / T) in fp64: x = z / T, m = max x, S = sum exp(x - m)
  const double m = (double)zmax / T;
  double part = 0.0;
  for (int v = threadIdx.x; v < a.V; v += kExpThreads) part += exp((double)z[v] / T - m);
  const double S = block_sum_f64(part, sh_d);
  if (threadIdx.x < a.topk) {
    const int c = threadIdx.x;
    int id = 0;
#pragma unroll
    for (int e = 0; e < kTreeMaxTopk; ++e)
      if (e == c) id = ids[e];
    const double q = exp((double)z[id] / T - m) / S;
    const int idx = n_base + a.topk * f + c;
    if (idx < kTreeNodes) {
      a.tok[idx] = id;
      a.parent[idx] = node;
      a.depth[idx] = a.row_depth[r] + 1;
      a.rank[idx] = c;
      a.score[idx] = a.score[node] * q;
    }
  }
}

void launch_tree_select(const TreeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(tree_select_kernel, dim3(1), dim3(kSelThreads), 0, st, a);
}

void launch_tree_expand(const TreeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(tree_expand_kernel, dim3(a.R), dim3(kExpThreads), 0, st, a);
}

}  // namespace vs
