/*
 * vstep.h: C ABI of the speculative-decoding verify-step library (gfx950).
 *
 * The library runs one self-speculative decoding round on one GPU:
 *   draft   first L layers + final norm + LM head, k serial steps, writing
 *           the first-L KV that verify reuses;
 *   verify  layers L..N-1 over k+1 chain rows or the rows of a draft tree,
 *           with a per-row ancestor mask, then the head;
 *   accept  greedy longest matching prefix / path, or stochastic
 *           min(1, p/q) with residual resampling from normalize(max(0, p-q));
 *   commit  roll the KV state back to the accepted prefix (or compact the
 *           accepted tree path).
 * Sources: self-speculative decoding page (m.lqnn.cn/news/278124) §2.1
 * (layer-skip draft, KV reuse, k+1 positions), §2.4 (acceptance rule), §3.3
 * (shared cache, rollback), §4.1-§4.3 (forward_layers interface, draft,
 * verify, accept_or_reject); "DSpark" page (0539edu.com/news/4524681) §2.1
 * (greedy block verification); "FlashSpec" page (lnrk.cn/news/47842) §2.2
 * and §3.2 (tree batch in level order, parent mask, per-node positions).
 *
 * Conventions
 * - Every device buffer is allocated by the caller and passed as a raw
 *   pointer; the library never allocates device memory and never
 *   synchronises, except where a call says so.  `stream` is a hipStream_t.
 * - Token ids int32; uniforms fp64 in [0,1); logits and hidden states fp32,
 *   row-major; weights and the KV cache bf16.
 * - Sequence state lives on the device: P (KV length = position of the
 *   pending token), the pending token (last committed token, no KV yet) and
 *   the committed count.  Invariant after every commit: P == committed - 1.
 * - Rows of one pass are grouped by sequence.  Row r of sequence s has an
 *   in-round index idx (0 = first row of s in the pass), writes its KV at
 *   slot P_s + idx, sits at position P_s + depth, and attends to all slots
 *   < P_s plus the in-round slots P_s + j whose bit j is set in its mask.
 *   A NULL depth/mask array means a chain: depth = idx, mask = bits 0..idx.
 * - Errors: every call validates its arguments on the host before anything
 *   is enqueued and returns a negative vs_status without touching device
 *   state; vs_last_error() describes the last failure of the calling thread.
 *   Faults of earlier asynchronous work surface as VS_E_DEVICE.
 */
#ifndef VSTEP_H
#define VSTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vs_status;
#define VS_OK 0
#define VS_E_INVAL (-1)  /* bad argument (NULL pointer, out-of-range id, bad mode) */
#define VS_E_SHAPE (-2)  /* shape not supported (alignment, row counts, head sizes) */
#define VS_E_NOKV (-3)   /* KV pool or sequence capacity exhausted */
#define VS_E_STATE (-4)  /* call order violated (sequence not open, no prefill) */
#define VS_E_DEVICE (-5) /* a HIP runtime call failed */

#define VS_GREEDY 0
#define VS_SAMPLE 1

#define VS_MAX_ROWS 64     /* rows per sequence per pass (uint64 masks) */
#define VS_MAX_PASS_ROWS 1088  /* rows per pass over all sequences (64 sequences x 17) */
#define VS_MAX_SEQS 64     /* sequences per pass */
#define VS_MAX_K 16        /* chain draft length */
#define VS_N_UNIFORMS 48   /* per sequence per round: 0..k-1 draft, 16.. accept, 32 residual/bonus */
#define VS_RESULT_INTS 24  /* per sequence: a, y, flags, n_path, path[20] */

/* Weight tensors, canonical bf16 row-major layout:
 *  EMBED [V][d]; ATTN_NORM [d]; WQ [H*hd][d]; WK [Hkv*hd][d]; WV [Hkv*hd][d];
 *  WO [d][H*hd]; FFN_NORM [d]; W_GATE [F][d]; W_UP [F][d]; W_DOWN [d][F];
 *  FINAL_NORM [d]; HEAD [V][d]. */
enum vs_tensor {
  VS_T_EMBED = 0, VS_T_ATTN_NORM, VS_T_WQ, VS_T_WK, VS_T_WV, VS_T_WO, VS_T_FFN_NORM,
  VS_T_W_GATE, VS_T_W_UP, VS_T_W_DOWN, VS_T_FINAL_NORM, VS_T_HEAD, VS_T_COUNT
};

/* Llama-style pre-norm decoder: RMSNorm(eps), rotate-half RoPE(theta) on q
 * and k, softmax attention scaled by 1/sqrt(head_dim) with grouped KV heads,
 * SwiGLU FFN, untied embedding and head.  exit_layer = L, the draft depth. */
typedef struct vs_model_cfg {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab, exit_layer;
  float rms_eps, rope_theta;
} vs_model_cfg;

typedef struct vs_model vs_model;
typedef struct vs_kv vs_kv;

/* One pass's rows: n_seq sequences (ids seq[i], host), n_rows[i] rows each
 * (host, 1..64), optional device arrays depth[M] / mask[M] (M = sum n_rows). */
typedef struct vs_batch {
  int32_t n_seq;
  const int32_t* seq;
  const int32_t* n_rows;
  const int32_t* d_depth;
  const uint64_t* d_mask;
} vs_batch;

const char* vs_last_error(void);

/* ---- sizing (host only, no GPU needed) ---- */
/* Bytes of the packed weight buffer. 0 if the shape is unsupported. */
size_t vs_weight_bytes(const vs_model_cfg* cfg);
/* Bytes of the model workspace for passes of up to max_rows rows in total,
 * max_seqs sequences and contexts up to max_ctx tokens. */
size_t vs_workspace_bytes(const vs_model_cfg* cfg, int32_t max_rows, int32_t max_seqs, int32_t max_ctx);
/* Bytes of a KV pool of n_blocks blocks of 16 tokens (all layers, K and V)
 * plus the per-sequence state for max_seqs sequences of up to
 * max_blocks_per_seq blocks. */
size_t vs_kv_bytes(const vs_model_cfg* cfg, int32_t n_blocks, int32_t max_seqs, int32_t max_blocks_per_seq);

/* ---- model ---- */
/* Create a model over caller-owned device buffers: d_weights
 * (vs_weight_bytes) receives packed weights through vs_model_set_tensor;
 * d_workspace (vs_workspace_bytes with the same limits) holds activations.
 * Zeroes the workspace counters on `stream`. */
vs_status vs_model_create(const vs_model_cfg* cfg, void* d_weights, void* d_workspace, int32_t max_rows,
                          int32_t max_seqs, int32_t max_ctx, void* stream, vs_model** out);
/* Pack one canonical bf16 tensor (device pointer, read during the call's
 * kernels only) into the weight buffer.  layer is ignored for EMBED,
 * FINAL_NORM and HEAD. */
vs_status vs_model_set_tensor(vs_model* m, int32_t tensor, int32_t layer, const void* d_src, void* stream);
void vs_model_destroy(vs_model* m);
/* Split length of the grouped attention kernel, the one that takes passes
 * whose KV heads carry more than one query group (GQA models, or more than
 * 16 rows of a sequence).  A sequence's committed keys are cut into splits
 * of `keys` keys at fixed absolute positions ("FlashSpec" page, §2.2: every
 * row attends to all committed keys and its in-round ancestors), so a row's
 * result does not depend on the other sequences of its pass; the setting
 * changes rounding only.  keys: a multiple of 32 in [32, 928]; the default
 * cuts about 4 MiB of K/V (all KV heads of a sequence) per split.  A context
 * may span at most 64 splits.  Errors: VS_E_INVAL (null model, bad keys).
 * vs_model_attn_split returns the current setting (0 for a null model). */
vs_status vs_model_set_attn_split(vs_model* m, int32_t keys);
int32_t vs_model_attn_split(const vs_model* m);

/* ---- KV cache ---- */
/* A paged KV pool of n_blocks blocks of 16 token slots over the caller's
 * buffer d_kv (vs_kv_bytes bytes; layouts of vs_kv_layer), shared by the
 * draft and the verify of every sequence (self-speculative decoding page,
 * §2.3 and §3.3: one cache, one slot per position, the draft's first-L
 * entries read back by the verify).  The pool must hold finite values when
 * it is created (zeroed memory will do): attention loads whole 16-slot
 * blocks and weights slots past a sequence's length by exactly zero, which
 * keeps them out of the result only if they are finite.  The caller keeps
 * d_kv alive until vs_kv_destroy, which waits for the device. */
vs_status vs_kv_create(vs_model* m, void* d_kv, int32_t n_blocks, int32_t max_seqs, int32_t max_blocks_per_seq,
                       void* stream, vs_kv** out);
void vs_kv_destroy(vs_kv* kv);
/* Open a sequence able to hold max_len KV slots (prompt + generated tokens
 * + in-round scratch); reserves its blocks from the pool up front and keeps
 * them until vs_seq_close (the "FlashSpec" page, §4.3 and §5.4, allocates
 * the KV cache statically for the longest generation; a rollback only moves
 * the sequence's length back, self-speculative decoding page §3.3, and the
 * slots past it are rewritten by the next round).  VS_E_NOKV when the pool
 * has too few free blocks, max_len needs more than max_blocks_per_seq
 * blocks, or every sequence slot is in use. */
vs_status vs_seq_open(vs_kv* kv, int32_t max_len, void* stream, int32_t* seq_id);
/* Declare a context the caller wrote itself: the K/V of slots 0..P-1 of
 * every layer are already in the sequence's blocks (layout of vs_kv_layer),
 * and the sequence continues with `pending` at position P (committed =
 * P + 1), as after a prefill of P + 1 tokens.  For a freshly opened
 * sequence; P below its capacity. */
vs_status vs_seq_assume(vs_kv* kv, int32_t seq, int32_t P, int32_t pending, void* stream);
/* Rewind a sequence that holds a context to its first P positions: KV of
 * slots 0..P-1 is kept as it is, `pending` becomes the token at position P
 * (no KV), committed = P + 1, and later slots become garbage.  P must not
 * exceed the sequence's current KV length, which the call reads back from
 * the device (it blocks on `stream`).  Errors: VS_E_STATE (not open, no
 * context), VS_E_NOKV (P beyond the length), VS_E_INVAL (token id). */
vs_status vs_seq_rewind(vs_kv* kv, int32_t seq, int32_t P, int32_t pending, void* stream);
vs_status vs_seq_close(vs_kv* kv, int32_t seq_id);
/* Device pointers of the per-sequence state arrays [max_seqs]:
 * P (KV length), pending token, committed count (read-only for callers). */
vs_status vs_kv_state(vs_kv* kv, int32_t** d_P, int32_t** d_pending, int32_t** d_committed);
/* Device pointers of layer `layer`'s K pool [n_blocks][Hkv][hd/8][16 keys][8]
 * (each block's K tile cut into 8-dim pieces, piece-major: key j, dim d at
 * ((d/8)*16 + j)*8 + d%8), V pool [n_blocks][Hkv][hd][16 keys] (bf16) and the
 * block table [max_seqs][max_blocks_per_seq] (int32). */
vs_status vs_kv_layer(vs_kv* kv, int32_t layer, void** d_k, void** d_v, int32_t** d_block_table);
/* Host-side upper bound of P for a sequence (exact after vs_kv_sync). */
vs_status vs_kv_sync(vs_kv* kv, void* stream); /* blocks: reads P back */

/* ---- the round ---- */
/* Prompt of n tokens (device) through all layers in passes of <= 64 rows;
 * sets P = n and pending = argmax (greedy) or a draw with d_u[32] (sample,
 * softmax at temperature temp) of the last row.  d_logits_last [V] optional.
 * This is the state every round starts from (self-speculative decoding page,
 * §4.2: the first draft input is the last accepted token, its position the
 * accepted length).  VS_E_STATE for a sequence that already holds a context,
 * VS_E_NOKV past its capacity. */
vs_status vs_prefill(vs_model* m, vs_kv* kv, int32_t seq, const int32_t* d_tokens, int32_t n, int32_t mode,
                     float temp, const double* d_u, float* d_logits_last, void* stream);

/* forward_layers(start, end) of the self-speculative decoding page (§4.2,
 * §4.3: one decoder over a shared cache, run from any start layer to any end
 * layer at a position offset): layers [start, end) over the batch rows.
 * Input: token ids (start == 0) or hidden rows [M][d] (start > 0), rows in
 * batch order.  Writes each layer's K/V at the rows' slots (P + in-round
 * index).  d_hidden_out [M][d] optional (the hidden rows after layer end-1,
 * before any final norm).  Errors as vs_verify. */
vs_status vs_forward_layers(vs_model* m, vs_kv* kv, const vs_batch* b, int32_t start, int32_t end,
                            const int32_t* d_tokens, const float* d_hidden_in, float* d_hidden_out, void* stream);
/* Final RMSNorm + LM head of hidden rows [M][d] -> logits [M][V] (fp32).
 * The page applies the final norm also after the exit layer (self-
 * speculative decoding page, §3.1 and §4.2).  M in 1..max_rows of the
 * model (VS_E_SHAPE otherwise). */
vs_status vs_head(vs_model* m, int32_t M, const float* d_hidden, float* d_logits, void* stream);

/* Chain draft (self-speculative decoding page, §2.1 and §4.2: the first L
 * layers + final norm + head, k serial steps, each writing its first-L KV
 * into the shared cache at slot P + s; §3.3 for the reuse by the verify) of
 * k[i] tokens for each sequence (host array, 0..16): k[i]
 * serial steps of layers 0..L-1 + final norm + head, then a finishing
 * first-L pass over the last draft token.  Greedy takes the argmax; sample
 * draws from softmax(z/temp) with uniform slot s of d_u[i][48].
 * Outputs, in verify-row order (sequence i owns rows R_i..R_i+k[i]):
 *   d_tokens [M]: x, d_1..d_k;  d_hidden_L [M][d]: layer-L input of each row;
 *   d_draft_logits [M][V] (optional; row R_i+s holds the logits that drew
 *   d_{s+1}, the last row of each sequence is left untouched). */
vs_status vs_draft(vs_model* m, vs_kv* kv, int32_t n_seq, const int32_t* seq, const int32_t* k, int32_t mode,
                   float temp, const double* d_u, int32_t* d_tokens, float* d_hidden_L, float* d_draft_logits,
                   void* stream);

/* Tree draft of one sequence ("FlashSpec" page, lnrk.cn/news/47842, §2.2,
 * §3.2; the shape is this library's reading of its 63-node tree): the root
 * is the pending token; every expanded node gets its `topk` most probable
 * children under softmax(z/temp) of the draft (layers 0..L-1 + final norm +
 * head, probabilities in fp64); a path's score is the product of the
 * probabilities along it; the kept set is the top `keep` non-root nodes by
 * (score desc, depth asc, creation order), grown level by level to `depth`
 * levels, expanding at each level only the kept nodes of that depth.
 * Outputs the verify rows (R = 1 + keep, root first, level order: depth,
 * then the parent's row, then child rank; rows past the kept nodes, if any,
 * are padding that sees only itself): d_tokens [R], d_depth [R],
 * d_mask [R] (ancestor-or-self bits over rows), d_parent [R] (parent's row,
 * -1 for the root and padding), d_hidden_L [R][d] (layer-L input of each
 * row; the rows' first-L KV is written at slots P + row).  d_level_logits
 * (optional) [depth][R][V] receives each level pass's head output.
 * Limits: topk <= 8, depth <= 8, 1 + keep <= 64 and <= max_rows, at most
 * 1024 nodes; the sequence needs capacity P + R. */
vs_status vs_draft_tree(vs_model* m, vs_kv* kv, int32_t seq, int32_t topk, int32_t depth, int32_t keep, float temp,
                        int32_t* d_tokens, int32_t* d_depth, uint64_t* d_mask, int32_t* d_parent, float* d_hidden_L,
                        float* d_level_logits, void* stream);

/* Verify (self-speculative decoding page, §4.3: one forward over the k+1
 * rows from the exit layer at position offset P, reusing the draft's
 * first-L KV, §2.3; "FlashSpec" page, §2.2 and §3.2, for a tree: the rows
 * in level order with ancestor masks and per-node positions P + depth):
 * layers start_layer..N-1 over the batch rows (input hidden_L rows [M][d],
 * or token ids [M] when start_layer == 0), then the final norm and head ->
 * d_logits [M][V] fp32, rows in batch order.  Writes the rows' K/V of layers
 * start_layer..N-1 at slots P + in-round index.  Enqueues only (no host
 * synchronisation).  Depth and mask arrays are device data and are not
 * checked: a mask bit must name an earlier row of the same sequence, or the
 * row itself.  Errors: VS_E_INVAL (start layer, NULL buffers, a sequence
 * listed twice), VS_E_SHAPE (more than 64 rows for a sequence, more than the
 * model's max_rows or VS_MAX_PASS_ROWS in all, a pass the attention
 * workspace cannot hold), VS_E_NOKV (rows past a sequence's capacity),
 * VS_E_STATE (sequence not open or without context). */
vs_status vs_verify(vs_model* m, vs_kv* kv, const vs_batch* b, int32_t start_layer, const int32_t* d_tokens,
                    const float* d_hidden_in, float* d_logits, void* stream);

/* Accept (self-speculative decoding page, §2.4 and §4.3: min(1, p/q) left
 * to right, residual max(0, p - q) renormalised on the first reject, p
 * itself if that is empty, a bonus draw from the last row when all pass;
 * "DSpark" page, §2.1, for greedy block verification; "FlashSpec" page,
 * §2.2, for the longest accepted root-to-leaf path of a tree; the
 * "推测解码" page, §2.2, for the three-stage flow).
 * Greedy (any mask shape): walk from row 0 of each sequence to the
 * child whose token equals the argmax of the current row (lowest id on
 * ties); a = path length, y = argmax at the last node.  Sample (chain only):
 * for i < k test u[16+i] < min(1, p_i(d)/q_i(d)) with p = softmax(z/temp) of
 * d_logits row i and q of d_draft_logits row i, both in fp64; on the first
 * reject draw y from normalize(max(0, p-q)) (p if that sums to <= 0) with
 * u[32]; if all pass draw y from p_k.
 * d_result [n_seq][24]: a, y, flags (bit0 near-tie), n_path, path rows. */
vs_status vs_accept(vs_model* m, const vs_batch* b, int32_t mode, float temp, const int32_t* d_tokens,
                    const float* d_logits, const float* d_draft_logits, const double* d_u, int32_t* d_result,
                    void* stream);

/* Stochastic chain accept with a top-p target ("self-speculative" page,
 * §3.4): the draft keeps its full distribution q (drafts are sampled from
 * it), the target p = softmax(logits / temp) of each row is truncated to its
 * top-p set and renormalised there, then the test of vs_accept runs with
 * that p: accept iff u < min(1, p(d)/q(d)), residual max(0, p - q), bonus
 * from the last row's truncated p.  The top-p set of a row is the shortest
 * prefix, in order of (probability desc, id asc), whose probability reaches
 * top_p.  top_p in (0, 1]; 1 is vs_accept.  Buffers, uniforms and result as
 * for vs_accept in VS_SAMPLE mode; errors as vs_accept, VS_E_INVAL for
 * top_p outside (0, 1]. */
vs_status vs_accept_top_p(vs_model* m, const vs_batch* b, float temp, double top_p, const int32_t* d_tokens,
                          const float* d_logits, const float* d_draft_logits, const double* d_u, int32_t* d_result,
                          void* stream);

/* vs_accept without a model or workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, rules and results as
 * vs_accept (VS_GREEDY any mask shape, VS_SAMPLE chains), with the model
 * handle replaced by the vocabulary size (a multiple of 16 in [16, 32768]).
 * The per-row statistics live in a fixed device array inside the library
 * (about 60 KB per GPU, held until the process ends): at most
 * VS_MAX_PASS_ROWS rows per call, VS_E_SHAPE beyond.  Calls no allocating
 * routine.  Calls on one GPU share that array: calls that overlap on one GPU
 * (different streams, or host threads) race and must be ordered by the
 * caller.  The stream must belong to the current device. */
vs_status vs_accept_noalloc(int32_t vocab, const vs_batch* b, int32_t mode, float temp, const int32_t* d_tokens,
                            const float* d_logits, const float* d_draft_logits, const double* d_u, int32_t* d_result,
                            void* stream);

/* Commit (self-speculative decoding page, §3.3: the write position goes back
 * to the accepted length, and the cache position must equal the sequence
 * length after it; §4.5: each sequence of a batch advances by its own
 * count): P += a + 1, pending = y, committed += a + 1, read from d_result
 * on the device (no host synchronisation).  For masks that are not
 * chains, first copies the K/V (all layers) of the accepted path rows
 * P + path[i] to slots P + 1 + i (the "FlashSpec" page, §2.2: the accepted
 * path is what the next round continues from).  Same batch as the accept
 * that wrote d_result. */
vs_status vs_commit(vs_model* m, vs_kv* kv, const vs_batch* b, const int32_t* d_result, void* stream);

/* One chain round: vs_draft + vs_verify(exit_layer) + vs_accept + vs_commit
 * with the model's own scratch for tokens, hidden rows and logits.
 * d_result as for vs_accept; d_tokens [M] receives the round's row tokens. */
vs_status vs_step(vs_model* m, vs_kv* kv, int32_t n_seq, const int32_t* seq, const int32_t* k, int32_t mode,
                  float temp, const double* d_u, int32_t* d_tokens, int32_t* d_result, void* stream);

/* Confidence of the target over each sequence's verify block ("DSpark" page,
 * §2.2): per sequence, the mean over its rows of p_top1 and of p_top1 - p_top2
 * with p = softmax(logits row / temp), computed in fp64 from the fp32 logits.
 * d_logits [M][V] in batch row order; d_conf [n_seq][2] (device, fp64):
 * (mean top-1 probability, mean top-1 minus top-2 gap).  Asynchronous on the
 * stream; errors: VS_E_INVAL (null pointer, temp <= 0), VS_E_SHAPE (batch). */
vs_status vs_confidence(vs_model* m, const vs_batch* b, float temp, const float* d_logits, double* d_conf,
                        void* stream);

/* Confidence-scheduled draft length per request ("DSpark" page, §2.2-§2.3),
 * host code only.  After a round with a accepted of k drafts:
 *   ema <- 0.2 * a/k + 0.8 * ema                      (ema starts at 0.5)
 *   C    = 0.4 * top1 + 0.3 * min(5 * gap, 1) + 0.3 * ema
 *   k'   = clamp(int(min_k + (max_k - min_k) * (C - low) / (high - low)))
 * and k' = min_k when the first draft was rejected (a == 0).  The caller owns
 * the state structs (one per request); vs_sched_init sets ema = 0.5 and k to
 * k0 clamped to [min_k, max_k].  Errors: VS_E_INVAL for a bad config
 * (1 <= min_k <= max_k <= VS_MAX_K, low < high), a outside [0, k] or a
 * non-finite confidence; the state is unchanged on error. */
typedef struct vs_sched_cfg {
  int32_t min_k, max_k; /* 2, 16 */
  double low, high;     /* 0.3, 0.7 */
} vs_sched_cfg;
typedef struct vs_spec_state {
  double ema;           /* moving average of the per-round acceptance a/k */
  int32_t k;            /* draft length of the next round */
  int32_t rounds;       /* rounds seen */
  int32_t last_a;       /* accepted drafts of the last round (-1 before the first) */
} vs_spec_state;
vs_status vs_sched_init(const vs_sched_cfg* c, int32_t k0, vs_spec_state* s);
vs_status vs_sched_update(const vs_sched_cfg* c, vs_spec_state* s, int32_t a, double avg_top1, double avg_gap);

/* Windowed dynamic draft length with a context-cost cut-off (self-speculative
 * decoding page, §3.2 and §5.3), host code only.  The state keeps the last
 * `window` rounds' (accepted, drafted) counts; alpha = sum accepted / sum
 * drafted over them.  After each round with drafts:
 *   alpha > up   -> k + 1,   alpha < down -> k - 1,   k kept in [min_k, max_k]
 * (the controller's k).  When c_draft > 0 (the cost of one draft step over
 * one full forward at the current context) the next round's draft length is
 * min(controller k, k_c) with k_c = the k in [1, max_k] that maximises
 * E(k) / (c_draft * k + 1), E(k) = (1 - alpha^(k+1)) / (1 - alpha) (the
 * smallest such k on ties); when k_c < min_k, or no k gives a speedup above
 * 1, the next round is a plain decoding step (*k_next = 0), which leaves the
 * window unchanged.  Errors: VS_E_INVAL for a bad config (1 <= window <=
 * VS_DYNK_MAX_WINDOW, 1 <= min_k <= max_k <= VS_MAX_K, down <= up), a
 * outside [0, k_used] or a negative k_used; the state is unchanged on error. */
#define VS_DYNK_MAX_WINDOW 256
typedef struct vs_dynk_cfg {
  int32_t window;       /* 64 */
  int32_t min_k, max_k; /* 2, 8 */
  double up, down;      /* 0.85, 0.7 */
} vs_dynk_cfg;
typedef struct vs_dynk_state {
  int32_t k;                            /* the controller's draft length */
  int32_t n, head;                      /* rounds in the window, next slot */
  int32_t a[VS_DYNK_MAX_WINDOW];        /* accepted drafts per round */
  int32_t drafted[VS_DYNK_MAX_WINDOW];  /* drafts per round */
  double alpha;                         /* window acceptance (1 before any round) */
} vs_dynk_state;
vs_status vs_dynk_init(const vs_dynk_cfg* c, int32_t k0, vs_dynk_state* s);
vs_status vs_dynk_update(const vs_dynk_cfg* c, vs_dynk_state* s, int32_t a, int32_t k_used, double c_draft,
                         int32_t* k_next);

/* n-gram (prompt-copy) drafting ("self-speculative" page, §2.2: draft
 * tokens copied from text that already appeared), host code only.  For g =
 * max_ngram down to min_ngram, take the last g tokens of tokens[0..n) and
 * find their latest earlier occurrence starting at i with i + g < limit,
 * limit = min(n, search_len); the proposal is tokens[i + g .. min(i + g +
 * k_max, limit)).  The first g that matches wins; *n_out = 0 when none does.
 * out receives at most k_max ids.  Errors: VS_E_INVAL (null pointers,
 * 1 <= min_ngram <= max_ngram, k_max in [0, VS_MAX_K], n >= 1). */
vs_status vs_ngram_propose(const int32_t* tokens, int32_t n, int32_t search_len, int32_t min_ngram,
                           int32_t max_ngram, int32_t k_max, int32_t* out, int32_t* n_out);

/* One greedy round of one sequence with an n-gram draft and a full-depth
 * verify (no draft model, so no first-L KV to reuse): h_history [n_hist]
 * (host) is the sequence's committed tokens, its last one the pending token
 * at position P.  Proposes d_1..d_k with vs_ngram_propose, writes [x,
 * d_1..d_k] to d_tokens, runs vs_verify(start_layer 0) over the k+1 rows
 * (k = 0 is a plain decoding step), vs_accept (greedy) and vs_commit, and
 * blocks until h_result [VS_RESULT_INTS] holds the result; *k_out = k.
 * Errors: as vs_ngram_propose and vs_verify. */
vs_status vs_step_ngram(vs_model* m, vs_kv* kv, int32_t seq, const int32_t* h_history, int32_t n_hist,
                        int32_t search_len, int32_t min_ngram, int32_t max_ngram, int32_t k_max, int32_t* d_tokens,
                        int32_t* d_result, int32_t* h_result, int32_t* k_out, void* stream);

/* One greedy chain round of n_seq requests with per-request draft lengths
 * states[i].k (vs_step), then vs_confidence over each request's k+1 verify
 * rows, then vs_sched_update of every state.  Blocks until the round is done:
 * h_result [n_seq][VS_RESULT_INTS] (host) receives d_result, and h_conf
 * [n_seq][2] (host, may be NULL) the confidences.  d_tokens [sum k+1] and
 * d_result [n_seq][VS_RESULT_INTS] are device buffers as for vs_step.
 * Errors: as vs_step; VS_E_STATE when a state's k lies outside the schedule. */
vs_status vs_step_sched(vs_model* m, vs_kv* kv, int32_t n_seq, const int32_t* seq, const vs_sched_cfg* c,
                        vs_spec_state* states, int32_t* d_tokens, int32_t* d_result, int32_t* h_result,
                        double* h_conf, void* stream);

/* Per-kernel-family timing with HIP events on the launching stream, for the
 * selected families only.  `mask` selects families by bit, in the order vs_stats_read
 * reports them: gemm_qkv, gemm_o, gemm_gate_up, gemm_down, gemm_head,
 * attention, small; 0 disables, -1 selects all.  While a mask is
 * set every launch gets an end event timestamped by the kernel itself, and a
 * selected launch is charged from the later of the previous launch's end and
 * its own start event to its end.  vs_stats_read synchronises. */
typedef struct vs_kernel_stat {
  char name[32];
  int64_t launches;
  double total_ms;
  double bytes; /* algorithmic HBM bytes of all timed launches */
} vs_kernel_stat;
vs_status vs_stats_enable(vs_model* m, int32_t mask);
vs_status vs_stats_read(vs_model* m, vs_kernel_stat* out, int32_t max, int32_t* n_out);
vs_status vs_stats_reset(vs_model* m);

/* Achievable HBM read bandwidth, the denominator beside the 8 TB/s peak when
 * the weight streams of the verify step are judged: one launch reads `bytes`
 * (a positive multiple of 16; d_src 16-byte aligned) with 16-byte loads,
 * 2048 workgroups of 256 threads each streaming one contiguous range, and
 * writes one checksum word per workgroup to d_sink (2048 words).  The caller
 * times it (events on `stream`).  Errors: VS_E_INVAL. */
vs_status vs_read_probe(const void* d_src, size_t bytes, uint32_t* d_sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif
