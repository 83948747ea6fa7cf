// Grouped attention (internal launch interface).
//
// For passes whose KV heads carry more than one query group (GQA heads, or
// many rows per sequence: a token tree), one workgroup takes one
// (sequence, KV head, block of up to four query groups, key split): its threads
// bring each 32-key step of K and V into LDS once, and each wave runs the
// online softmax of one query group over it.  The splits of a sequence are
// merged by a second, small kernel.
#pragma once
#include "kernels.h"

namespace vs {

// Map entries: i | kvh << 6 | qb << 13 | s << 20 (sequence index, KV head,
// query-group block, split), -1 for padding.  Sequence i has a.nsplit[i]
// splits of a.kps committed keys; its last split also takes the in-round
// keys.  With more than one split a workgroup writes, per query group, a
// partial record at split s of the layout of AttnArgs with wpb = a.n_split
// (the largest nsplit); the combine kernel then writes the result.
constexpr int kAttnStepKeys = 32;       // keys per step
constexpr int kAttnGroupSteps = 32;     // steps per split at most (two block-table entries per step, one per lane)
constexpr int kAttnGroupMaxSplits = 64;
constexpr int kAttnGroupWaves = 4;      // waves (query groups) per workgroup
void launch_attention_group(const AttnArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace vs
