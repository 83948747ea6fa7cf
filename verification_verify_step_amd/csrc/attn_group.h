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

// Workgroup layout of sequence i (AttnArgs.wg_start, 8-aligned): its
// groups g = s * Hkv + kvh (split of the host's bound, KV head; the count
// padded to a multiple of 8, splits the device's P does not need last) times its blocks of query groups, laid
// out so that the blocks of one group sit on one XCD back to back: local
// index ((g / 8) * nqb + qb) * 8 + g % 8 (block b runs on XCD b % 8).  The
// device's own split count max(1, ceil(P / kps)) decides which splits run;
// its last split also takes the in-round keys.  With more than one split a
// wave writes its query group's partial record at split s; the combine
// kernel then writes the result.
constexpr int kAttnXcds = 8;            // workgroup b runs on XCD b % 8
constexpr int kAttnStepKeys = 32;       // keys per step
constexpr int kAttnGroupSteps = 32;     // steps per split at most (two block-table entries per step, one per lane)
constexpr int kAttnGroupMaxSplits = 64;
constexpr int kAttnGroupWaves = 4;      // waves (query groups) per workgroup
void launch_attention_group(const AttnArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace vs
