// attn_launch.h -- what the host planner hands to a kernel launch.
//
// Internal to the library: shared by the host translation unit (argument
// checks, work planning) and the HIP translation unit (kernels, launches).
// Plain data only, so the struct can travel as a kernel argument.
#pragma once

#include <stdint.h>

namespace attn {

// Sequences per launch.  Longer batches are split over several launches on
// the same stream; each launch writes a disjoint set of output rows.
constexpr int kMaxSeqsPerLaunch = 64;

enum MaskKind : int32_t { kCausal = 0, kFull = 1, kWindow = 2 };

// One launch: a group of non-empty sequences sorted by length, longest
// first, and everything a workgroup needs to find its item.
struct LaunchArgs {
  const void *q;
  const void *k;
  const void *v;
  void *out;
  int32_t hq;          // query heads
  int32_t hkv;         // key/value heads
  int32_t group;       // hq / hkv
  int32_t mask_kind;   // MaskKind
  int32_t window;      // block length for kWindow
  float c;             // scale * log2(e): scores enter exp2 in these units
  int32_t n_seqs;      // sequences in this launch (<= kMaxSeqsPerLaunch)
  int32_t bm;          // query rows per workgroup
  int32_t total_items; // workgroups = hq * sum(seq_tiles)
  int32_t seq_start[kMaxSeqsPerLaunch];  // packed index of token 0
  int32_t seq_len[kMaxSeqsPerLaunch];    // tokens
  int32_t seq_tiles[kMaxSeqsPerLaunch];  // ceil(len / bm), non-increasing
  // Causal order only (items by query-tile level, heaviest first): query-tile
  // levels m in [seq_tiles[k], seq_tiles[k-1]) hold the k longest sequences,
  // and their items start at level_start[k-1]; level_start[n_seqs] =
  // total_items (seq_tiles[n_seqs] reads as 0).
  int32_t level_start[kMaxSeqsPerLaunch + 1];
};

// Kernel families.  Each returns 0 or a hipError_t value.
int launch_bf16(const LaunchArgs &a, int head_dim, void *stream);
int launch_f32(const LaunchArgs &a, int head_dim, void *stream);
// Query rows per workgroup of each family (the planner tiles with it).
int rows_per_workgroup_bf16(int head_dim);
int rows_per_workgroup_f32(int head_dim);

}  // namespace attn
