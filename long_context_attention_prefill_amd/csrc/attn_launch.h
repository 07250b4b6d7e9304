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

// bf16 launches of at most kKeyHalvesFewItems 128-row items (half the CUs of
// an MI355X), or of at most kKeyHalvesMaxItems (1.5 per CU) whose longest
// item has at least 1.5 times the mean key count, take key halves: 64-row
// items, each half of the keys swept by its own pair of waves, so the launch
// has twice the workgroups.
constexpr int64_t kKeyHalvesFewItems = 128;
constexpr int64_t kKeyHalvesMaxItems = 384;

// bf16 launches whose exp2-unit scale c = scale * log2(e) has |c| at most
// this take the query pre-multiplied by c and rounded to bf16 (scores leave
// the MFMAs in exp2 units; each moves by about |c| 2^-9 |q . k|): every usual
// 1/sqrt(d) scale (|c| = 0.18 at d 64, 0.13 at d 128).  Larger scales, whose
// sharper softmax would magnify that rounding, keep the exact query, and so
// do launches that return the log-sum-exp (for a row with one visible key it
// is that key's score, where the rounding would show undamped).
constexpr float kPrescaleMaxC = 0.25f;

enum MaskKind : int32_t { kCausal = 0, kFull = 1, kWindow = 2 };

// One launch: a group of sequences with at least one query, sorted by query
// count, most first, and everything a workgroup needs to find its item.
// Sequence i has q_len[i] queries and k_len[i] >= q_len[i] keys; its queries
// are the last q_len[i] positions, so local query r sits at position
// r + k_len[i] - q_len[i].
struct LaunchArgs {
  const void *q;
  const void *k;
  const void *v;
  void *out;
  float *lse;          // [Tq][hq] natural-log sum of exp(scale * score), or null
  int32_t hq;          // query heads
  int32_t hkv;         // key/value heads
  int32_t q_stride;    // elements between consecutive tokens of q (hq * d when packed)
  int32_t kv_stride;   // the same for k and v (hkv * d when packed); out is always packed
  int32_t group;       // hq / hkv
  int32_t mask_kind;   // MaskKind
  int32_t window;      // block length for kWindow
  float c;             // scale * log2(e): scores enter exp2 in these units
  int32_t n_seqs;      // sequences in this launch (<= kMaxSeqsPerLaunch)
  int32_t bm;          // query rows per workgroup
  int32_t total_items; // workgroups = hq * sum(seq_tiles)
  int32_t q_start[kMaxSeqsPerLaunch];    // packed index of the first query
  int32_t q_len[kMaxSeqsPerLaunch];      // queries
  int32_t k_start[kMaxSeqsPerLaunch];    // packed index of the first key/value
  int32_t k_len[kMaxSeqsPerLaunch];      // keys/values, >= q_len
  int32_t seq_tiles[kMaxSeqsPerLaunch];  // ceil(q_len / bm), non-increasing
  // Causal order only (items by query-tile level, heaviest first): query-tile
  // levels m in [seq_tiles[k], seq_tiles[k-1]) hold the k longest sequences,
  // and their items start at level_start[k-1]; level_start[n_seqs] =
  // total_items (seq_tiles[n_seqs] reads as 0).
  int32_t level_start[kMaxSeqsPerLaunch + 1];
  // Work tickets (device, two counters at zero), or null: workgroup b runs
  // item b of the order above if b < ticket_from, else item ticket_from +
  // tickets[0]++ claimed when it starts; tickets[1] counts finished
  // workgroups, and the last one puts both back to zero.
  int32_t *tickets;
  int32_t ticket_from;
  // bf16 only: 1 = key halves (bm = 64 rows; two pairs of waves sweep the two
  // halves of each item's key tiles and merge), for launches of few items
  int32_t key_halves;
  // full and window masks: the first xcd_tiles query tiles (a multiple of 16)
  // run XCD by XCD in runs of two tiles (see decode_item); 0 = plain order
  int32_t xcd_tiles;
};

// Decode: one query (the newest token) per sequence against its key/value
// cache.  An item is (sequence, KV head, block of up to 32 of its query heads,
// chunk of the visible keys); one wave computes an item.  Sequences of a
// launch are consecutive in the call.
constexpr int kMaxDecodeSeqsPerLaunch = 64;
constexpr int kDecodeTile = 32;  // keys per MFMA tile; chunks are multiples of it

struct DecodeArgs {
  const void *q;       // [n_seqs][hq][d], the launch's first sequence at row 0
  const void *k;       // [Tk][hkv][d], packed over the whole call
  const void *v;
  void *out;           // [n_seqs][hq][d], same rows as q
  float *lse;          // [n_seqs][hq] or null
  float *ws_o;         // [total_items][rows][d] unnormalised partial outputs (split mode)
  float *ws_ml;        // [total_items][rows][2]: exp2-unit reference and sum (split mode)
  int32_t hq;
  int32_t hkv;
  int32_t group;       // hq / hkv
  int32_t head_blocks; // ceil(group / 32)
  int32_t rows;        // min(group, 32): query heads per item
  int32_t chunk;       // keys per item, a multiple of kDecodeTile
  float c;             // scale * log2(e)
  int32_t n_seqs;
  int32_t total_items;
  int32_t direct;      // 1: one chunk per (sequence, head block): write out directly
  int32_t k_begin[kMaxDecodeSeqsPerLaunch];     // packed index of the first visible key
  int32_t k_count[kMaxDecodeSeqsPerLaunch];     // visible keys, >= 1
  int32_t splits[kMaxDecodeSeqsPerLaunch];      // ceil(k_count / chunk)
  int32_t item_start[kMaxDecodeSeqsPerLaunch + 1];
};

// Prefill over q, k, v whose tokens lie q_stride and kv_stride elements
// apart (heads still contiguous within a token; out packed), for callers
// inside the library that hold q, k and v as column blocks of one
// projection output.  Arguments as for attn_prefill_kv, checked by the
// caller; returns an ATTN_ status.
int prefill_strided(const void *q, const void *k, const void *v, void *out, float *lse,
                    const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t n_seqs,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                    int32_t mask_kind, int32_t window, float scale, int32_t q_stride,
                    int32_t kv_stride, void *stream);

// Kernel families.  Each returns 0 or a hipError_t value.
int launch_bf16(const LaunchArgs &a, int head_dim, void *stream);
int launch_f32(const LaunchArgs &a, int head_dim, void *stream);
// Decode (bf16, head_dim 64 or 128): the partial kernel, then, in split
// mode, the merge kernel; both on `stream`.
int launch_decode_bf16(const DecodeArgs &a, int head_dim, void *stream);

// Decode workspace the library holds itself (attn_decode_noalloc): a static
// device array of this many bytes on every GPU the library runs on.
constexpr uint64_t kDecodeScratchBytes = 16ull << 20;
// The device address of that array on the device `stream` belongs to (the
// current device for the null stream), looked up once per device; 0 or a
// hipError_t value.
int decode_scratch(void *stream, void **ptr);
// Query rows per workgroup of each family (the planner tiles with it).
int rows_per_workgroup_bf16(int head_dim);
int rows_per_workgroup_bf16_halves(int head_dim);  // with key halves
int rows_per_workgroup_f32(int head_dim);

// For a causal bf16 launch with many more items than workgroup slots: point
// a.tickets at the stream's counters (a static device array, one pair per
// stream and device) and set a.ticket_from to the device's workgroup slots;
// leaves a.tickets null (items bound to workgroups) on other launches, a
// stream under capture, the per-thread default stream, or a full array.
// 0 or a hipError_t.
int work_tickets(LaunchArgs &a, void *stream);

}  // namespace attn
