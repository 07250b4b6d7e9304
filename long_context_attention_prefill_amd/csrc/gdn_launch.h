// gdn_launch.h -- what the host planner hands to the gated-delta-rule kernels.
//
// Internal to the library: shared by the host translation unit (gdn_api.cpp)
// and the HIP translation unit (gdn_fwd.hip).  Plain data only, so the struct
// can travel as a kernel argument.
#pragma once

#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;              // tokens per chunk
constexpr int kMaxSeqsPerLaunch = 64;   // longer batches: several launches in order
constexpr int kDk = 128;
constexpr int kDv = 128;
constexpr int kSliceRows = 32;          // value dims of the state per scan workgroup

// Workspace per (chunk, head) item, each array item-major:
//   w    bf16 [64][128]  T diag(beta Gamma) K       (WY key combinations)
//   u    bf16 [128][64]  (T diag(beta) V)^T         (WY value combinations, transposed)
//   p    bf16 [64][64]   scale (Q K^T o M), M_ij = Gamma_i / Gamma_j (i >= j)
//   kd   bf16 [128][64]  K^T diag(Gamma_last / Gamma)  (transposed)
//   gam  f32  [64]       Gamma_i = exp(cumulative g within the chunk)
//   q    bf16 [64][128]  the chunk's queries (rows past its end zero)
// The bf16 matrices are stored in the order the scan's waves read them as
// MFMA operands (gdn_fwd.hip, frag_index and u_frag_index), so each 64-lane
// load of the scan reads 1 KB of consecutive bytes.
constexpr uint64_t kWBytes = kChunk * kDk * 2;
constexpr uint64_t kUBytes = kChunk * kDv * 2;
constexpr uint64_t kPBytes = kChunk * kChunk * 2;
constexpr uint64_t kKdBytes = kDk * kChunk * 2;
constexpr uint64_t kGamBytes = kChunk * 4;
constexpr uint64_t kQBytes = kChunk * kDk * 2;
constexpr uint64_t kItemBytes = kWBytes + kUBytes + kPBytes + kKdBytes + kGamBytes + kQBytes;

struct GdnArgs {
  const void *q;            // [T][H][128] bf16
  const void *k;
  const void *v;
  const float *g;           // [T][H]
  const float *beta;        // [T][H]
  const float *s0;          // [n][H][128][128] or null (call-wide sequence index)
  void *out;                // [T][H][128] bf16
  float *s_final;           // [n][H][128][128] or null
  void *ws_w;               // item-major arrays, items of this launch
  void *ws_u;
  void *ws_p;
  void *ws_kd;
  float *ws_gam;
  void *ws_q;
  int32_t h;                // heads
  float scale;
  int32_t n_seqs;           // sequences in this launch
  int32_t seq_base;         // call-wide index of the launch's first sequence (states)
  int32_t total_items;      // chunks of the launch x heads
  int32_t seq_start[kMaxSeqsPerLaunch];       // packed index of the first token
  int32_t seq_len[kMaxSeqsPerLaunch];         // tokens (may be 0)
  int32_t chunk_start[kMaxSeqsPerLaunch + 1]; // first chunk of each sequence in the launch
};

// Prep (parallel over chunks x heads), then the scan (one workgroup per
// sequence, head and 32 state rows); both on `stream`.  Returns 0 or a
// hipError_t value.
int launch_gdn(const GdnArgs &a, void *stream);

}  // namespace gdn
