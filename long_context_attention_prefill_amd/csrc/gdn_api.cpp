// gdn_api.cpp -- C ABI of the chunked gated-delta-rule prefill: argument
// checks and work planning (host only, no HIP headers).
//
// Every check runs before any device work.  A batch is cut into launches of at
// most gdn::kMaxSeqsPerLaunch consecutive sequences; each launch's items
// (64-token chunks x heads) use the workspace from its start, so launches run
// in order on the caller's stream and the workspace is sized for the largest.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "gdn_prefill.h"
#include "gdn_launch.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

int64_t chunks_of(int64_t len) { return (len + gdn::kChunk - 1) / gdn::kChunk; }

int check_shape(const int32_t *cu, int32_t n_seqs, int32_t h, int32_t dk, int32_t dv, int32_t dtype,
                int64_t *T_out) {
  if (n_seqs < 0 || h <= 0) return ATTN_EINVAL;
  if (n_seqs > 0 && cu == nullptr) return ATTN_EINVAL;
  int64_t T = 0;
  if (n_seqs > 0) {
    if (cu[0] != 0) return ATTN_EINVAL;
    for (int32_t b = 0; b < n_seqs; ++b)
      if (cu[b + 1] < cu[b]) return ATTN_EINVAL;
    T = cu[n_seqs];
  }
  if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (dk != gdn::kDk || dv != gdn::kDv) return ATTN_EUNSUPPORTED;
  // element offsets T * h * d and item counts must stay far from overflow
  if (static_cast<double>(T) * h * dk > 4.0e18 || static_cast<double>(n_seqs) * h * dv * dk > 4.0e18)
    return ATTN_EUNSUPPORTED;
  *T_out = T;
  return ATTN_OK;
}

// Items (chunks x heads) of the largest launch.
int64_t max_launch_items(const int32_t *cu, int32_t n_seqs, int32_t h) {
  int64_t best = 0;
  for (int32_t base = 0; base < n_seqs; base += gdn::kMaxSeqsPerLaunch) {
    const int32_t end = std::min(n_seqs, base + gdn::kMaxSeqsPerLaunch);
    int64_t chunks = 0;
    for (int32_t b = base; b < end; ++b) chunks += chunks_of(cu[b + 1] - cu[b]);
    best = std::max(best, chunks * h);
  }
  return best;
}

int check_all(const void *q, const void *k, const void *v, const float *g, const float *beta,
              const float *s0, const void *out, const float *s1, const int32_t *cu, int32_t n_seqs,
              int32_t h, int32_t dk, int32_t dv, int32_t dtype, float scale, const void *ws,
              uint64_t ws_bytes, int64_t *T_out, uint64_t *need_out) {
  int64_t T = 0;
  int rc = check_shape(cu, n_seqs, h, dk, dv, dtype, &T);
  if (rc != ATTN_OK) return rc;
  if (!std::isfinite(scale)) return ATTN_EINVAL;
  const uint64_t qk_bytes = static_cast<uint64_t>(T) * h * dk * 2;
  const uint64_t v_bytes = static_cast<uint64_t>(T) * h * dv * 2;
  const uint64_t gb_bytes = static_cast<uint64_t>(T) * h * 4;
  const uint64_t st_bytes = static_cast<uint64_t>(n_seqs) * h * dv * dk * 4;
  if (T > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr || out == nullptr)
      return ATTN_EINVAL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(g, 4) ||
        !aligned(beta, 4))
      return ATTN_EINVAL;
  }
  if ((s0 != nullptr && !aligned(s0, 16)) || (s1 != nullptr && !aligned(s1, 16))) return ATTN_EINVAL;
  // out and the final state may overlap nothing but (for the state) the initial state itself
  const void *ins[] = {q, k, v, g, beta};
  const uint64_t in_bytes[] = {qk_bytes, qk_bytes, v_bytes, gb_bytes, gb_bytes};
  for (int i = 0; i < 5; ++i) {
    if (overlaps(out, v_bytes, ins[i], in_bytes[i])) return ATTN_EINVAL;
    if (overlaps(s1, st_bytes, ins[i], in_bytes[i])) return ATTN_EINVAL;
  }
  if (overlaps(out, v_bytes, s0, st_bytes) || overlaps(out, v_bytes, s1, st_bytes)) return ATTN_EINVAL;
  if (s1 != nullptr && s0 != nullptr && s1 != s0 && overlaps(s1, st_bytes, s0, st_bytes)) return ATTN_EINVAL;
  const uint64_t need = static_cast<uint64_t>(max_launch_items(cu, n_seqs, h)) * gdn::kItemBytes;
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need || !aligned(ws, 16)) return ATTN_EINVAL;
    const void *all[] = {q, k, v, g, beta, s0, out, s1};
    const uint64_t all_bytes[] = {qk_bytes, qk_bytes, v_bytes, gb_bytes, gb_bytes, st_bytes, v_bytes, st_bytes};
    for (int i = 0; i < 8; ++i)
      if (overlaps(ws, need, all[i], all_bytes[i])) return ATTN_EINVAL;
  }
  *T_out = T;
  *need_out = need;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int gdn_prefill_workspace_size(const int32_t *cu_seqlens, int32_t n_seqs, int32_t n_heads,
                               int32_t head_dim_k, int32_t head_dim_v, int32_t dtype, uint64_t *bytes) {
  if (bytes == nullptr) return ATTN_EINVAL;
  int64_t T = 0;
  const int rc = check_shape(cu_seqlens, n_seqs, n_heads, head_dim_k, head_dim_v, dtype, &T);
  if (rc != ATTN_OK) return rc;
  *bytes = static_cast<uint64_t>(max_launch_items(cu_seqlens, n_seqs, n_heads)) * gdn::kItemBytes;
  return ATTN_OK;
}

int gdn_prefill_check(const void *q, const void *k, const void *v, const float *g, const float *beta,
                      const float *initial_state, const void *out, const float *final_state,
                      const int32_t *cu_seqlens, int32_t n_seqs, int32_t n_heads, int32_t head_dim_k,
                      int32_t head_dim_v, int32_t dtype, float scale, const void *workspace,
                      uint64_t workspace_bytes) {
  int64_t T = 0;
  uint64_t need = 0;
  return check_all(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens, n_seqs, n_heads,
                   head_dim_k, head_dim_v, dtype, scale, workspace, workspace_bytes, &T, &need);
}

int gdn_prefill(const void *q, const void *k, const void *v, const float *g, const float *beta,
                const float *initial_state, void *out, float *final_state, const int32_t *cu_seqlens,
                int32_t n_seqs, int32_t n_heads, int32_t head_dim_k, int32_t head_dim_v, int32_t dtype,
                float scale, void *workspace, uint64_t workspace_bytes, void *stream) {
  int64_t T = 0;
  uint64_t need = 0;
  int rc = check_all(q, k, v, g, beta, initial_state, out, final_state, cu_seqlens, n_seqs, n_heads,
                     head_dim_k, head_dim_v, dtype, scale, workspace, workspace_bytes, &T, &need);
  if (rc != ATTN_OK) return rc;
  // nothing to compute and no state to pass through
  if (T == 0 && final_state == nullptr) return ATTN_OK;
  std::vector<gdn::GdnArgs> plan;
  for (int32_t base = 0; base < n_seqs; base += gdn::kMaxSeqsPerLaunch) {
    const int32_t end = std::min(n_seqs, base + gdn::kMaxSeqsPerLaunch);
    gdn::GdnArgs a = {};
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.s0 = initial_state;
    a.out = out;
    a.s_final = final_state;
    a.h = n_heads;
    a.scale = scale;
    a.n_seqs = end - base;
    a.seq_base = base;
    int64_t chunks = 0;
    for (int32_t b = base; b < end; ++b) {
      const int32_t i = b - base;
      a.seq_start[i] = cu_seqlens[b];
      a.seq_len[i] = cu_seqlens[b + 1] - cu_seqlens[b];
      a.chunk_start[i] = static_cast<int32_t>(chunks);
      chunks += chunks_of(a.seq_len[i]);
    }
    a.chunk_start[a.n_seqs] = static_cast<int32_t>(chunks);
    const int64_t items = chunks * n_heads;
    if (items > INT32_MAX || static_cast<int64_t>(a.n_seqs) * n_heads * (gdn::kDv / gdn::kSliceRows) > INT32_MAX)
      return ATTN_EUNSUPPORTED;
    a.total_items = static_cast<int32_t>(items);
    char *base_ptr = static_cast<char *>(workspace);
    const uint64_t it = static_cast<uint64_t>(items);
    a.ws_w = base_ptr;
    a.ws_u = base_ptr + it * gdn::kWBytes;
    a.ws_p = base_ptr + it * (gdn::kWBytes + gdn::kUBytes);
    a.ws_kd = base_ptr + it * (gdn::kWBytes + gdn::kUBytes + gdn::kPBytes);
    a.ws_gam = reinterpret_cast<float *>(base_ptr + it * (gdn::kWBytes + gdn::kUBytes + gdn::kPBytes + gdn::kKdBytes));
    a.ws_q = base_ptr + it * (gdn::kWBytes + gdn::kUBytes + gdn::kPBytes + gdn::kKdBytes + gdn::kGamBytes);
    // without a final state, a launch of empty sequences has nothing to do
    if (items == 0 && final_state == nullptr) continue;
    plan.push_back(a);
  }
  for (const gdn::GdnArgs &a : plan)
    if (gdn::launch_gdn(a, stream) != 0) return ATTN_ELAUNCH;
  return ATTN_OK;
}

}  // extern "C"
