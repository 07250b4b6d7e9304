// vision_api.cpp -- C ABI of the vision attention block (include/vision_block.h):
// argument checks, workspace carving and the three stream-ordered steps.
// The QKV projection writes [q | k | v] rows of 3 H d values with the bias
// added in the GEMM's epilogue; the attention reads q, k and v in place as
// column blocks of those rows; the output projection adds its bias the same
// way.  Host only.
#include <algorithm>
#include <cstdint>

#include "vision_block.h"
#include "attn_launch.h"
#include "proj_launch.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

uint64_t round256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Workspace regions, each starting on a 256-byte boundary, both of the
// block's dtype: qkv [T][3 H d] (the QKV projection with its bias) and
// a [T][H d] (the attention output).
struct Carve {
  uint64_t qkv_bytes, a_bytes, total;
};

int shape_ok(int32_t h, int32_t d, int32_t hidden, int32_t dtype) {
  if (h <= 0 || hidden <= 0 || hidden % 8 != 0) return ATTN_EINVAL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_EUNSUPPORTED;
  if (d != 64 && d != 72 && d != 128) return ATTN_EUNSUPPORTED;
  if (static_cast<int64_t>(3) * h * d >= (int64_t(1) << 31)) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

Carve carve(int64_t t, int32_t h, int32_t d, int32_t dtype) {
  const uint64_t es = dtype == ATTN_F32 ? 4 : 2;
  const uint64_t hd = static_cast<uint64_t>(h) * d;
  Carve c;
  c.qkv_bytes = round256(static_cast<uint64_t>(t) * 3 * hd * es);
  c.a_bytes = round256(static_cast<uint64_t>(t) * hd * es);
  c.total = c.qkv_bytes + c.a_bytes;
  return c;
}

}  // namespace

extern "C" {

int vision_attention_block_workspace_size(int64_t tokens, int32_t n_heads, int32_t head_dim, int32_t hidden,
                                          int32_t dtype, uint64_t *bytes) {
  if (bytes == nullptr || tokens < 0) return ATTN_EINVAL;
  const int rc = shape_ok(n_heads, head_dim, hidden, dtype);
  if (rc != ATTN_OK) return rc;
  if (tokens >= (int64_t(1) << 31)) return ATTN_EUNSUPPORTED;
  *bytes = tokens == 0 ? 0 : carve(tokens, n_heads, head_dim, dtype).total;
  return ATTN_OK;
}

int vision_attention_block(const void *x, const void *w_qkv, const void *b_qkv, const void *w_o,
                           const void *b_o, void *out, const int32_t *cu_seqlens, int32_t n_seqs,
                           int32_t n_heads, int32_t head_dim, int32_t hidden, int32_t dtype,
                           int32_t mask_kind, int32_t window, float scale, void *workspace,
                           uint64_t workspace_bytes, void *stream) {
  int rc = shape_ok(n_heads, head_dim, hidden, dtype);
  if (rc != ATTN_OK) return rc;
  if (n_seqs < 0 || (n_seqs > 0 && cu_seqlens == nullptr)) return ATTN_EINVAL;
  int64_t T = 0;
  if (n_seqs > 0) {
    if (cu_seqlens[0] != 0) return ATTN_EINVAL;
    for (int32_t b = 0; b < n_seqs; ++b)
      if (cu_seqlens[b + 1] < cu_seqlens[b]) return ATTN_EINVAL;
    T = cu_seqlens[n_seqs];
  }
  if (T == 0) {
    // nothing to compute; the mask and scale must still be valid
    return attn_prefill_check(nullptr, nullptr, nullptr, nullptr, cu_seqlens, n_seqs, n_heads, n_heads, head_dim,
                              dtype, mask_kind, window, scale);
  }
  const void *ptrs[] = {x, w_qkv, b_qkv, w_o, b_o, out};
  for (const void *p : ptrs)
    if (p == nullptr || !aligned(p, 16)) return ATTN_EINVAL;
  const uint64_t es = dtype == ATTN_F32 ? 4 : 2;
  const uint64_t hd = static_cast<uint64_t>(n_heads) * head_dim;
  const uint64_t bytes[] = {static_cast<uint64_t>(T) * hidden * es, 3 * hd * hidden * es, 3 * hd * es,
                            static_cast<uint64_t>(hidden) * hd * es, static_cast<uint64_t>(hidden) * es,
                            static_cast<uint64_t>(T) * hidden * es};
  for (int i = 0; i < 5; ++i)
    if (overlaps(out, bytes[5], ptrs[i], bytes[i])) return ATTN_EINVAL;
  const Carve c = carve(T, n_heads, head_dim, dtype);
  if (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < c.total) return ATTN_EINVAL;
  for (int i = 0; i < 6; ++i)
    if (overlaps(workspace, c.total, ptrs[i], bytes[i])) return ATTN_EINVAL;
  char *ws = static_cast<char *>(workspace);
  char *qkv = ws;
  void *a = ws + c.qkv_bytes;
  const uint64_t block = hd * es;  // bytes of one of q, k, v within a qkv row
  // the attention's own checks (mask kind, window, scale, offsets) before any device work
  rc = attn_prefill_check(qkv, qkv + block, qkv + 2 * block, a, cu_seqlens, n_seqs, n_heads, n_heads, head_dim,
                          dtype, mask_kind, window, scale);
  if (rc != ATTN_OK) return rc;
  if (T >= (int64_t(1) << 31)) return ATTN_EUNSUPPORTED;
  const bool f32 = dtype == ATTN_F32;
  if (proj::gemm_nt_bias(x, w_qkv, b_qkv, qkv, T, static_cast<int64_t>(3 * hd), hidden, f32, stream) != 0)
    return ATTN_ELAUNCH;
  rc = attn::prefill_strided(qkv, qkv + block, qkv + 2 * block, a, nullptr, cu_seqlens, cu_seqlens, n_seqs, n_heads,
                             n_heads, head_dim, dtype, mask_kind, window, scale, static_cast<int32_t>(3 * hd),
                             static_cast<int32_t>(3 * hd), stream);
  if (rc != ATTN_OK) return rc;
  if (proj::gemm_nt_bias(a, w_o, b_o, out, T, hidden, static_cast<int64_t>(hd), f32, stream) != 0)
    return ATTN_ELAUNCH;
  return ATTN_OK;
}

}  // extern "C"
