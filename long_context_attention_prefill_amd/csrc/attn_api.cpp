// attn_api.cpp -- the library's C ABI: argument checks and work planning.
//
// Host-only code (no HIP headers): every check runs before any device work,
// so a rejected call leaves the stream and `out` untouched.  Planning splits
// the packed batch into launches of at most kMaxSeqsPerLaunch non-empty
// sequences, longest first, and hands each to a kernel family.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/attn_prefill.h"
#include "attn_launch.h"

namespace {

constexpr int kVersion = 1 * 10000 + 1 * 100 + 0;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  if (na == 0 || nb == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Checks of every entry point.  cu_q / cu_k: host int32[n_seqs + 1]; with
// cu_k == cu_q (the square case) every sequence has as many keys as queries.
int check(const void *q, const void *k, const void *v, const void *out, const float *lse,
          const int32_t *cu_q, const int32_t *cu_k, int32_t n_seqs, int32_t hq, int32_t hkv,
          int32_t d, int32_t dtype, int32_t mask, int32_t window, float scale, int64_t *Tq_out,
          int64_t *Tk_out) {
  if (n_seqs < 0) return ATTN_EINVAL;
  if (n_seqs > 0 && (cu_q == nullptr || cu_k == nullptr)) return ATTN_EINVAL;
  if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return ATTN_EINVAL;
  if (mask != ATTN_CAUSAL && mask != ATTN_FULL && mask != ATTN_WINDOW) return ATTN_EINVAL;
  if (mask == ATTN_WINDOW && window <= 0) return ATTN_EINVAL;
  if (!std::isfinite(scale)) return ATTN_EINVAL;
  int64_t Tq = 0, Tk = 0;
  if (n_seqs > 0) {
    if (cu_q[0] != 0 || cu_k[0] != 0) return ATTN_EINVAL;
    for (int32_t b = 0; b < n_seqs; ++b) {
      if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return ATTN_EINVAL;
      // the queries are the last positions of their sequence's keys
      if (static_cast<int64_t>(cu_q[b + 1]) - cu_q[b] > static_cast<int64_t>(cu_k[b + 1]) - cu_k[b])
        return ATTN_EINVAL;
    }
    Tq = cu_q[n_seqs];
    Tk = cu_k[n_seqs];
  }
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_EUNSUPPORTED;
  if (d != 64 && d != 72 && d != 128) return ATTN_EUNSUPPORTED;
  // element offsets: T * h * d must fit comfortably in 63 bits
  if (static_cast<double>(Tq) * hq * d > 9.0e18 || static_cast<double>(Tk) * hkv * d > 9.0e18)
    return ATTN_EUNSUPPORTED;
  if (Tq > 0) {
    if (!q || !k || !v || !out) return ATTN_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_EINVAL;
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_EINVAL;
    const uint64_t es = dtype == ATTN_BF16 ? 2 : 4;
    const uint64_t nq = static_cast<uint64_t>(Tq) * hq * d * es;
    const uint64_t nkv = static_cast<uint64_t>(Tk) * hkv * d * es;
    if (overlaps(out, nq, q, nq) || overlaps(out, nq, k, nkv) || overlaps(out, nq, v, nkv))
      return ATTN_EINVAL;
    if (lse != nullptr) {
      const uint64_t nl = static_cast<uint64_t>(Tq) * hq * sizeof(float);
      if (overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv) ||
          overlaps(lse, nl, out, nq))
        return ATTN_EINVAL;
    }
  }
  *Tq_out = Tq;
  *Tk_out = Tk;
  return ATTN_OK;
}

// Plan and enqueue one call (arguments already checked, Tq > 0).
int run(const void *q, const void *k, const void *v, void *out, float *lse,
        const int32_t *cu_q, const int32_t *cu_k, int32_t n_seqs, int32_t n_q_heads,
        int32_t n_kv_heads, int32_t head_dim, int32_t dtype, int32_t mask_kind, int32_t window,
        float scale, void *stream) {
  const bool bf16 = dtype == ATTN_BF16;
  const int bm = bf16 ? attn::rows_per_workgroup_bf16(head_dim)
                      : attn::rows_per_workgroup_f32(head_dim);
  auto nq = [&](int32_t b) { return cu_q[b + 1] - cu_q[b]; };

  // sequences with queries, most queries first (ties: batch order)
  std::vector<int32_t> order;
  order.reserve(n_seqs);
  for (int32_t b = 0; b < n_seqs; ++b)
    if (nq(b) > 0) order.push_back(b);
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return nq(x) > nq(y); });

  attn::LaunchArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.hq = n_q_heads;
  a.hkv = n_kv_heads;
  a.group = n_q_heads / n_kv_heads;
  a.mask_kind = mask_kind;
  a.window = mask_kind == ATTN_WINDOW ? window : 0;
  a.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);  // log2(e)
  a.bm = bm;

  // plan every launch before enqueuing any, so a rejected plan leaves no work behind
  std::vector<attn::LaunchArgs> plan;
  for (size_t base = 0; base < order.size(); base += attn::kMaxSeqsPerLaunch) {
    const size_t cnt = std::min(order.size() - base, static_cast<size_t>(attn::kMaxSeqsPerLaunch));
    int64_t items = 0;
    a.n_seqs = static_cast<int32_t>(cnt);
    for (size_t i = 0; i < cnt; ++i) {
      const int32_t b = order[base + i];
      a.q_start[i] = cu_q[b];
      a.q_len[i] = nq(b);
      a.k_start[i] = cu_k[b];
      a.k_len[i] = cu_k[b + 1] - cu_k[b];
      a.seq_tiles[i] = (a.q_len[i] + bm - 1) / bm;
      items += static_cast<int64_t>(a.seq_tiles[i]) * n_q_heads;
    }
    if (items > INT32_MAX) return ATTN_EUNSUPPORTED;
    a.total_items = static_cast<int32_t>(items);
    // causal item order: levels [seq_tiles[k], seq_tiles[k-1]) of the k longest
    // sequences follow each other, longest level first
    int64_t start = 0;
    for (size_t k = 1; k <= cnt; ++k) {
      a.level_start[k - 1] = static_cast<int32_t>(start);
      const int32_t below = k < cnt ? a.seq_tiles[k] : 0;
      start += static_cast<int64_t>(a.seq_tiles[k - 1] - below) * static_cast<int64_t>(k) * n_q_heads;
    }
    a.level_start[cnt] = static_cast<int32_t>(start);  // == total_items
    plan.push_back(a);
  }
  for (const attn::LaunchArgs &la : plan) {
    const int err = bf16 ? attn::launch_bf16(la, head_dim, stream)
                         : attn::launch_f32(la, head_dim, stream);
    if (err != 0) return ATTN_ELAUNCH;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_prefill_check(const void *q, const void *k, const void *v, const void *out,
                       const int32_t *cu_seqlens, int32_t n_seqs, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                       int32_t mask_kind, int32_t window, float scale) {
  int64_t Tq = 0, Tk = 0;
  return check(q, k, v, out, nullptr, cu_seqlens, cu_seqlens, n_seqs, n_q_heads, n_kv_heads,
               head_dim, dtype, mask_kind, window, scale, &Tq, &Tk);
}

int attn_prefill(const void *q, const void *k, const void *v, void *out,
                 const int32_t *cu_seqlens, int32_t n_seqs, int32_t n_q_heads,
                 int32_t n_kv_heads, int32_t head_dim, int32_t dtype, int32_t mask_kind,
                 int32_t window, float scale, void *stream) {
  int64_t Tq = 0, Tk = 0;
  int rc = check(q, k, v, out, nullptr, cu_seqlens, cu_seqlens, n_seqs, n_q_heads, n_kv_heads,
                 head_dim, dtype, mask_kind, window, scale, &Tq, &Tk);
  if (rc != ATTN_OK || Tq == 0) return rc;
  return run(q, k, v, out, nullptr, cu_seqlens, cu_seqlens, n_seqs, n_q_heads, n_kv_heads,
             head_dim, dtype, mask_kind, window, scale, stream);
}

int attn_prefill_kv_check(const void *q, const void *k, const void *v, const void *out,
                          const float *lse, const int32_t *cu_seqlens_q,
                          const int32_t *cu_seqlens_k, int32_t n_seqs, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                          int32_t mask_kind, int32_t window, float scale) {
  int64_t Tq = 0, Tk = 0;
  return check(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads,
               head_dim, dtype, mask_kind, window, scale, &Tq, &Tk);
}

int attn_prefill_kv(const void *q, const void *k, const void *v, void *out, float *lse,
                    const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t n_seqs,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                    int32_t mask_kind, int32_t window, float scale, void *stream) {
  int64_t Tq = 0, Tk = 0;
  int rc = check(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads,
                 head_dim, dtype, mask_kind, window, scale, &Tq, &Tk);
  if (rc != ATTN_OK || Tq == 0) return rc;
  return run(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads,
             head_dim, dtype, mask_kind, window, scale, stream);
}

const char *attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported head_dim, dtype or size";
    case ATTN_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int attn_version(void) { return kVersion; }

}  // extern "C"
