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

#include "attn_prefill.h"
#include "attn_launch.h"

namespace {

constexpr int kVersion = 1 * 10000 + 2 * 100 + 0;

static_assert(ATTN_DECODE_SCRATCH_BYTES == attn::kDecodeScratchBytes, "one scratch size");

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  if (na == 0 || nb == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Checks of every entry point that involve no pointer.  cu_q / cu_k: host
// int32[n_seqs + 1]; with cu_k == cu_q (the square case) every sequence has as
// many keys as queries.
int check_shape(const int32_t *cu_q, const int32_t *cu_k, int32_t n_seqs, int32_t hq, int32_t hkv,
                int32_t d, int32_t dtype, int32_t mask, int32_t window, float scale,
                int64_t *Tq_out, int64_t *Tk_out) {
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
  *Tq_out = Tq;
  *Tk_out = Tk;
  return ATTN_OK;
}

// Every check of an entry point: the shape, then the buffers.
int check(const void *q, const void *k, const void *v, const void *out, const float *lse,
          const int32_t *cu_q, const int32_t *cu_k, int32_t n_seqs, int32_t hq, int32_t hkv,
          int32_t d, int32_t dtype, int32_t mask, int32_t window, float scale, int64_t *Tq_out,
          int64_t *Tk_out) {
  int64_t Tq = 0, Tk = 0;
  const int rc = check_shape(cu_q, cu_k, n_seqs, hq, hkv, d, dtype, mask, window, scale, &Tq, &Tk);
  if (rc != ATTN_OK) return rc;
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
        float scale, void *stream, int32_t q_stride = 0, int32_t kv_stride = 0) {
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
  a.q_stride = q_stride > 0 ? q_stride : n_q_heads * head_dim;
  a.kv_stride = kv_stride > 0 ? kv_stride : n_kv_heads * head_dim;
  a.group = n_q_heads / n_kv_heads;
  a.mask_kind = mask_kind;
  a.window = mask_kind == ATTN_WINDOW ? window : 0;
  a.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);  // log2(e)

  // plan every launch before enqueuing any, so a rejected plan leaves no work behind
  std::vector<attn::LaunchArgs> plan;
  for (size_t base = 0; base < order.size(); base += attn::kMaxSeqsPerLaunch) {
    const size_t cnt = std::min(order.size() - base, static_cast<size_t>(attn::kMaxSeqsPerLaunch));
    // bf16 launches of few items take key halves: half-height items whose two
    // pairs of waves sweep the two halves of the keys (twice the workgroups).
    // That pays when the items leave CUs idle, or when they are unequal (the
    // longest item sets the time: causal tiles over a short prefix); equal
    // items that already fill the CUs run as fast on whole rows.
    int64_t items = 0, key_sum = 0, key_max = 0, max_keys = 0;
    for (size_t i = 0; i < cnt; ++i) {
      const int32_t b = order[base + i];
      items += static_cast<int64_t>((nq(b) + bm - 1) / bm) * n_q_heads;
      max_keys = std::max<int64_t>(max_keys, cu_k[b + 1] - cu_k[b]);
    }
    if (bf16 && items <= attn::kKeyHalvesMaxItems) {
      for (size_t i = 0; i < cnt; ++i) {
        const int32_t b = order[base + i];
        const int64_t n_q = nq(b), n_k = cu_k[b + 1] - cu_k[b], offk = n_k - n_q;
        for (int64_t q0 = 0; q0 < n_q; q0 += bm) {
          const int64_t q1 = std::min<int64_t>(q0 + bm, n_q) - 1 + offk;  // last row's position
          int64_t lo = 0, hi = n_k;  // keys of the tile's rows
          if (mask_kind == ATTN_CAUSAL) {
            hi = q1 + 1;
          } else if (mask_kind == ATTN_WINDOW) {
            lo = ((q0 + offk) / window) * window;
            hi = std::min<int64_t>((q1 / window) * window + window, n_k);
          }
          key_sum += hi - lo;
          key_max = std::max(key_max, hi - lo);
        }
      }
    }
    const bool few = items <= attn::kKeyHalvesFewItems;
    const bool unequal = items <= attn::kKeyHalvesMaxItems && 2 * key_max * items >= 3 * key_sum * n_q_heads;
    // (the kernel's buffer offsets into one head's keys stay below 2^31 bytes)
    const bool halves = bf16 && (few || unequal) && max_keys * a.kv_stride * 2 < (int64_t{1} << 30);
    const int bm_l = halves ? attn::rows_per_workgroup_bf16_halves(head_dim) : bm;
    a.bm = bm_l;
    a.key_halves = halves ? 1 : 0;
    items = 0;
    a.n_seqs = static_cast<int32_t>(cnt);
    for (size_t i = 0; i < cnt; ++i) {
      const int32_t b = order[base + i];
      a.q_start[i] = cu_q[b];
      a.q_len[i] = nq(b);
      a.k_start[i] = cu_k[b];
      a.k_len[i] = cu_k[b + 1] - cu_k[b];
      a.seq_tiles[i] = (a.q_len[i] + bm_l - 1) / bm_l;
      items += static_cast<int64_t>(a.seq_tiles[i]) * n_q_heads;
    }
    if (items > INT32_MAX) return ATTN_EUNSUPPORTED;
    a.total_items = static_cast<int32_t>(items);
    // window launches whose windows span at most two query tiles: whole runs
    // of 16 query tiles (two per XCD) in the XCD-blocked order, so a window's
    // keys and values reach one XCD's L2 once for every head
    a.xcd_tiles = mask_kind == ATTN_WINDOW && window <= 2 * bm_l
                      ? static_cast<int32_t>(((items / n_q_heads) / 16) * 16)
                      : 0;
    // causal item order: levels [seq_tiles[k], seq_tiles[k-1]) of the k longest
    // sequences follow each other, longest level first
    int64_t start = 0;
    for (size_t k = 1; k <= cnt; ++k) {
      a.level_start[k - 1] = static_cast<int32_t>(start);
      const int32_t below = k < cnt ? a.seq_tiles[k] : 0;
      start += static_cast<int64_t>(a.seq_tiles[k - 1] - below) * static_cast<int64_t>(k) * n_q_heads;
    }
    a.level_start[cnt] = static_cast<int32_t>(start);  // == total_items
    a.tickets = nullptr;
    a.ticket_from = a.total_items;
    if (bf16 && attn::work_tickets(a, stream) != 0) return ATTN_ELAUNCH;
    plan.push_back(a);
  }
  for (const attn::LaunchArgs &la : plan) {
    const int err = bf16 ? attn::launch_bf16(la, head_dim, stream)
                         : attn::launch_f32(la, head_dim, stream);
    if (err != 0) return ATTN_ELAUNCH;
  }
  return ATTN_OK;
}

// ---------------------------------------------------------------- decode

// The bf16 decode kernels cover head_dim 64 and 128; other requests run
// through the prefill path as one query per sequence.
bool decode_fast(int32_t dtype, int32_t d) { return dtype == ATTN_BF16 && (d == 64 || d == 128); }

// Workers to aim for: 256 CUs x 4 waves, twice over, so chunks stay short
// enough to spread a small batch over the whole GPU; but no chunk shorter
// than kDecodeMinTiles tiles, whose per-chunk costs (query load, partial
// store, merge) would outweigh the keys they cover (measured: 2 tiles beat
// 4 by 10 % at batch 8 over 10k-token caches; 1 tile gains nothing more).
constexpr int64_t kDecodeTargetItems = 2048;
constexpr int64_t kDecodeMinTiles = 2;

struct DecodePlan {
  int32_t chunk = attn::kDecodeTile;
  int64_t total_items = 0;
  bool direct = true;
  int32_t rows = 0, head_blocks = 0;
};

// Visible keys of the newest token of a sequence of n keys: [lo, n).
int64_t decode_lo(int32_t mask, int32_t window, int64_t n) {
  return mask == ATTN_WINDOW ? ((n - 1) / window) * window : 0;
}

DecodePlan plan_decode(const int32_t *cu_k, int32_t n_seqs, int32_t hq, int32_t hkv,
                       int32_t mask, int32_t window) {
  DecodePlan p;
  const int32_t group = hq / hkv;
  p.head_blocks = (group + 31) / 32;
  p.rows = group < 32 ? group : 32;
  int64_t tiles = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t n = cu_k[b + 1] - cu_k[b];
    const int64_t vis = n - decode_lo(mask, window, n);
    tiles += (vis + attn::kDecodeTile - 1) / attn::kDecodeTile;
  }
  tiles *= static_cast<int64_t>(hkv) * p.head_blocks;
  const int64_t per = (tiles + kDecodeTargetItems - 1) / kDecodeTargetItems;
  p.chunk = static_cast<int32_t>(std::max<int64_t>(kDecodeMinTiles, std::min<int64_t>(per, 1 << 20)) *
                                 attn::kDecodeTile);
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t n = cu_k[b + 1] - cu_k[b];
    const int64_t vis = n - decode_lo(mask, window, n);
    const int64_t splits = (vis + p.chunk - 1) / p.chunk;
    if (splits > 1) p.direct = false;
    p.total_items += splits * hkv * p.head_blocks;
  }
  return p;
}

uint64_t decode_workspace_bytes(const DecodePlan &p, int32_t d) {
  if (p.direct) return 0;
  return static_cast<uint64_t>(p.total_items) * p.rows * (static_cast<uint64_t>(d) + 2) * sizeof(float);
}

// Decode takes one query (the newest token) per sequence, so every sequence
// must hold at least one key; cu_q receives the queries' packing 0, 1, ..., n.
int check_decode_shape(const int32_t *cu_k, int32_t n_seqs, int32_t hq, int32_t hkv, int32_t d,
                       int32_t dtype, int32_t mask, int32_t window, float scale,
                       std::vector<int32_t> *cu_q) {
  if (n_seqs < 0 || (n_seqs > 0 && cu_k == nullptr)) return ATTN_EINVAL;
  for (int32_t b = 0; b < n_seqs; ++b)
    if (cu_k[b + 1] <= cu_k[b]) return ATTN_EINVAL;  // an empty cache has no newest token
  cu_q->resize(static_cast<size_t>(n_seqs) + 1);
  for (int32_t b = 0; b <= n_seqs; ++b) (*cu_q)[b] = b;
  int64_t Tq = 0, Tk = 0;
  return check_shape(cu_q->data(), cu_k, n_seqs, hq, hkv, d, dtype, mask, window, scale, &Tq, &Tk);
}

int check_decode(const void *q, const void *k, const void *v, const void *out, const float *lse,
                 const int32_t *cu_k, int32_t n_seqs, int32_t hq, int32_t hkv, int32_t d,
                 int32_t dtype, int32_t mask, int32_t window, float scale,
                 std::vector<int32_t> *cu_q) {
  const int rc = check_decode_shape(cu_k, n_seqs, hq, hkv, d, dtype, mask, window, scale, cu_q);
  if (rc != ATTN_OK) return rc;
  int64_t Tq = 0, Tk = 0;
  return check(q, k, v, out, lse, cu_q->data(), cu_k, n_seqs, hq, hkv, d, dtype, mask, window,
               scale, &Tq, &Tk);
}

// Workspace bytes of a checked decode shape: the largest over its launches.
uint64_t decode_need(const int32_t *cu_seqlens_k, int32_t n_seqs, int32_t n_q_heads,
                     int32_t n_kv_heads, int32_t head_dim, int32_t dtype, int32_t mask_kind,
                     int32_t window) {
  if (n_seqs == 0 || !decode_fast(dtype, head_dim)) return 0;
  uint64_t total = 0;
  for (int32_t base = 0; base < n_seqs; base += attn::kMaxDecodeSeqsPerLaunch) {
    const int32_t cnt = std::min(n_seqs - base, attn::kMaxDecodeSeqsPerLaunch);
    std::vector<int32_t> cu(cnt + 1);
    for (int32_t i = 0; i <= cnt; ++i) cu[i] = cu_seqlens_k[base + i] - cu_seqlens_k[base];
    const DecodePlan p = plan_decode(cu.data(), cnt, n_q_heads, n_kv_heads, mask_kind, window);
    total = std::max(total, decode_workspace_bytes(p, head_dim));
  }
  return total;
}

}  // namespace

namespace attn {

int prefill_strided(const void *q, const void *k, const void *v, void *out, float *lse,
                    const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t n_seqs,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                    int32_t mask_kind, int32_t window, float scale, int32_t q_stride,
                    int32_t kv_stride, void *stream) {
  if (q_stride < n_q_heads * head_dim || kv_stride < n_kv_heads * head_dim || q_stride % 8 != 0 ||
      kv_stride % 8 != 0)
    return ATTN_EINVAL;
  if (n_seqs == 0 || cu_seqlens_q[n_seqs] == 0) return ATTN_OK;
  return run(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads, head_dim, dtype,
             mask_kind, window, scale, stream, q_stride, kv_stride);
}

}  // namespace attn

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

int attn_decode_workspace_size(const int32_t *cu_seqlens_k, int32_t n_seqs, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                               int32_t mask_kind, int32_t window, uint64_t *bytes) {
  if (bytes == nullptr) return ATTN_EINVAL;
  std::vector<int32_t> cu_q;
  const int rc = check_decode_shape(cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads, head_dim, dtype,
                                    mask_kind, window, 1.0f, &cu_q);
  if (rc != ATTN_OK) return rc;
  *bytes = decode_need(cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads, head_dim, dtype, mask_kind,
                       window);
  return ATTN_OK;
}

int attn_decode(const void *q, const void *k, const void *v, void *out, float *lse,
                const int32_t *cu_seqlens_k, int32_t n_seqs, int32_t n_q_heads,
                int32_t n_kv_heads, int32_t head_dim, int32_t dtype, int32_t mask_kind,
                int32_t window, float scale, void *workspace, uint64_t workspace_bytes,
                void *stream) {
  std::vector<int32_t> cu_q;
  int rc = check_decode(q, k, v, out, lse, cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads, head_dim,
                        dtype, mask_kind, window, scale, &cu_q);
  if (rc != ATTN_OK || n_seqs == 0) return rc;
  if (!decode_fast(dtype, head_dim))
    return run(q, k, v, out, lse, cu_q.data(), cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads,
               head_dim, dtype, mask_kind, window, scale, stream);
  // plan every launch (at most kMaxDecodeSeqsPerLaunch sequences each; they
  // run one after another on the stream and reuse the workspace) before any
  std::vector<attn::DecodeArgs> plan;
  const size_t es = 2;
  for (int32_t base = 0; base < n_seqs; base += attn::kMaxDecodeSeqsPerLaunch) {
    const int32_t cnt = std::min(n_seqs - base, attn::kMaxDecodeSeqsPerLaunch);
    std::vector<int32_t> cu(cnt + 1);
    for (int32_t i = 0; i <= cnt; ++i) cu[i] = cu_seqlens_k[base + i] - cu_seqlens_k[base];
    const DecodePlan p = plan_decode(cu.data(), cnt, n_q_heads, n_kv_heads, mask_kind, window);
    if (p.total_items > INT32_MAX) return ATTN_EUNSUPPORTED;
    const uint64_t need = decode_workspace_bytes(p, head_dim);
    if (need > 0) {
      if (workspace == nullptr || workspace_bytes < need ||
          (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
        return ATTN_EINVAL;
      const uint64_t nq = static_cast<uint64_t>(n_seqs) * n_q_heads * head_dim * es;
      const uint64_t nkv = static_cast<uint64_t>(cu_seqlens_k[n_seqs]) * n_kv_heads * head_dim * es;
      const uint64_t nl = static_cast<uint64_t>(n_seqs) * n_q_heads * sizeof(float);
      if (overlaps(workspace, need, q, nq) || overlaps(workspace, need, k, nkv) ||
          overlaps(workspace, need, v, nkv) || overlaps(workspace, need, out, nq) ||
          (lse != nullptr && overlaps(workspace, need, lse, nl)))
        return ATTN_EINVAL;
    }
    attn::DecodeArgs a{};
    const size_t qrow = static_cast<size_t>(n_q_heads) * head_dim * es;
    a.q = static_cast<const char *>(q) + static_cast<size_t>(base) * qrow;
    a.k = k;
    a.v = v;
    a.out = static_cast<char *>(out) + static_cast<size_t>(base) * qrow;
    a.lse = lse == nullptr ? nullptr : lse + static_cast<size_t>(base) * n_q_heads;
    // partial outputs first (16-byte rows), then the references and sums
    a.ws_o = p.direct ? nullptr : static_cast<float *>(workspace);
    a.ws_ml = p.direct ? nullptr
                       : static_cast<float *>(workspace) +
                             static_cast<size_t>(p.total_items) * p.rows * head_dim;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.group = n_q_heads / n_kv_heads;
    a.head_blocks = p.head_blocks;
    a.rows = p.rows;
    a.chunk = p.chunk;
    a.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);  // log2(e)
    a.n_seqs = cnt;
    a.total_items = static_cast<int32_t>(p.total_items);
    a.direct = p.direct ? 1 : 0;
    int64_t item = 0;
    for (int32_t i = 0; i < cnt; ++i) {
      const int32_t b = base + i;
      const int64_t n = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
      const int64_t lo = decode_lo(mask_kind, window, n);
      a.k_begin[i] = static_cast<int32_t>(cu_seqlens_k[b] + lo);
      a.k_count[i] = static_cast<int32_t>(n - lo);
      a.splits[i] = static_cast<int32_t>((n - lo + p.chunk - 1) / p.chunk);
      a.item_start[i] = static_cast<int32_t>(item);
      item += static_cast<int64_t>(a.splits[i]) * n_kv_heads * p.head_blocks;
    }
    a.item_start[cnt] = static_cast<int32_t>(item);
    plan.push_back(a);
  }
  for (const attn::DecodeArgs &a : plan)
    if (attn::launch_decode_bf16(a, head_dim, stream) != 0) return ATTN_ELAUNCH;
  return ATTN_OK;
}

int attn_decode_noalloc(const void *q, const void *k, const void *v, void *out, float *lse,
                        const int32_t *cu_seqlens_k, int32_t n_seqs, int32_t n_q_heads,
                        int32_t n_kv_heads, int32_t head_dim, int32_t dtype, int32_t mask_kind,
                        int32_t window, float scale, void *stream) {
  std::vector<int32_t> cu_q;
  const int rc = check_decode(q, k, v, out, lse, cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads,
                              head_dim, dtype, mask_kind, window, scale, &cu_q);
  if (rc != ATTN_OK || n_seqs == 0) return rc;
  const uint64_t need = decode_need(cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads, head_dim, dtype,
                                    mask_kind, window);
  if (need > attn::kDecodeScratchBytes) return ATTN_EUNSUPPORTED;
  void *scratch = nullptr;
  if (need > 0 && attn::decode_scratch(stream, &scratch) != 0) return ATTN_ELAUNCH;
  return attn_decode(q, k, v, out, lse, cu_seqlens_k, n_seqs, n_q_heads, n_kv_heads, head_dim,
                     dtype, mask_kind, window, scale, scratch,
                     need > 0 ? attn::kDecodeScratchBytes : 0, stream);
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
