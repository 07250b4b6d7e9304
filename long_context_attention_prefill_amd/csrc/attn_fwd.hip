// attn_fwd.hip -- fused exact attention-prefill kernels for gfx950 (MI355X).
//
// One pass per (sequence, query head, tile of query rows): K and V tiles are
// streamed through LDS, scores live only in registers, and an online softmax
// carries the running maximum and sum, so the N x N score matrix never
// touches memory.  This replaces the per-head GEMMs into an N x N score
// buffer that the paper "A Modern Multimodal Assistant on a 6 GB 2011 GPU"
// uses on Fermi (abstract, result (iii); gist.science technical summary,
// Metodologia, attention rewrite); the result is the same exact attention.
//
// bf16 family: QK^T and PV on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// Scores are computed transposed, S^T = K Q^T, so each lane owns one query
// column and 16 keys of each 32x32 block: the row max and row sum are mostly
// in-lane, and the probabilities already sit in the B-operand layout of
// O^T = V^T P^T, whose V^T operand comes from LDS through transposing reads.
// head_dim 72 runs five 16-wide k steps (the last half over zero padding in
// LDS) and three 32-row blocks of O^T (rows past 72 are dropped).
//
// fp32 family: v_mfma_f32_32x32x2_f32 (exact fp32 products, fp32 sums), the
// scores kept in registers as the B operand of the PV product, V transposed
// in LDS.
//
// A sequence holds nq queries and nk >= nq keys; its queries are the last nq
// positions, so local query row r sits at position i = r + (nk - nq) (equal
// counts: i = r).  Visible keys of position i form one interval
// [lo(i), hi(i)) for all three masks, computed with integers only:
//   causal [0, i+1)   full [0, nk)  window [W*floor(i/W), min(W*floor(i/W)+W, nk))
// lo and hi never decrease with i, so a tile of rows sees the union
// [lo(first), hi(last)) and every row sees the intersection
// [lo(last), hi(first)); only key tiles not inside the intersection are
// masked element by element, and tiles outside the union are never loaded.
// With lse requested, each row also stores ln(sum_j exp(scale * s_j)) =
// (m + log2(l)) * ln 2 from its exp2-unit reference m and sum l.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <set>
#include <type_traits>
#include <utility>
#include <vector>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {



struct Item {
  int seq;
  int tile;
  int head;
};

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time
// (for builtins whose operands must be constants).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Workgroup r -> (sequence, query tile, query head), heaviest work first.
// Causal: tile m costs ~(m+1) key tiles in every sequence, so items are
// ordered by m descending across the batch, the sequences holding a level in
// length order; the levels where the k longest sequences are active form one
// segment, starting at item level_start[k-1], so the decode scans segments
// (at most one per sequence), not levels.  Otherwise items go by sequence
// length (sequences arrive longest first).  The hq heads of one (sequence,
// tile) are consecutive, and when hq is a multiple of 8 slot s maps to head
// (s % 8) * (hq / 8) + s / 8: consecutive workgroups land on different XCDs
// round-robin, so each XCD keeps to a contiguous block of query heads, i.e.
// to few key/value heads, and their K/V stays in that XCD's L2.
__device__ __forceinline__ Item decode_item(const LaunchArgs &a, int r) {
  Item it{0, 0, 0};
  int slot = 0;
  if (a.mask_kind == kCausal) {
    int k = 1;  // segment: the k longest sequences are active
    while (k < a.n_seqs && a.level_start[k] <= r) ++k;
    const int rel = r - a.level_start[k - 1];
    const int per_level = k * a.hq;
    const int lvl = rel / per_level;
    const int rem = rel - lvl * per_level;
    it.tile = a.seq_tiles[k - 1] - 1 - lvl;
    it.seq = rem / a.hq;
    slot = rem - it.seq * a.hq;
  } else {
    // Full and window launches.  Workgroup r runs on XCD r mod 8; with
    // a.xcd_tiles set (windows of at most two query tiles) the first
    // a.xcd_tiles query tiles (in sequence order) go to the XCDs in runs of
    // two consecutive tiles, all heads of a run back to back on one XCD, so
    // the keys and values of a window reach that XCD's L2 once for all its
    // heads (in the plain order each XCD holds a block of query heads for
    // every tile, and each key/value head is fetched by every XCD holding
    // one of its query heads).  Tiles past them keep the plain order.
    int g = 0;  // tile index over the launch's sequences
    if (r < a.xcd_tiles * a.hq) {
      const int x = r & 7, q = r >> 3;
      const int run = q / (2 * a.hq), in_run = q - run * 2 * a.hq;
      g = run * 16 + 2 * x + in_run / a.hq;
      slot = in_run - (in_run / a.hq) * a.hq;
    } else {
      g = r / a.hq;
      slot = r - g * a.hq;
    }
    for (int b = 0; b < a.n_seqs; ++b) {
      if (g < a.seq_tiles[b]) {
        it.seq = b;
        it.tile = g;
        break;
      }
      g -= a.seq_tiles[b];
    }
  }
  it.head = (a.hq % 8 == 0) ? (slot & 7) * (a.hq >> 3) + (slot >> 3) : slot;
  return it;
}

// Visible keys [lo, hi) of the query at position i of a sequence of n keys.
__device__ __forceinline__ void row_range(int mask, int W, int i, int n, int &lo, int &hi) {
  if (mask == kCausal) {
    lo = 0;
    hi = i + 1;
  } else if (mask == kFull) {
    lo = 0;
    hi = n;
  } else {
    lo = (i / W) * W;
    hi = min(lo + W, n);
  }
}


// ---------------------------------------------------------------------------
// bf16 / MFMA family, head_dim 64, 72 and 128.  K and V reach LDS by direct
// buffer->LDS loads: no staging registers, and rows past the key range read
// as zeros (buffer range check).  Inside each 16-key MFMA step keys are
// taken in the permuted order of attn_device.h.  head_dim 64 and 72 use its
// padded layout (one 16-byte pad slot per key row); head_dim 128 stores key
// rows unpadded, 256 bytes each, with chunk c of key k at slot c ^ (k mod 16):
// 16 keys read by 16 lanes (K, 16-byte reads) start at 16 distinct slots,
// and the 4 keys x 64 bytes of a V transposing read fill 4 distinct quarters
// of the 256-byte bank window, so both are free of bank conflicts, while
// every 64-lane load carries 1 KB of key data (the padded layout spent 4 of
// its 20 loads per head-dim-128 tile on padding and out-of-range spill).
// ---------------------------------------------------------------------------

// Each wave owns R consecutive 32-row query sub-blocks (the workgroup covers
// NW * 32 * R rows); every K or V fragment read from LDS feeds the R
// sub-blocks' MFMAs back to back.  R = 1 runs two workgroups per CU (two waves
// per SIMD, up to 256 registers each) and is the instance dispatched.  R = 2
// (one wave per SIMD, up to 512 registers) halves the LDS reads and K/V tile
// loads per MFMA, but with no second wave to hide latency and its scores
// spilling into AGPRs it measured ~30 % slower on gfx950, so it is not
// instantiated.  BN is the key tile: 64 keys, or at head_dim 128 32 keys,
// which halves the LDS buffers (32 KB per workgroup) and the scores' and
// probabilities' registers (168 VGPRs), so three workgroups fit on a CU
// (three waves per SIMD).
//
// SPLIT (key halves, for launches too small to fill the GPU): a workgroup
// covers 64 query rows, and its waves split the keys instead of the rows --
// waves 0 and 1 (rows 0-31, 32-63) sweep the first half of the key tiles,
// waves 2 and 3 (the same rows) the second half, in step: each LDS tile holds
// BN = 32 keys of each half (one 64-key tile's space), and every wave computes
// on its own half's 32 keys.  At the end waves 2 and 3 hand their rows'
// references, sums and unnormalised outputs to waves 0 and 1 through LDS,
// which fold them in (the merge of two softmax partitions) and store.  Twice
// the workgroups of the plain split by rows, each half as long.
template <int D, int NW, int R, int BN, bool SPLIT, bool SHIFT>
__global__ __launch_bounds__(NW * 64, BN == 32 && !SPLIT ? 3 : 2 / R) void fwd_bf16_fast(const LaunchArgs a) {
  // The host pass only needs this kernel's signature for its launch stub;
  // the body (gfx950-only builtins) is compiled for the device alone.
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(D == 64 || D == 72 || D == 128, "fast path covers head_dim 64, 72 and 128");
  static_assert(R == 1 || R == 2, "one or two query sub-blocks per wave");
  using L = FastLayout<D>;
  static_assert(BN == 64 || (BN == 32 && R == 1 && (D == 128 || SPLIT)),
                "64-key tiles, or 32-key tiles at head_dim 128 or with key halves");
  static_assert(!SPLIT || (BN == 32 && R == 1 && NW == 4), "key halves: four waves, 32-key steps");
  constexpr int HALVES = SPLIT ? 2 : 1;
  constexpr int BM = NW * 32 * R / HALVES;  // query rows per workgroup
  constexpr int NB = BN / 32;  // 32-key blocks of S^T per wave and tile
  constexpr int CH = L::CH;
  constexpr int KST = L::KST;         // MFMA k steps of S^T (the last one zero-padded when D = 72)
  constexpr int DB = (D + 31) / 32;  // 32-row blocks of O^T (rows past D are computed and dropped)
  // head_dim 128: unpadded 256-byte key rows whose 16-byte chunk c sits at
  // slot c ^ (key mod 16) (the XOR layout); 64 and 72: the padded layout
  constexpr bool XOR = D == 128;
  // SHIFT (scales |c| <= kPrescaleMaxC): the query fragments hold c q rounded
  // to bf16, so S^T leaves the MFMAs in exp2 units, and plain steps start
  // S^T from -m (one register block per sub-block, fixed for the sweep)
  // instead of subtracting m per score: one VALU op fewer per score.  The
  // extra rounding perturbs each score by about |c| 2^-9 |q . k| (relative
  // 2^-9 per query element), which is why larger scales keep exact queries
  // and the per-score FMA; so does the 32-key instance at three workgroups
  // per CU, which has no registers to spare.
  static_assert(!SHIFT || !(BN == 32 && !SPLIT), "no shifted start on the 32-key, three-workgroup instance");
  constexpr int ROWB = XOR ? D * 2 : L::ROWB;  // bytes per key row in LDS
  constexpr int KBUF = HALVES * BN * ROWB;  // bytes per K (or V) LDS tile (both halves)
  // A tile is NLOADS wave-wide direct loads (64 lanes x 16 bytes); wave w
  // issues NL of them, into the consecutive 1 KB slots NL w .. NL w + NL - 1,
  // and slots past the tile (when NW does not divide NLOADS) take loads with
  // every lane out of range that nothing reads, so the issue code has no
  // branches.
  constexpr int NLOADS = KBUF / 1024;
  constexpr int NL = (NLOADS + NW - 1) / NW;
  constexpr int BUF_BYTES = NL * NW * 1024;  // one LDS buffer
  static_assert(NLOADS * 1024 == KBUF, "a tile is a whole number of wave-wide loads");

  // One array per buffer half: the compiler can then tell that a direct
  // load into one half does not feed reads of the other, and does not make
  // those reads wait for the load.
  __shared__ __attribute__((aligned(1024))) char k_lds0[BUF_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[BUF_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[BUF_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[BUF_BYTES];
  auto k_buf = [](auto tag) -> char * {
    if constexpr (decltype(tag)::value == 0) return k_lds0; else return k_lds1;
  };
  auto v_buf = [](auto tag) -> char * {
    if constexpr (decltype(tag)::value == 0) return v_lds0; else return v_lds1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < NW);
  const int half = SPLIT ? wave >> 1 : 0;  // key half this wave sweeps
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // Item of this workgroup: its own index, or with work tickets (past the
  // first wave) the next unclaimed item.
  int item = blockIdx.x;
  if (a.tickets != nullptr && item >= a.ticket_from) {
    __shared__ int ticket;
    if (tid == 0) ticket = a.ticket_from + atomicAdd(&a.tickets[0], 1);
    __syncthreads();
    item = ticket;
  }
  // a ticket past the last item (counters not at zero, which a launch that
  // ran to completion never leaves) claims no work
  const bool has_item = item < a.total_items;
  if (!has_item) item = 0;
  const Item it = decode_item(a, item);
  const int s0q = a.q_start[it.seq], s0k = a.k_start[it.seq];
  // queries are the last nq of nk positions: local row i sits at i + off
  const int nq = a.q_len[it.seq], nk = a.k_len[it.seq], off = nk - nq;
  const int h = it.head;
  const int hk = h / a.group;
  const int mask = a.mask_kind;
  const int W = a.window;
  // scale 0 (uniform weights) runs as the smallest normal positive c: every
  // exp2(c*s) is then 1 in fp32 for |s| < 2^100, and masking by -inf works
  const float c = a.c == 0.0f ? 0x1p-126f : a.c;
  const bool neg = c < 0.0f;
  const float cabs = neg ? -c : c;

  const int q0 = it.tile * BM;
  const int qend = min(q0 + BM, nq);
  int kv_lo, kv_hi, tmp;
  row_range(mask, W, q0 + off, nk, kv_lo, tmp);
  row_range(mask, W, qend - 1 + off, nk, tmp, kv_hi);
  if (!has_item) kv_hi = kv_lo;  // no tiles

  // The wave's rows [wq0, wq0 + 32R): the union of their visible keys is
  // [w_lo, w_hi), the intersection [i_lo, i_hi).
  const int wq0 = q0 + (SPLIT ? 32 * (wave & 1) : wave * 32 * R);
  const bool wave_active = has_item && wq0 < nq;
  int w_lo = 0, w_hi = 0, i_lo = 0, i_hi = 0;
  if (wave_active) {
    const int wq1 = min(wq0 + 32 * R, nq);
    row_range(mask, W, wq0 + off, nk, w_lo, i_hi);
    row_range(mask, W, wq1 - 1 + off, nk, i_lo, w_hi);
  }
  // Sub-block r: this lane's query row wq0 + 32r + l32.
  int row[R], lo_r[R], hi_r[R];
  bool row_ok[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row[r] = wq0 + 32 * r + l32;
    row_ok[r] = row[r] < nq;
    lo_r[r] = 0;
    hi_r[r] = 0;
    if (row_ok[r]) row_range(mask, W, row[r] + off, nk, lo_r[r], hi_r[r]);
  }

  // Q fragments (B operand of S^T = K Q^T): lane (l32, g) of sub-block r
  // holds q[row[r]][16*kk + 8*g .. +7] (with SHIFT scaled by c and rounded to
  // bf16, so S^T comes out of the MFMAs in exp2 units).
  bf16x8 qf[R][KST];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const __bf16 *qrow = reinterpret_cast<const __bf16 *>(a.q) +
                         (size_t)(s0q + (row_ok[r] ? row[r] : 0)) * a.q_stride + (size_t)h * D;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      qf[r][kk] = row_ok[r] && 16 * kk + 8 * g < D ? *reinterpret_cast<const bf16x8 *>(qrow + 16 * kk + 8 * g)
                                                   : (bf16x8)((__bf16)0.0f);
      if constexpr (SHIFT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[r][kk][e] = (__bf16)((float)qf[r][kk][e] * c);
      }
    }
  }

  // Direct loads: wave-wide load j fills LDS slots 64j .. 64j+63 of a tile;
  // wave w's i-th load is load j = NL w + i.
  // Padded layout: slot p is row p / SLOTS, chunk p % SLOTS (chunks >= CH are
  // padding).  XOR layout: load j fills keys 4j .. 4j+3, lane l writing key
  // 4j + (l >> 4), slot l & 15, which holds chunk (l & 15) ^ (key & 15).
  // Key halves: LDS rows BN .. 2BN-1 hold the second half's tile, ntiles
  // tiles after the first half's, so their loads reach (ntiles - 1) BN rows
  // further than their LDS row.
  const int rowbytes = a.kv_stride * 2;  // bytes between consecutive tokens of one head
  const int n_key_tiles = (kv_hi - kv_lo + BN - 1) / BN;
  const int ntiles = SPLIT ? (n_key_tiles + 1) / 2 : n_key_tiles;  // steps of a sweep
  const int kv_w = kv_lo + half * ntiles * BN;  // first key of this wave's half
  const uint32_t b_shift = SPLIT ? (uint32_t)((ntiles - 1) * BN * rowbytes) : 0u;
  // Load i of a wave goes out with immediate offset (i mod 4) KB, which the
  // hardware adds to the LDS address (M0) and to the memory offset, range
  // check included; so four loads share one M0.  The memory side takes it
  // back through the lane offset, kept non-negative by a descriptor whose
  // base sits kLoadBias bytes before the tile (and whose range is that much
  // longer): lane offset = kLoadBias + (offset in the tile) - immediate.
  constexpr uint32_t kLoadBias = 4096;
  uint32_t ld_off[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int j = NL * wave + i;
    const uint32_t bias = kLoadBias - 1024u * (uint32_t)(i & 3);
    if constexpr (XOR) {
      const int key = 4 * j + (lane >> 4);
      ld_off[i] = key < HALVES * BN ? (uint32_t)(key * rowbytes + ((lane & 15) ^ (key & 15)) * 16) +
                                          (key >= BN ? b_shift : 0u) + bias
                                    : kOutOfRange;
    } else {
      const int p = j * 64 + lane;
      const int rr = p / L::SLOTS, cs = p % L::SLOTS;
      ld_off[i] = cs < CH && rr < HALVES * BN
                      ? (uint32_t)(rr * rowbytes + cs * 16) + (rr >= BN ? b_shift : 0u) + bias
                      : kOutOfRange;
    }
  }
  const char *kseq = reinterpret_cast<const char *>(a.k) + ((size_t)s0k * a.kv_stride + (size_t)hk * D) * 2;
  const char *vseq = reinterpret_cast<const char *>(a.v) + ((size_t)s0k * a.kv_stride + (size_t)hk * D) * 2;

  // Direct loads of the K (or V) rows kt .. kt+BN-1 (and with key halves the
  // second half's rows, ntiles tiles on) into an LDS buffer.
  // kt >= kv_hi is allowed: the range is then empty, nothing is fetched and
  // the (unused) buffer fills with zeros, so a step needs no branch.
  auto issue = [&](const char *seq, char *lds, int kt) {
    const int nrows = SPLIT ? kv_hi - kt : min(kv_hi - kt, BN);
    // later rows read as zeros
    const int rec = max(0, (nrows - 1) * rowbytes + D * 2) + (int)kLoadBias;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<char *>(reinterpret_cast<uintptr_t>(seq) + (size_t)kt * rowbytes - kLoadBias), (short)0,
        rec, kBufferWord3);
    static_for<0, NL>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(lds + (NL * wave + (i & ~3)) * 1024), 16,
                                               ld_off[i], 0, 1024 * (i & 3), 0);
    });
  };
  auto issue_k = [&](int kt, auto buf_tag) { issue(kseq, k_buf(buf_tag), kt); };
  auto issue_v = [&](int kt, auto buf_tag) { issue(vseq, v_buf(buf_tag), kt); };

  // Per-lane LDS read bases (bytes); every other term is an immediate.
  //   K: MFMA row l32 of S^T is key key_of_row(l32) (+32 nb); chunk 2kk + g.
  //   V: in each 16-lane group, lane 4r+q points at key g + 4r (+2 for the
  //   second half of a k step, +16 per k step) and columns
  //   32db + 16*(lane>>4 & 1) + 4q .. +3; the transpose hands lane j of the
  //   group column j of those four keys, in the order P holds them.
  const int hb = half * BN * ROWB;  // this wave's half of an LDS tile
  const int kread = key_of_row(l32) * ROWB + 16 * g + hb;
  const int vread = (g + 4 * ((lane & 15) >> 2)) * ROWB + 32 * ((lane >> 4) & 1) + 8 * (lane & 3) + hb;
  // XOR layout: chunk 2kk + g of key k sits at slot (2kk + g) ^ (k & 15), i.e.
  // at kaddr ^ 32 kk; the V chunk a lane reads for block db (and for the
  // second half of a k step, two keys on) sits at its db = 0 slot XOR 4 db
  // (XOR 2), so each fragment read has its own per-lane address.
  uint32_t kaddr[XOR ? KST : 1], vaddr[XOR ? DB : 1][2];
  if constexpr (XOR) {
    const int key = key_of_row(l32);
    const int k0 = key * ROWB + ((g ^ (key & 1)) | (key & 14)) * 16 + hb;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) kaddr[kk] = (uint32_t)(k0 ^ (32 * kk));
    const int r4 = (lane & 15) >> 2, q4 = lane & 3, hbit = (lane >> 4) & 1;
    const int key0 = g + 4 * r4;
    const int v0 = key0 * ROWB + ((2 * hbit + (q4 >> 1)) ^ key0) * 16 + 8 * (q4 & 1) + hb;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) vaddr[db][hi] = (uint32_t)((v0 ^ (64 * db) ^ (32 * hi)) + 2 * ROWB * hi);
  }
  // K fragment (A operand of S^T, k step kk of 32-key block nb) and V^T
  // fragment (A operand of O^T, k step ks, block db) of the tile at buf.
  auto kfrag = [&](const char *buf, int nb, int kk) __attribute__((always_inline)) -> bf16x8 {
    if constexpr (XOR)
      return *reinterpret_cast<const bf16x8 *>(buf + kaddr[kk] + nb * 32 * ROWB);
    else
      return *reinterpret_cast<const bf16x8 *>(buf + kread + nb * 32 * ROWB + kk * 32);
  };
  auto vfrag = [&](const char *buf, int ks, int db) __attribute__((always_inline)) -> bf16x8 {
    const char *lo_p, *hi_p;
    if constexpr (XOR) {
      lo_p = buf + vaddr[db][0] + ks * 16 * ROWB;
      hi_p = buf + vaddr[db][1] + ks * 16 * ROWB;
    } else {
      lo_p = buf + vread + ks * 16 * ROWB + db * 64;
      hi_p = lo_p + 2 * ROWB;
    }
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)lo_p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)hi_p);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 o[R][DB];
  float l_run[R];  // this lane's share of each row sum
  // Softmax reference of each row in exp2 units, fixed for a whole sweep:
  // the maximum of the first tile holding keys visible to the row.  Later
  // keys may score higher, so probabilities exp2(c*s - m) may exceed 1 (fp32
  // and bf16 keep the same 8 exponent bits, so relative precision is
  // unchanged) and O is never rescaled.  If a row's sum or output comes out
  // non-finite (a score more than ~127 doublings above that first maximum),
  // the workgroup sweeps once more for the exact row maxima and then repeats
  // the accumulation with them, where no probability exceeds 1.
  float m_ref[R];
  auto reset = [&]() {
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[r][db] = (f32x16)(0.0f);
      l_run[r] = 0.0f;
      m_ref[r] = row_ok[r] ? kNegInf : 0.0f;
    }
  };
  reset();

  // accumulator entry j of block nb (lane half g) holds key
  // kt + 32 nb + key_of_row(8 (j >> 2) + 4 g + (j & 3))
  auto visible = [&](int r, int kt, int nb, int j) {
    const int key = kt + nb * 32 + 16 * (j >> 3) + 2 * ((j >> 2) & 1) + 4 * (j & 3) + g;
    return key >= lo_r[r] && key < hi_r[r];
  };
  // a masked score: -inf in exp2 units (SHIFT), else a score that becomes
  // -inf once multiplied by c
  const float s_void = SHIFT || !neg ? kNegInf : __builtin_huge_valf();

  // S^T = K Q^T for the keys held in K buffer KB, every sub-block; each K
  // fragment feeds the R sub-blocks' MFMAs in a row.  The k steps are the
  // outer loop, so the NB 32-key blocks' accumulation chains interleave and
  // no MFMA issues right behind the one it accumulates onto.
  // With SHIFT the accumulation starts from -m (neg_ref) instead of 0, so the
  // scores leave the MFMAs as c s - m, ready for exp2.
  f32x16 neg_ref[R];
  auto qk = [&](auto kbuf_tag, f32x16 (&sc)[R][NB], auto shift_tag) {
    constexpr bool SHIFTED = decltype(shift_tag)::value;
    const char *kb = k_buf(kbuf_tag);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < R; ++r) sc[r][nb] = SHIFTED ? neg_ref[r] : (f32x16)(0.0f);
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 kf = kfrag(kb, nb, kk);
#pragma unroll
        for (int r = 0; r < R; ++r)
          sc[r][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[r][kk], sc[r][nb], 0, 0, 0);
      }
  };
  // Schedule of a plain tile (one basic block; sched_group_barrier masks:
  // 0x2 VALU, 0x8 MFMA, 0x20 VMEM read, 0x100 DS read, 0x400 transcendental
  // -- the VALU mask does not cover v_exp_f32, which only the 0x400 groups
  // place).
  auto plain_tile_schedule = [&]() {
    if constexpr (NB == 1) {
      // 32-key tiles: S^T with the next tile's loads, the softmax of the
      // first k step, the PV MFMAs of that k step under the softmax of the
      // second, then the second k step's PV
      constexpr int SV = 24;  // VALU ops of one k step's softmax
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < KST; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x002, SV, 0);
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, SV / DB, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      return;
    }
    // 64-key tiles: three coarse phases.  Two waves of different workgroups
    // share each SIMD, and the matrix pipe stays busiest when each wave
    // alternates long MFMA runs with long VALU runs, so that one wave's
    // softmax burst runs under the other wave's MFMAs: all of S^T (the two
    // blocks' chains interleaved) with the K fragment reads four ahead and
    // the next tile's loads one per two MFMAs; then the whole tile's
    // softmax as one burst (exp2, conversion, row sums); then PV with its V
    // fragments read one MFMA ahead.  Measured on the 10k causal launch
    // against the earlier order (block 1's S^T under block 0's softmax, PV
    // steps under block 1's softmax): 1.9 % faster; spreading the exp2 two
    // per MFMA instead was 4 % slower, and putting the loads inside the
    // softmax burst 3 % slower.
    constexpr int QK_MFMA = NB * KST * R;
    constexpr int PV_MFMA = (BN / 16) * DB * R;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < QK_MFMA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i % 2 == 1 && i / 2 < 2 * NL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x400, (BN / 2) * R, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, BN * R, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < PV_MFMA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };
  auto apply_mask = [&](f32x16 (&sc)[R][NB], int kt) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[r][nb][j] = visible(r, kt, nb, j) ? sc[r][nb][j] : s_void;
  };
  // Row maximum of c*s over the tile for sub-block r, both lane halves combined.
  auto row_max = [&](const f32x16 (&scr)[NB]) {
    float mx = kNegInf;
    if (!SHIFT && neg) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, -scr[nb][j]);
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, scr[nb][j]);
    }
    const float mt = SHIFT ? mx : mx * cabs;
    return fmaxf(mt, xor32(mt));
  };
  // P = exp2(c*s - m) as bf16 B operands of O^T = V^T P^T, and the row sum
  // of those same bf16 values (SHIFTED: the scores hold c*s - m already).
  // k step ks covers keys 16ks .. 16ks+15, held in accumulator entries
  // 8*(ks&1) .. +7 of block ks>>1; entry e of lane half g is key
  // 16ks + g + 4(e & 3) + 2(e >> 2).
  auto softmax = [&](f32x16 (&sc)[R][NB], bf16x8 (&pf)[R][BN / 16], auto shift_tag) {
    constexpr bool SHIFTED = decltype(shift_tag)::value;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // a row with no visible key yet has every score at -inf here
        const float neg_m = m_ref[r] == kNegInf ? 0.0f : -m_ref[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = sc[r][ks >> 1][8 * (ks & 1) + e];
          pf[r][ks][e] = (__bf16)fast_exp2(SHIFTED ? x : SHIFT ? x + neg_m : __builtin_fmaf(x, c, neg_m));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pr = {pf[r][ks][2 * e], pf[r][ks][2 * e + 1]};
          l_run[r] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run[r], false);
        }
      }
  };
  // O += P V with V from V buffer VB; each V fragment feeds the R
  // sub-blocks' MFMAs in a row.
  auto pv = [&](auto vbuf_tag, const bf16x8 (&pf)[R][BN / 16]) {
    const char *vb = v_buf(vbuf_tag);
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 vf = vfrag(vb, ks, db);
#pragma unroll
        for (int r = 0; r < R; ++r)
          o[r][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[r][ks], o[r][db], 0, 0, 0);
      }
  };

  // Step t: the workgroup loads tile t of each half (first key
  // load_base(t)), and this wave computes on keys kv_w + t BN ..
  auto load_base = [&](int t) { return t < ntiles ? kv_lo + t * BN : kv_hi; };
  auto wave_sees = [&](int t) {
    const int kt = kv_w + t * BN;
    return kt < w_hi && kt + BN > w_lo;
  };
  auto needs_mask = [&](int t) {
    const int kt = kv_w + t * BN;
    return kt < i_lo || kt + BN > i_hi;
  };
  // Key tiles inside every row's visible range of the workgroup (the
  // intersection [lo(last row), hi(first row)) of its rows) need no mask for
  // any wave: steps whose tiles (in both halves) all lie there form one run
  // [t_plain0, t_plain1) of the sweep.  The first step always takes the
  // general step, which sets the softmax reference.
  int t_plain0 = 1, t_plain1 = 1;
  {
    int wlo, whi, tmp2;
    row_range(mask, W, qend - 1 + off, nk, wlo, tmp2);
    row_range(mask, W, q0 + off, nk, tmp2, whi);
    int first = 1, last = ntiles;
#pragma unroll
    for (int hh = 0; hh < HALVES; ++hh) {
      const int base = kv_lo + hh * ntiles * BN;
      const int tiles_h = min(ntiles, n_key_tiles - hh * ntiles);  // tiles of this half
      // tiles [first, last) of the half start at or after wlo and end at or before whi
      first = max(first, (wlo - base + BN - 1) / BN);
      last = min(last, min(tiles_h, (whi - base) / BN));
    }
    if (has_item && last > first) {
      t_plain0 = first;
      t_plain1 = last;
    }
  }

  // General step (first tile, diagonal and edge tiles): a wave that sees
  // none of the tile only joins the barrier; otherwise masking and the
  // reference update touch only S and m_ref, then the same softmax and PV run.
  auto k_rt = [&](int buf) -> const char * { return buf ? k_lds1 : k_lds0; };
  auto v_rt = [&](int buf) -> const char * { return buf ? v_lds1 : v_lds0; };
  auto general_step = [&](int t) __attribute__((always_inline)) {
    const int kt = kv_w + t * BN;
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      const int kn = load_base(t + 1);
      if (buf) {
        issue_k(kn, std::integral_constant<int, 0>{});
        issue_v(kn, std::integral_constant<int, 0>{});
      } else {
        issue_k(kn, std::integral_constant<int, 1>{});
        issue_v(kn, std::integral_constant<int, 1>{});
      }
    }
    if (wave_sees(t)) {
      f32x16 sc[R][NB];
      {
        const char *kb = k_rt(buf);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int r = 0; r < R; ++r) sc[r][nb] = (f32x16)(0.0f);
#pragma unroll
          for (int kk = 0; kk < KST; ++kk) {
            const bf16x8 kf = kfrag(kb, nb, kk);
#pragma unroll
            for (int r = 0; r < R; ++r)
              sc[r][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[r][kk], sc[r][nb], 0, 0, 0);
          }
        }
      }
      if (needs_mask(t)) apply_mask(sc, kt);
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (__builtin_amdgcn_ballot_w64(m_ref[r] == kNegInf)) {
          const float mt = row_max(sc[r]);
          m_ref[r] = m_ref[r] == kNegInf ? mt : m_ref[r];
        }
      bf16x8 pf[R][BN / 16];
      softmax(sc, pf, std::false_type{});
      {
        const char *vb = v_rt(buf);
#pragma unroll
        for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 vf = vfrag(vb, ks, db);
#pragma unroll
            for (int r = 0; r < R; ++r)
              o[r][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[r][ks], o[r][db], 0, 0, 0);
          }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Plain step: one basic block, scheduled so MFMA and softmax work overlap.
  auto plain_step = [&](auto buf_tag, int t) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    // the last tile's "next" loads are empty (range starts at kv_hi)
    const int kn = load_base(t + 1);
    issue_k(kn, std::integral_constant<int, BUF ^ 1>{});
    issue_v(kn, std::integral_constant<int, BUF ^ 1>{});
    f32x16 sc[R][NB];
    bf16x8 pf[R][BN / 16];
    qk(buf_tag, sc, std::integral_constant<bool, SHIFT>{});
    softmax(sc, pf, std::integral_constant<bool, SHIFT>{});
    pv(buf_tag, pf);
    plain_tile_schedule();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Accumulating sweep over the double-buffered K/V tiles; the loads of tile
  // t+1 are in flight while tile t is computed.
  auto accumulate_sweep = [&]() __attribute__((always_inline)) {
    issue_k(kv_lo, std::integral_constant<int, 0>{});
    issue_v(kv_lo, std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int t = 0;
    for (; t < t_plain0 && t < ntiles; ++t) general_step(t);
    if constexpr (SHIFT) {
#pragma unroll
      for (int r = 0; r < R; ++r) neg_ref[r] = (f32x16)(m_ref[r] == kNegInf ? 0.0f : -m_ref[r]);
    }
    if (t < t_plain1 && (t & 1)) plain_step(std::integral_constant<int, 1>{}, t++);
    for (; t + 1 < t_plain1; t += 2) {
      plain_step(std::integral_constant<int, 0>{}, t);
      plain_step(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t < t_plain1) plain_step(std::integral_constant<int, 0>{}, t++);
    for (; t < ntiles; ++t) general_step(t);
  };
  // Exact row maxima (after an overflow): scores only, no accumulation.
  auto max_sweep = [&]() __attribute__((always_inline)) {
    auto step = [&](auto buf_tag, int t) {
      constexpr int BUF = decltype(buf_tag)::value;
      const int kt = kv_w + t * BN;
      issue_k(load_base(t + 1), std::integral_constant<int, BUF ^ 1>{});
      if (wave_sees(t)) {
        f32x16 sc[R][NB];
        qk(buf_tag, sc, std::false_type{});
        if (needs_mask(t)) apply_mask(sc, kt);
#pragma unroll
        for (int r = 0; r < R; ++r) m_ref[r] = fmaxf(m_ref[r], row_max(sc[r]));
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    issue_k(kv_lo, std::integral_constant<int, 0>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
      step(std::integral_constant<int, 0>{}, t);
      if (t + 1 < ntiles) step(std::integral_constant<int, 1>{}, t + 1);
    }
  };

  for (int pass = 0;; ++pass) {
    accumulate_sweep();
    if (pass == 1) break;
    // A row whose sum or output overflowed: the workgroup redoes its rows
    // with the exact row maxima as references.
    // x * 0 is 0 for finite x and NaN for an infinity or a NaN, so one sum
    // of such products flags every non-finite value of a row; a test per
    // element (short-circuit ||) compiles to a branch per accumulator entry,
    // microseconds per workgroup.  Entry j of block db holds columns
    // 32 db + 8 (j >> 2) .. +7 of O^T across both lane halves, all real or
    // all padding, since D is a multiple of 8.
    bool bad = false;
    if (wave_active) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float probe = (l_run[r] + xor32(l_run[r])) * 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (32 * db + 8 * (j >> 2) < D) probe = __builtin_fmaf(o[r][db][j], 0.0f, probe);
        bad = bad || (row_ok[r] && !__builtin_isfinite(probe));
      }
    }
    if (!__syncthreads_or(bad)) break;
    reset();
    max_sweep();
  }

  if constexpr (SPLIT) {
    // Merge of the key halves: waves 2 and 3 leave each lane's reference,
    // share of the row sum and unnormalised outputs in LDS (the V buffers
    // and a corner of the second K buffer, all free after the last barrier),
    // lane-major so every access is one 64-lane stride; waves 0 and 1 rescale
    // both partitions to the larger reference m:
    //   o = o_a 2^(m_a - m) + o_b 2^(m_b - m),  l likewise
    // (a half with no visible key for a row has reference -inf and weight 0).
    float *po = reinterpret_cast<float *>((wave & 1) ? v_lds1 : v_lds0);
    float *pml = reinterpret_cast<float *>(k_lds1) + (wave & 1) * 128;
    if (wave >= 2 && wave_active) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) po[(db * 16 + j) * 64 + lane] = o[0][db][j];
      pml[lane] = m_ref[0];
      pml[64 + lane] = l_run[0];
    }
    __syncthreads();
    if (wave < 2 && wave_active) {
      const float ma = m_ref[0], mb = pml[lane];
      const float m = fmaxf(ma, mb);
      const float fa = ma == kNegInf ? 0.0f : fast_exp2(ma - m);
      const float fb = mb == kNegInf ? 0.0f : fast_exp2(mb - m);
      l_run[0] = l_run[0] * fa + pml[64 + lane] * fb;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[0][db][j] = o[0][db][j] * fa + po[(db * 16 + j) * 64 + lane] * fb;
      m_ref[0] = m;
    }
  }

  // (with key halves only waves 0 and 1 store)
  if (wave_active && (!SPLIT || wave < 2)) {
    // Output rows go through LDS (the wave's own 32 rows of the K buffers,
    // free once the sweep is over): the accumulator holds 4-column pieces of
    // 32 rows, and read back, consecutive lanes hold consecutive 16-byte
    // chunks of whole rows, so each store writes whole rows (for head_dim
    // 128, four 256-byte rows).  head_dim 128 stages row i's chunk c at slot
    // c ^ (i mod 16) (no conflicts on the reads, 2-way on the writes); 64 and
    // 72 pad each staged row by one chunk.
    constexpr int CHR = D / 8;                    // 16-byte chunks per output row
    constexpr int SR = XOR ? D * 2 : D * 2 + 16;  // bytes per staged row
    char *stage;
    if constexpr (2 * 32 * SR <= BUF_BYTES) {
      stage = (wave < 2 ? k_lds0 : k_lds1) + (wave & 1) * 32 * SR;
    } else {  // 32-key tiles: one wave per K or V buffer
      static_assert(NW == 4 && 32 * SR <= BUF_BYTES, "a wave's staged rows fit one buffer");
      stage = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float l_tot = l_run[r] + xor32(l_run[r]);
      const float inv = row_ok[r] ? 1.0f / l_tot : 0.0f;
      if (row_ok[r] && a.lse != nullptr && g == 0)
        a.lse[(size_t)(s0q + row[r]) * a.hq + h] = (m_ref[r] + log2f(l_tot)) * kLn2;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = 32 * db + 8 * jj + 4 * g;
          if (d >= D) continue;  // padding rows of O^T
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[r][db][4 * jj + e] * inv);
          const int off = XOR ? (((d >> 3) ^ (l32 & 15)) << 4) + 8 * g : 2 * d;
          *reinterpret_cast<bf16x4 *>(stage + l32 * SR + off) = w;
        }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the staged rows are in LDS
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < (32 * CHR + 63) / 64; ++i) {
        const int f = 64 * i + lane;
        const int sr = f / CHR, cc = f - sr * CHR;
        const int qr = wq0 + 32 * r + sr;
        if (sr < 32 && qr < nq) {
          const int off = XOR ? ((cc ^ (sr & 15)) << 4) : 16 * cc;
          const bf16x8 val = *reinterpret_cast<const bf16x8 *>(stage + sr * SR + off);
          *reinterpret_cast<bf16x8 *>(reinterpret_cast<__bf16 *>(a.out) + ((size_t)(s0q + qr) * a.hq + h) * D +
                                      8 * cc) = val;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next sub-block's writes
      __builtin_amdgcn_wave_barrier();
    }
  }
  // every workgroup counts itself out; the last one leaves the counters at
  // zero for the stream's next launch
  if (a.tickets != nullptr && tid == 0 && atomicAdd(&a.tickets[1], 1) == a.total_items - 1) {
    atomicExch(&a.tickets[0], 0);
    atomicExch(&a.tickets[1], 0);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// fp32 / matrix-core family: v_mfma_f32_32x32x2_f32, exact fp32 products with
// fp32 accumulation (157.3 TFLOP/s peak against 78.6 for unpacked vector
// FMAs).  One workgroup per (sequence, query head, 128 query rows), four
// waves of 32 rows; 32-key tiles.
//   S^T = K Q^T: step s of the D/2 k steps takes column s from lane half 0
//   and column s + D/2 from lane half 1, so each lane's q values and K row
//   reads are contiguous (16-byte LDS reads feed four steps).
//   O^T = V^T P^T: the scores stay in registers as the B operand -- step t
//   of 16 takes, in lane half g, the key of accumulator element t
//   (8 (t >> 2) + 4 g + (t & 3)) -- and V is stored transposed in LDS,
//   [d][key], so four steps' V^T values are one 16-byte read.
// Online softmax per tile in exp2 units with the lazy rescale; rows past D
// (head dim 72 takes three 32-row blocks) are computed over zero rows of
// V^T and dropped.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_f32_mfma(const LaunchArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(D % 8 == 0, "head dim in whole float4 pairs");
  constexpr int BN = 32;
  constexpr int H2 = D / 2;             // k steps of S^T
  constexpr int DB = (D + 31) / 32;     // 32-row blocks of O^T
  constexpr int KROW = D + 4;           // K tile row stride (floats); odd multiple of 16 bytes
  constexpr int VROW = BN + 4;          // V^T tile row stride (floats)
  constexpr int KT_F = BN * KROW, VT_F = DB * 32 * VROW;
  constexpr int NF4 = BN * D / 4;           // float4s of a K (or V) tile
  constexpr int LOADS = (NF4 + 255) / 256;  // per thread (the last round partial for D = 72)
  __shared__ __attribute__((aligned(16))) float k_lds[2][KT_F];
  __shared__ __attribute__((aligned(16))) float v_lds[2][VT_F];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const Item it = decode_item(a, blockIdx.x);
  const int s0q = a.q_start[it.seq], s0k = a.k_start[it.seq];
  const int nq = a.q_len[it.seq], nk = a.k_len[it.seq], off = nk - nq;
  const int h = it.head;
  const int hk = h / a.group;
  const int mask = a.mask_kind;
  const int W = a.window;
  const float c = a.c == 0.0f ? 0x1p-126f : a.c;  // scale 0: every weight exp2(~0) = 1

  const int q0 = it.tile * 128;
  const int qend = min(q0 + 128, nq);
  int kv_lo, kv_hi, tmp;
  row_range(mask, W, q0 + off, nk, kv_lo, tmp);
  row_range(mask, W, qend - 1 + off, nk, tmp, kv_hi);

  const int row = q0 + 32 * wave + l32;
  const bool row_ok = row < nq;
  int lo_r = 0, hi_r = 0;
  if (row_ok) row_range(mask, W, row + off, nk, lo_r, hi_r);

  // q[row][s + g D/2], s = 0 .. D/2 - 1
  float qv[H2];
  {
    const float *qrow = reinterpret_cast<const float *>(a.q) + (size_t)(s0q + (row_ok ? row : 0)) * a.q_stride +
                        (size_t)h * D + g * H2;
#pragma unroll
    for (int s4 = 0; s4 < H2; s4 += 4) {
      const f32x4 x = row_ok ? *reinterpret_cast<const f32x4 *>(qrow + s4) : (f32x4)(0.0f);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[s4 + e] = x[e];
    }
  }

  // V^T rows past D stay zero in both buffers
  for (int i = tid; i < (DB * 32 - D) * VROW; i += 256) {
    v_lds[0][D * VROW + i] = 0.0f;
    v_lds[1][D * VROW + i] = 0.0f;
  }

  const size_t kv_rs = (size_t)a.kv_stride;
  const float *kbase = reinterpret_cast<const float *>(a.k) + (size_t)s0k * kv_rs + (size_t)hk * D;
  const float *vbase = reinterpret_cast<const float *>(a.v) + (size_t)s0k * kv_rs + (size_t)hk * D;
  // tile kt: thread loads float4 u = tid + 256 i of K and of V (key u / (D/4))
  f32x4 kr[LOADS], vr[LOADS];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int u = min(tid + 256 * i, NF4 - 1);  // a partial last round repeats the final float4
      const int key = u / (D / 4), col = (u % (D / 4)) * 4;
      const int j = min(kt + key, kv_hi - 1);  // rows past the range are masked in the scores
      kr[i] = *reinterpret_cast<const f32x4 *>(kbase + (size_t)j * kv_rs + col);
      vr[i] = *reinterpret_cast<const f32x4 *>(vbase + (size_t)j * kv_rs + col);
      if (kt + key >= kv_hi) vr[i] = (f32x4)(0.0f);  // their probabilities are 0; keep V finite
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int u = min(tid + 256 * i, NF4 - 1);  // repeats write the same values again
      const int key = u / (D / 4), col = (u % (D / 4)) * 4;
      *reinterpret_cast<f32x4 *>(&k_lds[buf][key * KROW + col]) = kr[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) v_lds[buf][(col + e) * VROW + key] = vr[i][e];
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16)(0.0f);
  float m_run = kNegInf, l_run = 0.0f;  // reference (exp2 units), this lane's share of the sum

  int buf = 0;
  if (kv_lo < kv_hi) {
    load_tile(kv_lo);
    store_tile(0);
  }
  __syncthreads();
  for (int kt = kv_lo; kt < kv_hi; kt += BN) {
    const bool more = kt + BN < kv_hi;
    if (more) load_tile(kt + BN);
    // S^T block: keys kt .. kt+31 (rows) x this wave's 32 queries (columns)
    f32x16 sc = (f32x16)(0.0f);
    {
      const float *krow = &k_lds[buf][l32 * KROW + g * H2];
#pragma unroll
      for (int s4 = 0; s4 < H2; s4 += 4) {
        const f32x4 kx = *reinterpret_cast<const f32x4 *>(krow + s4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc = __builtin_amdgcn_mfma_f32_32x32x2f32(kx[e], qv[s4 + e], sc, 0, 0, 0);
      }
    }
    // mask, reference, probabilities (element e: key kt + 8 (e >> 2) + 4 g + (e & 3))
    float mt = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kt + 8 * (e >> 2) + 4 * g + (e & 3);
      const bool vis = row_ok && key >= lo_r && key < hi_r;
      sc[e] = vis ? sc[e] * c : kNegInf;
      mt = fmaxf(mt, sc[e]);
    }
    mt = fmaxf(mt, xor32(mt));
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack)) {
      const float m_new = mt > m_run + kRescaleSlack ? mt : m_run;
      const float alpha = m_run == kNegInf ? 0.0f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m_run = m_new;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      sc[e] = sc[e] == kNegInf ? 0.0f : fast_exp2(sc[e] - m_run);
      l_run += sc[e];
    }
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const float *vrow = &v_lds[buf][(32 * db + l32) * VROW + 4 * g];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const f32x4 vx = *reinterpret_cast<const f32x4 *>(vrow + 8 * t4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vx[e], sc[4 * t4 + e], o[db], 0, 0, 0);
      }
    }
    // the other buffer's last readers finished before the previous barrier
    if (more) {
      store_tile(buf ^ 1);
      __syncthreads();
    }
    buf ^= 1;
  }

  const float l_tot = l_run + xor32(l_run);
  if (row_ok) {
    const float inv = 1.0f / l_tot;
    if (a.lse != nullptr && g == 0) a.lse[(size_t)(s0q + row) * a.hq + h] = (m_run + log2f(l_tot)) * kLn2;
    float *orow = reinterpret_cast<float *>(a.out) + ((size_t)(s0q + row) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = 32 * db + 8 * jj + 4 * g;
        if (d >= D) continue;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[db][4 * jj + e] * inv;
        *reinterpret_cast<f32x4 *>(orow + d) = w;
      }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <typename K>
int launch(K kernel, const LaunchArgs &a, int threads, void *stream) {
  void *args[] = {const_cast<LaunchArgs *>(&a)};
  return static_cast<int>(hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3(a.total_items),
                                          dim3(threads), args, 0,
                                          static_cast<hipStream_t>(stream)));
}

constexpr int kWavesBf16 = 4;
// head_dim 128 full and window launches of at least this many items (12
// rounds of 256 CUs' workgroups) take 32-key tiles at three workgroups per
// CU: the third workgroup hides more of each item's fixed costs (packed
// window-256 batch -11 %).  Causal launches keep 64-key tiles at two
// workgroups per CU, whose plain steps start S^T from -m (the 32-key
// instance has no registers for that): packed causal batch -2 % against
// 32-key tiles, which were 2 % faster than 64-key tiles with the per-score
// FMA.
constexpr int kManyItems = 3072;

// The prescaled-query instance of a kernel for scales up to kPrescaleMaxC
// when no log-sum-exp is returned, the exact-query one otherwise.
template <int D, int R, int BN, bool SPLIT>
int launch_sh(const LaunchArgs &a, void *stream) {
  return (a.lse == nullptr && a.c <= kPrescaleMaxC && a.c >= -kPrescaleMaxC)
             ? launch(fwd_bf16_fast<D, kWavesBf16, R, BN, SPLIT, true>, a, kWavesBf16 * 64, stream)
             : launch(fwd_bf16_fast<D, kWavesBf16, R, BN, SPLIT, false>, a, kWavesBf16 * 64, stream);
}

}  // namespace

int rows_per_workgroup_bf16(int) { return kWavesBf16 * 32; }
int rows_per_workgroup_bf16_halves(int) { return kWavesBf16 * 32 / 2; }
int rows_per_workgroup_f32(int) { return 128; }

int launch_bf16(const LaunchArgs &a, int head_dim, void *stream) {
  if (a.key_halves) {
    switch (head_dim) {
      case 64: return launch_sh<64, 1, 32, true>(a, stream);
      case 72: return launch_sh<72, 1, 32, true>(a, stream);
      case 128: return launch_sh<128, 1, 32, true>(a, stream);
      default: return static_cast<int>(hipErrorInvalidValue);
    }
  }
  switch (head_dim) {
    case 64: return launch_sh<64, 1, 64, false>(a, stream);
    case 72: return launch_sh<72, 1, 64, false>(a, stream);
    case 128:
      return a.total_items >= kManyItems && a.mask_kind != kCausal
                 ? launch(fwd_bf16_fast<128, kWavesBf16, 1, 32, false, false>, a, kWavesBf16 * 64, stream)
                 : launch_sh<128, 1, 64, false>(a, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

// ---------------------------------------------------------------------------
// Work tickets.  The hardware hands workgroup b to XCD b mod 8, and each XCD
// runs its share at its own pace: on a 10k-token causal launch the XCDs'
// per-tile times differ by up to ~8 %, so with items bound to workgroups the
// fast XCDs idle while the slowest finishes.  For heavy causal launches the
// first wave of workgroups (one per slot) keeps items 0 .. slots-1, and every
// later workgroup takes the next item, heaviest first, from a device counter
// when it starts, whichever XCD it runs on: list scheduling over the whole
// chip.  Each stream owns one pair of counters (ticket, finished) in a static
// device array; launches on one stream run one after another, so they share
// it, and the last workgroup of a launch puts both counters back to zero.
// Streams under capture (whose graph may later replay beside eager launches
// on the same stream) and the per-thread default stream (one handle, many
// streams) launch without tickets, as does any stream once the array is full.
// ---------------------------------------------------------------------------

constexpr int kTicketSlots = 1024;  // streams per device
static __device__ int32_t ticket_pool[2 * kTicketSlots];

namespace {

constexpr int kTicketDevices = 64;
constexpr int kSlotsPerCu = 2;  // resident workgroups of the bf16 kernel

struct DeviceTickets {
  int32_t *pool = nullptr;
  int slots = 0;  // workgroup slots of the device
  std::map<hipStream_t, int> owner;
};
std::mutex ticket_mutex;
DeviceTickets device_tickets[kTicketDevices];

}  // namespace

int work_tickets(LaunchArgs &a, void *stream) {
  a.tickets = nullptr;
  a.ticket_from = a.total_items;
  if (a.mask_kind != kCausal) return 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (st == hipStreamPerThread) return 0;
  int dev = 0;
  hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kTicketDevices) return 0;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if ((e = hipStreamIsCapturing(st, &cs)) != hipSuccess) return static_cast<int>(e);
  if (cs != hipStreamCaptureStatusNone) return 0;
  std::lock_guard<std::mutex> lock(ticket_mutex);
  DeviceTickets &dt = device_tickets[dev];
  if (dt.pool == nullptr) {
    int cur = 0, cus = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return static_cast<int>(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return static_cast<int>(e);
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(ticket_pool));
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return static_cast<int>(e);
    if (p == nullptr || cus <= 0) return static_cast<int>(hipErrorInvalidSymbol);
    dt.pool = static_cast<int32_t *>(p);
    dt.slots = kSlotsPerCu * cus;
  }
  // with a few items per slot the static heaviest-first order already
  // balances, and a ticket's round trip would only lengthen each item
  if (a.total_items <= 2 * dt.slots) return 0;
  auto it = dt.owner.find(st);
  if (it == dt.owner.end()) {
    if (static_cast<int>(dt.owner.size()) >= kTicketSlots) return 0;
    it = dt.owner.emplace(st, static_cast<int>(dt.owner.size())).first;
  }
  a.tickets = dt.pool + 2 * it->second;
  a.ticket_from = dt.slots;
  return 0;
}

int launch_f32(const LaunchArgs &a, int head_dim, void *stream) {
  switch (head_dim) {
    case 64: return launch(fwd_f32_mfma<64>, a, 256, stream);
    case 72: return launch(fwd_f32_mfma<72>, a, 256, stream);
    case 128: return launch(fwd_f32_mfma<128>, a, 256, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace attn
