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

#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {



struct Item {
  int seq;
  int tile;
  int head;
};

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
__device__ Item decode_item(const LaunchArgs &a, int r) {
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
    for (int b = 0; b < a.n_seqs; ++b) {
      const int cnt = a.seq_tiles[b] * a.hq;
      if (r < cnt) {
        it.seq = b;
        it.tile = r / a.hq;
        slot = r - it.tile * a.hq;
        break;
      }
      r -= cnt;
    }
  }
  it.head = (a.hq % 8 == 0) ? (slot & 7) * (a.hq >> 3) + (slot >> 3) : slot;
  return it;
}

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
// as zeros (buffer range check).  Both tiles use the padded, key-permuted
// layout of attn_device.h, whose K row reads and V transposing reads are
// free of bank conflicts.
// ---------------------------------------------------------------------------

// Each wave owns R consecutive 32-row query sub-blocks (the workgroup covers
// NW * 32 * R rows); every K or V fragment read from LDS feeds the R
// sub-blocks' MFMAs back to back.  R = 1 runs two workgroups per CU (two waves
// per SIMD, up to 256 registers each) and is the instance dispatched.  R = 2
// (one wave per SIMD, up to 512 registers) halves the LDS reads and K/V tile
// loads per MFMA, but with no second wave to hide latency and its scores
// spilling into AGPRs it measured ~30 % slower on gfx950, so it is not
// instantiated.
template <int D, int NW, int R>
__global__ __launch_bounds__(NW * 64, 2 / R) void fwd_bf16_fast(const LaunchArgs a) {
  // The host pass only needs this kernel's signature for its launch stub;
  // the body (gfx950-only builtins) is compiled for the device alone.
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(D == 64 || D == 72 || D == 128, "fast path covers head_dim 64, 72 and 128");
  static_assert(R == 1 || R == 2, "one or two query sub-blocks per wave");
  using L = FastLayout<D>;
  constexpr int BM = NW * 32 * R;
  constexpr int BN = 64;
  constexpr int CH = L::CH;
  constexpr int KST = L::KST;         // MFMA k steps of S^T (the last one zero-padded when D = 72)
  constexpr int DB = (D + 31) / 32;  // 32-row blocks of O^T (rows past D are computed and dropped)
  constexpr int KBUF = BN * L::ROWB;  // bytes per K (or V) tile
  // A tile is NLOADS wave-wide direct loads (64 lanes x 16 bytes); each wave
  // issues NL of them, and a wave whose last load falls past the tile sends
  // it, all lanes out of range, into a 1 KB spill slot after the tile, so
  // the issue code has no branches.
  constexpr int NLOADS = KBUF / 1024;
  constexpr int NL = (NLOADS + NW - 1) / NW;
  constexpr int BUF_BYTES = KBUF + (NL * NW > NLOADS ? 1024 : 0);  // one LDS buffer
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
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const Item it = decode_item(a, blockIdx.x);
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

  // The wave's rows [wq0, wq0 + 32R): the union of their visible keys is
  // [w_lo, w_hi), the intersection [i_lo, i_hi).
  const int wq0 = q0 + wave * 32 * R;
  const bool wave_active = wq0 < nq;
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
  // holds q[row[r]][16*kk + 8*g .. +7].
  bf16x8 qf[R][KST];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const __bf16 *qrow = reinterpret_cast<const __bf16 *>(a.q) +
                         (size_t)(s0q + (row_ok[r] ? row[r] : 0)) * a.q_stride + (size_t)h * D;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      qf[r][kk] = row_ok[r] && 16 * kk + 8 * g < D ? *reinterpret_cast<const bf16x8 *>(qrow + 16 * kk + 8 * g)
                                                   : (bf16x8)((__bf16)0.0f);
  }

  // Direct loads: wave-wide load j fills LDS slots 64j .. 64j+63 of a tile;
  // slot p is row p / SLOTS, chunk p % SLOTS (chunks >= CH are padding).
  const int rowbytes = a.kv_stride * 2;  // bytes between consecutive tokens of one head
  uint32_t ld_off[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int p = (wave + NW * i) * 64 + lane;
    const int rr = p / L::SLOTS, cs = p % L::SLOTS;
    ld_off[i] = cs < CH ? (uint32_t)(rr * rowbytes + cs * 16) : kOutOfRange;
  }
  const char *kseq = reinterpret_cast<const char *>(a.k) + ((size_t)s0k * a.kv_stride + (size_t)hk * D) * 2;
  const char *vseq = reinterpret_cast<const char *>(a.v) + ((size_t)s0k * a.kv_stride + (size_t)hk * D) * 2;

  // Direct loads of the K (or V) rows kt .. kt+63 into an LDS buffer.
  // kt >= kv_hi is allowed: the range is then empty, nothing is fetched and
  // the (unused) buffer fills with zeros, so a step needs no branch.
  auto issue = [&](const char *seq, char *lds, int kt) {
    const int nrows = min(kv_hi - kt, BN);
    const int rec = max(0, (nrows - 1) * rowbytes + D * 2);  // later rows read as zeros
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(seq + (size_t)kt * rowbytes), (short)0, rec, kBufferWord3);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int j = min(wave + NW * i, NLOADS);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(lds + j * 1024), 16, ld_off[i], 0, 0, 0);
    }
  };
  auto issue_k = [&](int kt, auto buf_tag) { issue(kseq, k_buf(buf_tag), kt); };
  auto issue_v = [&](int kt, auto buf_tag) { issue(vseq, v_buf(buf_tag), kt); };

  // Per-lane LDS read bases (bytes); every other term is an immediate.
  //   K: MFMA row l32 of S^T is key key_of_row(l32) (+32 nb); chunk 2kk + g.
  //   V: in each 16-lane group, lane 4r+q points at key g + 4r (+2 for the
  //   second half of a k step, +16 per k step) and columns
  //   32db + 16*(lane>>4 & 1) + 4q .. +3; the transpose hands lane j of the
  //   group column j of those four keys, in the order P holds them.
  const int kread = key_of_row(l32) * L::ROWB + 16 * g;
  const int vread = (g + 4 * ((lane & 15) >> 2)) * L::ROWB + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

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
  // a score that becomes -inf once multiplied by c
  const float s_void = neg ? __builtin_huge_valf() : kNegInf;

  // S^T = K Q^T for the 64 keys held in K buffer KB, every sub-block; each K
  // fragment feeds the R sub-blocks' MFMAs in a row.
  auto qk = [&](auto kbuf_tag, f32x16 (&sc)[R][2]) {
    const char *kb = k_buf(kbuf_tag) + kread;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int r = 0; r < R; ++r) sc[r][nb] = (f32x16)(0.0f);
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kb + nb * 32 * L::ROWB + kk * 32);
#pragma unroll
        for (int r = 0; r < R; ++r)
          sc[r][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[r][kk], sc[r][nb], 0, 0, 0);
      }
    }
  };
  // Schedule of a plain tile (one basic block): the MFMAs of the second
  // 32-key block of S^T run under the softmax of the first, and the PV MFMAs
  // of the first two k steps under the softmax of the second, with a few LDS
  // reads kept ahead of their MFMAs and the next tile's loads one per MFMA
  // of the first block (any left over follow: issued in a burst, eight
  // waves' loads back up the CU's load pipe and stall the MFMA issue; one
  // per MFMA measured 0.7 % faster at 10k and 3-7 % at 1-2k tokens) (mask:
  // 2 VALU, 8 MFMA, 0x20 VMEM read, 0x100 DS read).
  auto plain_tile_schedule = [&]() {
    constexpr int SOFT = 3 * (BN / 2) / KST;  // softmax VALU ops per QK MFMA
    constexpr int PV_HALF = DB * (BN / 32);   // PV k-step pairs' fragments
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < KST; ++i) {  // S^T block 0, with the next tile's loads
      __builtin_amdgcn_sched_group_barrier(0x008, R, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < KST * R; ++i) {  // S^T block 1 under softmax of block 0
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, SOFT, 0);
      if (i % R == R - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < PV_HALF * R; ++i) {  // PV of k steps 0-1 under softmax of block 1
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2 * KST * SOFT / PV_HALF, 0);
      if (i % R == R - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < PV_HALF * R; ++i) {  // PV of k steps 2-3
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i % R == R - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };
  auto apply_mask = [&](f32x16 (&sc)[R][2], int kt) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[r][nb][j] = visible(r, kt, nb, j) ? sc[r][nb][j] : s_void;
  };
  // Row maximum of c*s over the tile for sub-block r, both lane halves combined.
  auto row_max = [&](const f32x16 (&scr)[2]) {
    float mx = kNegInf;
    if (neg) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, -scr[nb][j]);
    } else {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, scr[nb][j]);
    }
    const float mt = mx * cabs;
    return fmaxf(mt, xor32(mt));
  };
  // P = exp2(c*s - m) as bf16 B operands of O^T = V^T P^T, and the row sum
  // of those same bf16 values.  k step ks covers keys 16ks .. 16ks+15, held
  // in accumulator entries 8*(ks&1) .. +7 of block ks>>1; entry e of lane
  // half g is key 16ks + g + 4(e & 3) + 2(e >> 2).
  auto softmax = [&](f32x16 (&sc)[R][2], bf16x8 (&pf)[R][BN / 16]) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // a row with no visible key yet has every score at -inf here
        const float neg_m = m_ref[r] == kNegInf ? 0.0f : -m_ref[r];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[r][ks][e] = (__bf16)fast_exp2(__builtin_fmaf(sc[r][ks >> 1][8 * (ks & 1) + e], c, neg_m));
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
    const char *vb = v_buf(vbuf_tag) + vread;
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char *vp = vb + ks * 16 * L::ROWB + db * 64;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vp));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vp + 2 * L::ROWB));
        const bf16x8 vf = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int r = 0; r < R; ++r)
          o[r][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[r][ks], o[r][db], 0, 0, 0);
      }
  };

  const int ntiles = (kv_hi - kv_lo + BN - 1) / BN;
  auto wave_sees = [&](int t) {
    const int kt = kv_lo + t * BN;
    return kt < w_hi && kt + BN > w_lo;
  };
  auto needs_mask = [&](int t) {
    const int kt = kv_lo + t * BN;
    return kt < i_lo || kt + BN > i_hi;
  };
  // Key tiles inside every row's visible range of the workgroup (the
  // intersection [lo(last row), hi(first row)) of its rows) need no mask for
  // any wave: they form one run [t_plain0, t_plain1) of the sweep.  The first
  // tile always takes the general step, which sets the softmax reference.
  int t_plain0 = 1, t_plain1 = 1;
  {
    int wlo, whi, tmp2;
    row_range(mask, W, qend - 1 + off, nk, wlo, tmp2);
    row_range(mask, W, q0 + off, nk, tmp2, whi);
    const int first = max(1, (wlo - kv_lo + BN - 1) / BN);
    const int last = max(0, (whi - kv_lo) / BN);  // tiles [0, last) end at or before whi
    if (last > first) {
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
    const int kt = kv_lo + t * BN;
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      if (buf) {
        issue_k(kt + BN, std::integral_constant<int, 0>{});
        issue_v(kt + BN, std::integral_constant<int, 0>{});
      } else {
        issue_k(kt + BN, std::integral_constant<int, 1>{});
        issue_v(kt + BN, std::integral_constant<int, 1>{});
      }
    }
    if (wave_sees(t)) {
      f32x16 sc[R][2];
      {
        const char *kb = k_rt(buf) + kread;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
          for (int r = 0; r < R; ++r) sc[r][nb] = (f32x16)(0.0f);
#pragma unroll
          for (int kk = 0; kk < KST; ++kk) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kb + nb * 32 * L::ROWB + kk * 32);
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
      softmax(sc, pf);
      {
        const char *vb = v_rt(buf) + vread;
#pragma unroll
        for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const char *vp = vb + ks * 16 * L::ROWB + db * 64;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vp));
            const i16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vp + 2 * L::ROWB));
            const bf16x8 vf = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
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
    const int kt = kv_lo + t * BN;
    // the last tile's "next" loads are empty (range starts at kv_hi)
    const int kn = min(kt + BN, kv_hi);
    issue_k(kn, std::integral_constant<int, BUF ^ 1>{});
    issue_v(kn, std::integral_constant<int, BUF ^ 1>{});
    f32x16 sc[R][2];
    bf16x8 pf[R][BN / 16];
    qk(buf_tag, sc);
    softmax(sc, pf);
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
      const int kt = kv_lo + t * BN;
      issue_k(min(kt + BN, kv_hi), std::integral_constant<int, BUF ^ 1>{});
      if (wave_sees(t)) {
        f32x16 sc[R][2];
        qk(buf_tag, sc);
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
    bool bad = false;
    if (wave_active) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float l_tot = l_run[r] + xor32(l_run[r]);
        bad = bad || (row_ok[r] && !__builtin_isfinite(l_tot));
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            bad = bad || (row_ok[r] && 32 * db + 8 * (j >> 2) + 4 * g + (j & 3) < D &&
                          !__builtin_isfinite(o[r][db][j]));
      }
    }
    if (!__syncthreads_or(bad)) break;
    reset();
    max_sweep();
  }

  if (wave_active) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float l_tot = l_run[r] + xor32(l_run[r]);
      if (row_ok[r]) {
        const float inv = 1.0f / l_tot;
        if (a.lse != nullptr && g == 0)
          a.lse[(size_t)(s0q + row[r]) * a.hq + h] = (m_ref[r] + log2f(l_tot)) * kLn2;
        __bf16 *orow = reinterpret_cast<__bf16 *>(a.out) + ((size_t)(s0q + row[r]) * a.hq + h) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int d = 32 * db + 8 * jj + 4 * g;
            if (d >= D) continue;  // padding rows of O^T
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[r][db][4 * jj + e] * inv);
            *reinterpret_cast<bf16x4 *>(orow + d) = w;
          }
      }
    }
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
  return static_cast<int>(hipLaunchKernel(reinterpret_cast<const void *>(kernel),
                                          dim3(a.total_items), dim3(threads), args, 0,
                                          static_cast<hipStream_t>(stream)));
}

constexpr int kWavesBf16 = 4;

}  // namespace

int rows_per_workgroup_bf16(int) { return kWavesBf16 * 32; }
int rows_per_workgroup_f32(int) { return 128; }

int launch_bf16(const LaunchArgs &a, int head_dim, void *stream) {
  switch (head_dim) {
    case 64: return launch(fwd_bf16_fast<64, kWavesBf16, 1>, a, kWavesBf16 * 64, stream);
    case 72: return launch(fwd_bf16_fast<72, kWavesBf16, 1>, a, kWavesBf16 * 64, stream);
    case 128: return launch(fwd_bf16_fast<128, kWavesBf16, 1>, a, kWavesBf16 * 64, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
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
