// gdn_fwd.hip -- chunked gated-delta-rule prefill for gfx950 (MI355X).
//
// The recurrence (per sequence and head, state S [d_v][d_k], alpha = exp(g))
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//     o_t = S_t (scale q_t)
// is the gated delta rule of the hybrid gated-delta-net backbone in the paper
// "A Modern Multimodal Assistant on a 6 GB 2011 GPU" (abstract; gist.science
// technical summary, Metodologia), whose prefill replaces the token scan by a
// chunked intra-/inter-chunk form (abstract, result (i); summary, Metodologia,
// recurrent layers).  Within a chunk of 64 tokens, with cumulative log-gates
// gam_i and Gam_i = exp(gam_i), unrolling the recurrence gives
//     A_ij = beta_i (Gam_i / Gam_j) k_i . k_j  (i > j),   T = (I + A)^-1,
//     W = T diag(beta Gam) K,   U = T diag(beta) V,   U' = U - W S^T,
//     O = diag(Gam) Q' S^T + (Q' K^T o M) U',   M_ij = Gam_i / Gam_j (i >= j),
//     S <- Gam_last S + U'^T diag(Gam_last / Gam) K,
// with Q' = scale Q and S the state entering the chunk.  Everything but the
// last three lines is independent of S, so:
//
//   gdn_prep  (one workgroup per chunk and head, all in parallel): loads the
//             chunk's K, Q, V, g, beta; cumulative gates by a wave scan;
//             K K^T and Q K^T on MFMA; A and the masked, gated scores P;
//             T by blocked forward substitution (16 x 16 diagonal blocks by
//             rows, the off-diagonal blocks by distance from the diagonal on
//             fp32 MFMA); W and U on MFMA; stores W, U, P,
//             K^T diag(Gam_last / Gam), Gam and a copy of Q in the
//             workspace, in the order the scan reads them as MFMA operands.
//   gdn_scan  (one workgroup per sequence, head and 32 state rows): carries
//             its 32 x 128 slice of S in fp32 MFMA accumulators through the
//             sequence's chunks in order; per chunk U' = U - W S^T and
//             Q S^T (MFMA), O = diag(scale Gam) Q S^T + P U' (MFMA), then
//             S <- Gam_last S + Kd U' (MFMA).  Each wave loads its own
//             operands of a chunk straight into registers a few chunks
//             ahead; the four slices of a (sequence, head) run on one XCD.
//             Eight waves split the chunk step by role (see gdn_scan).
//
// MFMA operands are bf16 (the state is rounded to bf16 for each product and
// kept in fp32 between chunks); accumulation is fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

using attn::bf16x2;
using attn::bf16x4;
using attn::bf16x8;
using attn::f32x16;
using attn::f32x4;

constexpr int C = kChunk;
constexpr int DK = kDk;
constexpr int DV = kDv;
constexpr int RB = DK + 8;  // bf16 row stride of [*][128] LDS tiles (272 bytes: 17 16-byte slots)
constexpr int RT = C + 8;   // bf16 row stride of [*][64] LDS tiles (144 bytes: 9 slots)

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of a 32 x 32 MFMA accumulator held in element e by a lane of half g.
__device__ __forceinline__ int acc_row(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }

// Workspace order of element (r, c) of a row-major bf16 matrix with
// 16 * ksteps columns: the order in which a wave reads it as the A (or B)
// operand of 32 x 32 x 16 MFMAs -- 32-row blocks, then 16-column steps, then
// the 64 lanes (lane = 32 * (8-column half) + row in the block), 8 columns per
// lane -- so each 64-lane load of 16 bytes reads 1 KB of consecutive bytes.
__device__ __forceinline__ int frag_index(int r, int c, int ksteps) {
  return ((((r >> 5) * ksteps + (c >> 4)) * 64 + ((c >> 3) & 1) * 32 + (r & 31)) << 3) + (c & 7);
}

// Workspace order of U^T (value dim v, token t): what the scan's lane
// (v % 32, half h) needs for U' = U - W S^T of the 32-token block holding t
// is the accumulator rows 8j + 4h + i (j, i < 4) of that block, so per
// (32-dim slice, token block) the lane's 16 tokens are two 16-byte loads, in
// two halves of 64 lanes x 8.
__device__ __forceinline__ int u_frag_index(int v, int t) {
  const int tt = t & 31;
  return (((((v >> 5) * 2 + (t >> 5)) * 2 + (tt >> 4)) * 64 + ((tt >> 2) & 1) * 32 + (v & 31)) << 3) +
         ((tt >> 3) & 1) * 4 + (tt & 3);
}

// Launch-local chunk index -> sequence.
__device__ __forceinline__ int seq_of_chunk(const GdnArgs &a, int cg) {
  int b = 0;
  while (b + 1 < a.n_seqs && a.chunk_start[b + 1] <= cg) ++b;
  return b;
}

// LDS of gdn_prep, one byte array in four regions reused across phases:
//   R0  K rows [64][RB] bf16                         (whole kernel)
//   R1  V rows [64][RB] bf16                         (whole kernel)
//   R2  Q rows [64][RB] bf16  -> T [64][RF4] fp32     (scores, then the inverse)
//   R3  A [64][RF4] fp32 + Y                          (the inverse)
//       -> T diag(beta Gam), T diag(beta) [64][RT] bf16  (the WY products)
constexpr int RF4 = C + 4;  // fp32 row stride of the 64 x 64 systems (16-byte aligned rows)
constexpr int kR0 = 0;
constexpr int kR1 = kR0 + C * RB * 2;
constexpr int kR2 = kR1 + C * RB * 2;
constexpr int kR3 = kR2 + C * RB * 2;
constexpr int kYFloats = 16 * (16 + 32 + 48);  // T_ii A[block i][blocks < i], i = 1..3
constexpr int kR3Bytes = C * RF4 * 4 + kYFloats * 4;
constexpr int kPrepLds = kR3 + kR3Bytes;
static_assert(C * RF4 * 4 <= C * RB * 2, "T fits where Q was");
static_assert(2 * C * RT * 2 <= kR3Bytes, "both scaled T copies fit where A was");
static_assert(kPrepLds <= 80 * 1024, "two workgroups per CU");

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__global__ __launch_bounds__(256, 2) void gdn_prep(const GdnArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kPrepLds];
  __shared__ __attribute__((aligned(16))) float gam_s[C];
  __shared__ float beta_s[C], big_s[C], fd_s[C];
  __bf16 *kl = reinterpret_cast<__bf16 *>(lds + kR0);
  __bf16 *vl = reinterpret_cast<__bf16 *>(lds + kR1);
  __bf16 *ql = reinterpret_cast<__bf16 *>(lds + kR2);
  float *tf = reinterpret_cast<float *>(lds + kR2);
  float *af = reinterpret_cast<float *>(lds + kR3);
  float *yf = af + C * RF4;
  __bf16 *tbk = reinterpret_cast<__bf16 *>(lds + kR3);
  __bf16 *tbv = tbk + C * RT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int item = blockIdx.x;
  const int h = item % a.h;
  const int cg = item / a.h;
  const int b = seq_of_chunk(a, cg);
  const int c = cg - a.chunk_start[b];
  const int t0 = a.seq_start[b] + c * C;
  const int n = min(C, a.seq_len[b] - c * C);  // >= 1: sequences without tokens have no chunks

  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k);
  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q);
  const __bf16 *V = reinterpret_cast<const __bf16 *>(a.v);
  __bf16 *w_out = reinterpret_cast<__bf16 *>(a.ws_w) + (size_t)item * C * DK;
  __bf16 *u_out = reinterpret_cast<__bf16 *>(a.ws_u) + (size_t)item * C * DV;
  __bf16 *p_out = reinterpret_cast<__bf16 *>(a.ws_p) + (size_t)item * C * C;
  __bf16 *kd_out = reinterpret_cast<__bf16 *>(a.ws_kd) + (size_t)item * DK * C;
  __bf16 *q_out = reinterpret_cast<__bf16 *>(a.ws_q) + (size_t)item * C * DK;
  float *gam_out = a.ws_gam + (size_t)item * C;

  // K, Q, V rows of the chunk (rows past its end are zero), gates, betas.
  // Every load is issued before any is used (rows past the end load the
  // last row and are replaced by zeros), so the item pays one memory
  // latency here, not one per row group.
  const bf16x8 zero8 = (bf16x8)((__bf16)0.0f);
  constexpr int kRowLoads = C * (DK / 8) / 256;  // 16-byte pieces per thread and matrix
  bf16x8 kv[kRowLoads], qv[kRowLoads], vv[kRowLoads];
#pragma unroll
  for (int it = 0; it < kRowLoads; ++it) {
    const int idx = tid + 256 * it;
    const int r = idx >> 4, cc = idx & 15;
    const size_t row = (size_t)(t0 + min(r, n - 1)) * a.h + h;
    kv[it] = *reinterpret_cast<const bf16x8 *>(K + row * DK + cc * 8);
    qv[it] = *reinterpret_cast<const bf16x8 *>(Q + row * DK + cc * 8);
    vv[it] = *reinterpret_cast<const bf16x8 *>(V + row * DV + cc * 8);
  }
  float gx = 0.0f, gb = 0.0f;
  if (wave == 0) {
    const size_t th = (size_t)(t0 + min(lane, n - 1)) * a.h + h;
    gx = a.g[th];
    gb = a.beta[th];
  }
  // (stored unconditionally, then overwritten past the end: a select here
  // lets the compiler move loads into a branch and wait inside it)
#pragma unroll
  for (int it = 0; it < kRowLoads; ++it) {
    const int idx = tid + 256 * it;
    const int r = idx >> 4, cc = idx & 15;
    *reinterpret_cast<bf16x8 *>(kl + r * RB + cc * 8) = kv[it];
    *reinterpret_cast<bf16x8 *>(ql + r * RB + cc * 8) = qv[it];
    *reinterpret_cast<bf16x8 *>(vl + r * RB + cc * 8) = vv[it];
    if (r >= n) {
      *reinterpret_cast<bf16x8 *>(kl + r * RB + cc * 8) = zero8;
      *reinterpret_cast<bf16x8 *>(ql + r * RB + cc * 8) = zero8;
      *reinterpret_cast<bf16x8 *>(vl + r * RB + cc * 8) = zero8;
    }
  }
  if (wave == 0) {
    // inclusive scan of the log-gates over the chunk (padding adds 0), kept
    // in log2 units so every decay below is one exp2
    float x = lane < n ? gx * kLog2e : 0.0f;
    const float bt = lane < n ? gb : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    const float last = __shfl(x, 63);
    gam_s[lane] = x;
    beta_s[lane] = bt;
    const float G = exp2_fast(x);
    big_s[lane] = G;
    fd_s[lane] = exp2_fast(last - x);  // Gam_last / Gam_m <= 1
    gam_out[lane] = G;
  }
  __syncthreads();

  // the queries again, in the scan's operand order: 16-byte piece pc of the
  // copy is row 32 (pc >> 9) + (pc & 31), columns 16 ((pc >> 6) & 7) +
  // 8 ((pc >> 5) & 1) .. +7 (frag_index)
  for (int pc = tid; pc < C * DK / 8; pc += 256) {
    const int r = 32 * (pc >> 9) + (pc & 31), c0 = 16 * ((pc >> 6) & 7) + 8 * ((pc >> 5) & 1);
    *reinterpret_cast<bf16x8 *>(q_out + 8 * pc) = *reinterpret_cast<const bf16x8 *>(ql + r * RB + c0);
  }

  // K K^T and Q K^T: wave w -> 32 x 32 block (w >> 1, w & 1); block (0, 1)
  // lies above the diagonal, where both A and P are zero.
  {
    const int bi = wave >> 1, bj = wave & 1;
    f32x16 kk = (f32x16)(0.0f), qk = (f32x16)(0.0f);
    if (bi >= bj) {
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(kl + (32 * bi + l32) * RB + 16 * ks + 8 * g);
        const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(ql + (32 * bi + l32) * RB + 16 * ks + 8 * g);
        const bf16x8 bk = *reinterpret_cast<const bf16x8 *>(kl + (32 * bj + l32) * RB + 16 * ks + 8 * g);
        // transposed products: the lane's column is row i of the block
        kk = mfma(bk, ak, kk);
        qk = mfma(bk, aq, qk);
      }
    }
    // entry 4 jj + e of lane (l32, g): i = 32 bi + l32, j = 32 bj + 8 jj + 4 g + e,
    // so each lane writes rows of four consecutive j (16-byte A rows in LDS,
    // 8-byte pieces of P that a wave's store lays down as 512 contiguous bytes)
    const int i = 32 * bi + l32;
    const float gi = gam_s[i], bti = beta_s[i];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j0 = 32 * bj + 8 * jj + 4 * g;
      f32x4 arow = (f32x4)(0.0f);
      bf16x4 prow = (bf16x4)((__bf16)0.0f);
      if (bi >= bj) {  // the block above the diagonal is zero
        const f32x4 gj = *reinterpret_cast<const f32x4 *>(&gam_s[j0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + e;
          const float dec = i >= j ? exp2_fast(gi - gj[e]) : 0.0f;  // Gam_i / Gam_j <= 1 for i >= j
          arow[e] = i > j ? bti * dec * kk[4 * jj + e] : 0.0f;
          prow[e] = (__bf16)(a.scale * dec * qk[4 * jj + e]);
        }
      }
      *reinterpret_cast<f32x4 *>(af + i * RF4 + j0) = arow;
      *reinterpret_cast<bf16x4 *>(p_out + frag_index(i, j0, C / 16)) = prow;
    }
  }
  __syncthreads();  // Q is no longer read: its region takes T

  // T = (I + A)^-1, A strictly lower.  Diagonal 16 x 16 blocks: wave w
  // inverts block w, lane c < 16 computing column c row by row.  T above the
  // block diagonal is never stored: the bf16 copies below write its zeros.
  if (lane < 16) {
    const int base = 16 * wave, cc = lane;
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float arow[16];
#pragma unroll
      for (int j = 0; j < i; ++j) arow[j] = af[(base + i) * RF4 + base + j];
      float s = (i == cc) ? 1.0f : 0.0f;
#pragma unroll
      for (int j = 0; j < i; ++j) s -= arow[j] * col[j];
      col[i] = (i >= cc) ? s : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) tf[(base + i) * RF4 + base + cc] = col[i];
  }
  __syncthreads();
  // The rest of T by blocks, on fp32 MFMA (16 x 16 x 4: lane l supplies
  // A[l % 16][l / 16] and B[l / 16][l % 16] of a k step and holds
  // D[4 (l / 16) + e][l % 16]).  First Y_i = T_ii A[block i][columns < 16 i]
  // for i = 1..3 (16 x 16i each, row stride 16i, at yf + 128 i (i - 1)):
  // six 16 x 16 blocks (i, c), wave w taking blocks w and w + 4.
  const int rr = lane & 15, kq = lane >> 4;
  for (int b6 = wave; b6 < 6; b6 += 4) {
    const int i = b6 < 1 ? 1 : (b6 < 3 ? 2 : 3), c = b6 - i * (i - 1) / 2;
    f32x4 acc = (f32x4)(0.0f);
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(tf[(16 * i + rr) * RF4 + 16 * i + k0 + kq],
                                                 af[(16 * i + k0 + kq) * RF4 + 16 * c + rr], acc, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) yf[128 * i * (i - 1) + (4 * kq + e) * (16 * i) + 16 * c + rr] = acc[e];
  }
  __syncthreads();
  // Off-diagonal blocks by distance d: T_ij = -Y_i[:, 16j .. 16i) T[16j .. 16i, block j];
  // wave w < 4 - d takes block (j = w, i = w + d), K = 16 d.
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (wave < 4 - d) {
      const int bj = wave, bi = bj + d;
      const float *yrow = yf + 128 * bi * (bi - 1) + rr * (16 * bi) + 16 * bj;
      f32x4 acc = (f32x4)(0.0f);
#pragma unroll
      for (int k0 = 0; k0 < 16 * d; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(yrow[k0 + kq], tf[(16 * bj + k0 + kq) * RF4 + 16 * bj + rr], acc,
                                                   0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) tf[(16 * bi + 4 * kq + e) * RF4 + 16 * bj + rr] = -acc[e];
    }
    __syncthreads();
  }

  // bf16 T diag(beta Gam) and T diag(beta) (A and Y are no longer needed);
  // T is zero right of the block diagonal
  for (int idx = tid; idx < C * C / 4; idx += 256) {
    const int r = idx >> 4, cq = idx & 15;
    const f32x4 t = cq < 4 * ((r >> 4) + 1) ? *reinterpret_cast<const f32x4 *>(tf + r * RF4 + 4 * cq) : (f32x4)(0.0f);
    bf16x4 xk, xv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * cq + e;
      xk[e] = (__bf16)(t[e] * beta_s[m] * big_s[m]);
      xv[e] = (__bf16)(t[e] * beta_s[m]);
    }
    *reinterpret_cast<bf16x4 *>(tbk + r * RT + 4 * cq) = xk;
    *reinterpret_cast<bf16x4 *>(tbv + r * RT + 4 * cq) = xv;
  }
  // K^T diag(Gam_last / Gam) to the workspace, one 16-byte piece of its
  // operand order per task, consecutive tasks on consecutive pieces
  // (frag_index): key dim 32 (task >> 8) + (task & 31), tokens
  // 16 ((task >> 6) & 3) + 8 ((task >> 5) & 1) .. +7
  for (int task = tid; task < DK * (C / 8); task += 256) {
    const int k = 32 * (task >> 8) + (task & 31), m0 = 16 * ((task >> 6) & 3) + 8 * ((task >> 5) & 1);
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (__bf16)(fd_s[m0 + e] * (float)kl[(m0 + e) * RB + k]);
    *reinterpret_cast<bf16x8 *>(kd_out + 8 * task) = x;
  }
  __syncthreads();

  // W = (T diag(beta Gam)) K, U = (T diag(beta)) V: wave w -> columns
  // 32w .. 32w+31 of both, all 64 rows; K and V are read down their columns
  // (W computed transposed, so its rows leave as 8-byte pieces).
  {
    f32x16 wacc[2] = {(f32x16)(0.0f), (f32x16)(0.0f)};
    f32x16 uacc[2] = {(f32x16)(0.0f), (f32x16)(0.0f)};
    const int col = 32 * wave + l32;
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      bf16x8 bw, bu;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bw[e] = kl[(16 * ks + 8 * g + e) * RB + col];
        bu[e] = vl[(16 * ks + 8 * g + e) * RB + col];
      }
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        // W transposed: the lane's column is token 32 ib + l32
        wacc[ib] = mfma(bw, *reinterpret_cast<const bf16x8 *>(tbk + (32 * ib + l32) * RT + 16 * ks + 8 * g), wacc[ib]);
        uacc[ib] = mfma(*reinterpret_cast<const bf16x8 *>(tbv + (32 * ib + l32) * RT + 16 * ks + 8 * g), bu, uacc[ib]);
      }
    }
    // W: the lane holds token 32 ib + l32, key dims 32 wave + 8 jj + 4 g .. +3
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (__bf16)wacc[ib][4 * jj + e];
        *reinterpret_cast<bf16x4 *>(w_out + frag_index(32 * ib + l32, 32 * wave + 8 * jj + 4 * g, DK / 16)) = x;
      }
    // U transposed, [v][t]: four consecutive tokens per store
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (__bf16)uacc[ib][4 * q4 + e];
        *reinterpret_cast<bf16x4 *>(u_out + u_frag_index(col, 32 * ib + 8 * q4 + 4 * g)) = x;
      }
  }
}

// Eight waves per workgroup (two per SIMD, so one hides the other's
// latencies), each with one role per chunk step:
//   waves 0, 1  X = W S^T for token block 32w .. (8 MFMAs), then U' = U - X
//               into LDS: the chain the next chunk depends on
//   waves 2, 3  Y^T = S Q^T for token block 32(w-2) .., then after U' is
//               ready O^T = diag(scale Gam) Y^T + U'^T P^T and the output
//               store (each lane holds four consecutive value dims of one
//               token: 8-byte row pieces straight from the accumulator)
//   waves 4..7  after U' is ready S^T[32(w-4) ..] <- Gam_last S^T + Kd U'.
// Every workspace row of a chunk is an MFMA operand of exactly one wave, so
// each wave loads its own operands from global memory straight into
// registers, in the half of the step where its role leaves it idle: kDepth
// chunks ahead for waves 0..3, kDepth - 1 for the state waves (a ring of
// register sets, the step loop unrolled by kDepth so every set is named
// statically); LDS holds only what
// waves exchange: the bf16 state S and U'.  Each role runs its own loop; all
// of them pass the same barriers (one before the first chunk, two per chunk).
constexpr int kScanWaves = 8;
constexpr int kDepth = 3;

struct XRegs {      // waves 0, 1: W rows of the token block, U^T pieces
  bf16x8 w[DK / 16];
  bf16x8 u[2];
};
struct YRegs {      // waves 2, 3: query rows and P rows of the token block, Gam
  bf16x8 q[DK / 16];
  bf16x8 p[C / 16];
  float gam;
};
struct SRegs {      // waves 4..7: Kd rows of the key block, Gam_last
  bf16x8 kd[C / 16];
  float glast;
};

// Runs step(c, r[c % kDepth], r[(c - 1) % kDepth]) for c = 0 .. nchunks-1:
// the set holding chunk c, and the one chunk c - 1 used (free again).  The
// main loop takes whole groups of kDepth chunks with no early exit, so at
// its head the loads in flight are always the same (the register sets in
// issue order) and the compiler waits for the oldest set only; the last
// nchunks % kDepth steps follow in a guarded tail.
template <typename R, typename F>
__device__ __forceinline__ void run_chunks(int nchunks, R (&r)[kDepth], F &&step) {
  int c = 0;
  for (; c + kDepth <= nchunks; c += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) step(c + d, r[d], r[(d + kDepth - 1) % kDepth]);
  }
#pragma unroll
  for (int d = 0; d < kDepth - 1; ++d)
    if (c + d < nchunks) step(c + d, r[d], r[(d + kDepth - 1) % kDepth]);
}

// The compiler chains the three role branches through shared join blocks,
// so loads a role leaves in flight when it ends would count, for its wait
// counts, against the next role's loop.  Each role ends with none in flight
// (its last loads are operands past the end, never used), which costs
// nothing: the wave has no work left.
__device__ __forceinline__ void drain_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

__global__ __launch_bounds__(kScanWaves * 64, 1) void gdn_scan(const GdnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 sb[kSliceRows * RB];   // S rows [v][k], bf16
  __shared__ __attribute__((aligned(16))) __bf16 upt[kSliceRows * RT];  // U'^T rows [v][t], bf16

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform, and known to be: the roles below are then plain branches,
  // not one exec-masked path through all three (whose loads the compiler
  // would then wait for in every role)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // Workgroup -> (pair = sequence x head, slice of 32 value dims).
  // Consecutive workgroups go to the eight XCDs in turn, so the four slices
  // of a pair are placed eight apart: they run on one XCD and share the
  // chunk rows in its L2.
  constexpr int SLICES = DV / kSliceRows;
  const int xcd = blockIdx.x & 7;
  const int j8 = blockIdx.x >> 3;
  const int pair = xcd + 8 * (j8 / SLICES);
  const int s = j8 % SLICES;
  if (pair >= a.n_seqs * a.h) return;  // grid padding; whole workgroup, before any barrier
  const int h = pair % a.h;
  const int b = pair / a.h;
  const int nchunks = a.chunk_start[b + 1] - a.chunk_start[b];
  const int seq_len = a.seq_len[b];
  const int seq0 = a.seq_start[b];
  const int v0 = kSliceRows * s;
  const size_t state_off = ((size_t)(a.seq_base + b) * a.h + h) * DV * DK;
  const int tb = 32 * (wave & 1);  // token block of X / Y / O
  auto item_of = [&](int c) { return (size_t)(a.chunk_start[b] + c) * a.h + h; };

  // B operand of X and A operand of Y^T: the bf16 state rows [v][k]
  auto load_state_rows = [&](bf16x8 (&bv)[DK / 16]) {
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks)
      bv[ks] = *reinterpret_cast<const bf16x8 *>(&sb[l32 * RB + 16 * ks + 8 * g]);
  };
  // A or B operand over the chunk's tokens: U'^T rows [v][t]
  auto load_upt = [&](bf16x8 (&bu)[C / 16]) {
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks)
      bu[ks] = *reinterpret_cast<const bf16x8 *>(&upt[l32 * RT + 16 * ks + 8 * g]);
  };

  if (wave < 2) {
    // ---- X waves: U' = U - W S^T ----
    auto load = [&](int c, XRegs &r) {
      const size_t item = item_of(c);
      // (frag_index and u_frag_index: this lane's pieces are 1 KB apart)
      const __bf16 *w = reinterpret_cast<const __bf16 *>(a.ws_w) + item * C * DK + frag_index(tb, 8 * g, DK / 16) + 8 * l32;
      const __bf16 *u = reinterpret_cast<const __bf16 *>(a.ws_u) + item * C * DV + u_frag_index(v0 + l32, tb + 4 * g);
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) r.u[j2] = *reinterpret_cast<const bf16x8 *>(u + 512 * j2);
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) r.w[ks] = *reinterpret_cast<const bf16x8 *>(w + 512 * ks);
    };
    auto step = [&](int c, XRegs &r, XRegs &) __attribute__((always_inline)) {
      bf16x8 bv[DK / 16];
      load_state_rows(bv);
      f32x16 x = (f32x16)(0.0f);
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) x = mfma(r.w[ks], bv[ks], x);
      // U' = U - X, stored transposed [v][t] in bf16
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 up;
#pragma unroll
        for (int e = 0; e < 4; ++e) up[e] = (__bf16)((float)r.u[j >> 1][4 * (j & 1) + e] - x[4 * j + e]);
        *reinterpret_cast<bf16x4 *>(&upt[l32 * RT + tb + 8 * j + 4 * g]) = up;
      }
      __syncthreads();  // U' ready; every read of sb done
      // operands of the chunk kDepth ahead, in the half of the step where
      // this wave has nothing else to do (past the end: the last chunk
      // again, never used; unconditional, so the loads in flight are counted
      // exactly)
      load(min(c + kDepth, nchunks - 1), r);
      __syncthreads();  // the new state ready
    };
    XRegs r[kDepth];
    if (nchunks > 0) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) load(min(d, nchunks - 1), r[d]);
    }
    __syncthreads();  // initial state in sb
    run_chunks(nchunks, r, step);
    drain_loads();
  } else if (wave < 4) {
    // ---- Y waves: O^T = diag(scale Gam) S Q^T + U'^T P^T ----
    auto load_q = [&](int c, YRegs &r) {
      // the prep's copy of the chunk's queries (rows past its end are zero:
      // they only feed output columns that are never stored)
      const __bf16 *q = reinterpret_cast<const __bf16 *>(a.ws_q) + item_of(c) * C * DK + frag_index(tb, 8 * g, DK / 16) + 8 * l32;
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) r.q[ks] = *reinterpret_cast<const bf16x8 *>(q + 512 * ks);
    };
    auto load_p = [&](int c, YRegs &r) {
      const size_t item = item_of(c);
      const __bf16 *p = reinterpret_cast<const __bf16 *>(a.ws_p) + item * C * C + frag_index(tb, 8 * g, C / 16) + 8 * l32;
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) r.p[ks] = *reinterpret_cast<const bf16x8 *>(p + 512 * ks);
      r.gam = a.ws_gam[item * C + tb + l32];
    };
    __bf16 *orow = reinterpret_cast<__bf16 *>(a.out);
    auto step = [&](int c, YRegs &r, YRegs &) __attribute__((always_inline)) {
      const int cn = min(c + kDepth, nchunks - 1);
      bf16x8 bv[DK / 16];
      load_state_rows(bv);
      f32x16 y = (f32x16)(0.0f);
#pragma unroll
      for (int ks = 0; ks < DK / 16; ++ks) y = mfma(bv[ks], r.q[ks], y);
      load_q(cn, r);
      __syncthreads();  // U' ready; every read of sb done
      const float sg = a.scale * r.gam;
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] *= sg;
      bf16x8 bu[C / 16];
      load_upt(bu);
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) y = mfma(bu[ks], r.p[ks], y);
      load_p(cn, r);
      // lane: token tb + l32, value dims v0 + 8j + 4g .. +3
      const int t0 = seq0 + c * C;
      const int n = min(C, seq_len - c * C);
      if (tb + l32 < n) {
        __bf16 *o = orow + ((size_t)(t0 + tb + l32) * a.h + h) * DV + v0 + 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (__bf16)y[4 * j + e];
          *reinterpret_cast<bf16x4 *>(o + 8 * j) = x;
        }
      }
      __syncthreads();  // the new state ready
    };
    YRegs r[kDepth];
    if (nchunks > 0) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        load_q(min(d, nchunks - 1), r[d]);
        load_p(min(d, nchunks - 1), r[d]);
      }
    }
    __syncthreads();  // initial state in sb
    run_chunks(nchunks, r, step);
    drain_loads();
  } else {
    // ---- state waves: S^T[kb ..] <- Gam_last S^T + Kd U' ----
    const int kb = 32 * (wave - 4);  // key rows of the state
    f32x16 st = (f32x16)(0.0f);      // S^T[kb + row][v0 + l32]
    if (a.s0 != nullptr) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(a.s0 + state_off + (size_t)(v0 + l32) * DK + kb +
                                                         8 * q4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) st[4 * q4 + e] = x[e];
      }
    }
    // bf16 copy of the state as S rows [v][k]
    auto store_state = [&]() {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (__bf16)st[4 * q4 + e];
        *reinterpret_cast<bf16x4 *>(&sb[l32 * RB + kb + 8 * q4 + 4 * g]) = x;
      }
    };
    auto load = [&](int c, SRegs &r) {
      const size_t item = item_of(c);
      const __bf16 *kd = reinterpret_cast<const __bf16 *>(a.ws_kd) + item * DK * C + frag_index(kb, 8 * g, C / 16) + 8 * l32;
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) r.kd[ks] = *reinterpret_cast<const bf16x8 *>(kd + 512 * ks);
      r.glast = a.ws_gam[item * C + C - 1];
    };
    auto step = [&](int c, SRegs &r, SRegs &free_set) __attribute__((always_inline)) {
      // the chunk kDepth - 1 ahead into the set chunk c - 1 used, in the
      // half of the step where this wave waits anyway
      load(min(c + kDepth - 1, nchunks - 1), free_set);
      __syncthreads();  // U' ready; every read of sb done
      bf16x8 bu[C / 16];
      load_upt(bu);
#pragma unroll
      for (int e = 0; e < 16; ++e) st[e] *= r.glast;
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) st = mfma(r.kd[ks], bu[ks], st);
      store_state();
      __syncthreads();  // the new state ready
    };
    store_state();
    SRegs r[kDepth];
    if (nchunks > 0) {
#pragma unroll
      for (int d = 0; d < kDepth - 1; ++d) load(min(d, nchunks - 1), r[d]);
    }
    __syncthreads();  // initial state in sb
    run_chunks(nchunks, r, step);
    drain_loads();
    if (a.s_final != nullptr) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = st[4 * q4 + e];
        *reinterpret_cast<f32x4 *>(a.s_final + state_off + (size_t)(v0 + l32) * DK + kb + 8 * q4 + 4 * g) = x;
      }
    }
  }
}

}  // namespace

int launch_gdn(const GdnArgs &a, void *stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void *args[] = {const_cast<GdnArgs *>(&a)};
  hipError_t e = hipSuccess;
  if (a.total_items > 0)
    e = hipLaunchKernel(reinterpret_cast<const void *>(gdn_prep), dim3(a.total_items), dim3(256), args, 0, st);
  if (e == hipSuccess && a.n_seqs > 0)
    // pairs rounded up to a multiple of 8 (see gdn_scan's workgroup map)
    e = hipLaunchKernel(reinterpret_cast<const void *>(gdn_scan),
                        dim3((a.n_seqs * a.h + 7) / 8 * 8 * (kDv / kSliceRows)), dim3(kScanWaves * 64), args, 0,
                        st);
  return static_cast<int>(e);
}

}  // namespace gdn
