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
//             rows, off-diagonal blocks by distance from the diagonal, fp32);
//             W and U on MFMA; stores W, U, P, K^T diag(Gam_last / Gam) and
//             Gam in the workspace.
//   gdn_scan  (one workgroup per sequence, head and 32 state rows): carries
//             its 32 x 128 slice of S in fp32 MFMA accumulators through the
//             sequence's chunks in order; per chunk U' = U - W S^T and
//             Q S^T (MFMA), O = diag(scale Gam) Q S^T + P U' (MFMA), then
//             S <- Gam_last S + Kd U' (MFMA).  The next chunk's workspace
//             rows are loaded into registers while the current one computes.
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
constexpr int RF = C + 1;   // fp32 row stride of the 64 x 64 systems
constexpr int RU = kSliceRows + 8;  // bf16 row stride of a chunk's U slice [64][32]

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of a 32 x 32 MFMA accumulator held in element e by a lane of half g.
__device__ __forceinline__ int acc_row(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }

// Launch-local chunk index -> sequence.
__device__ __forceinline__ int seq_of_chunk(const GdnArgs &a, int cg) {
  int b = 0;
  while (b + 1 < a.n_seqs && a.chunk_start[b + 1] <= cg) ++b;
  return b;
}

__global__ __launch_bounds__(256, 1) void gdn_prep(const GdnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 kl[C * RB];
  __shared__ __attribute__((aligned(16))) __bf16 ql[C * RB];   // Q; later K^T diag(Gam_last/Gam)
  __shared__ __attribute__((aligned(16))) __bf16 vl[C * RB];
  __shared__ float af[C * RF];
  __shared__ float tf[C * RF];
  __shared__ float xf[3 * 16 * 17];
  __shared__ __attribute__((aligned(16))) __bf16 tb[C * RT];
  __shared__ __attribute__((aligned(16))) __bf16 kts[DK * RT];  // (diag(beta Gam) K)^T
  __shared__ __attribute__((aligned(16))) __bf16 vts[DV * RT];  // (diag(beta) V)^T
  __shared__ float gam_s[C], beta_s[C], big_s[C];
  __bf16 *kdl = ql;  // Q is read only by the score products: its tile then holds [128][64]

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
  float *gam_out = a.ws_gam + (size_t)item * C;

  // K, Q, V rows of the chunk (rows past its end are zero), gates, betas
  const bf16x8 zero8 = (bf16x8)((__bf16)0.0f);
  for (int idx = tid; idx < C * (DK / 8); idx += 256) {
    const int r = idx >> 4, cc = idx & 15;
    bf16x8 kv = zero8, qv = zero8, vv = zero8;
    if (r < n) {
      const size_t row = (size_t)(t0 + r) * a.h + h;
      kv = *reinterpret_cast<const bf16x8 *>(K + row * DK + cc * 8);
      qv = *reinterpret_cast<const bf16x8 *>(Q + row * DK + cc * 8);
      vv = *reinterpret_cast<const bf16x8 *>(V + row * DV + cc * 8);
    }
    *reinterpret_cast<bf16x8 *>(kl + r * RB + cc * 8) = kv;
    *reinterpret_cast<bf16x8 *>(ql + r * RB + cc * 8) = qv;
    *reinterpret_cast<bf16x8 *>(vl + r * RB + cc * 8) = vv;
  }
  for (int idx = tid; idx < C * RF; idx += 256) tf[idx] = 0.0f;
  if (wave == 0) {
    // inclusive scan of the log-gates over the chunk (padding adds 0)
    float x = 0.0f, bt = 0.0f;
    if (lane < n) {
      const size_t th = (size_t)(t0 + lane) * a.h + h;
      x = a.g[th];
      bt = a.beta[th];
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    gam_s[lane] = x;
    beta_s[lane] = bt;
    const float G = expf(x);
    big_s[lane] = G;
    gam_out[lane] = G;
  }
  __syncthreads();

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
        kk = mfma(ak, bk, kk);
        qk = mfma(aq, bk, qk);
      }
    }
    const int j = 32 * bj + l32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = 32 * bi + acc_row(e, g);
      float av = 0.0f, pv = 0.0f;
      if (i >= j) {
        const float dec = expf(gam_s[i] - gam_s[j]);  // <= 1: gates are <= 1
        if (i > j) av = beta_s[i] * dec * kk[e];
        pv = a.scale * dec * qk[e];
      }
      af[i * RF + j] = av;
      p_out[i * C + j] = (__bf16)pv;
    }
  }
  __syncthreads();

  // T = (I + A)^-1, A strictly lower.  Diagonal 16 x 16 blocks first: wave w
  // inverts block w, lane c < 16 computing column c row by row.
  if (lane < 16) {
    const int base = 16 * wave, cc = lane;
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == cc) ? 1.0f : 0.0f;
#pragma unroll
      for (int j = 0; j < i; ++j) s -= af[(base + i) * RF + base + j] * col[j];
      col[i] = (i >= cc) ? s : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) tf[(base + i) * RF + base + cc] = col[i];
  }
  __syncthreads();
  // Off-diagonal blocks by distance d from the diagonal: for i = j + d,
  //   X = sum_{m in blocks j..i-1} A[i-block][m] T[m][j-block],  T_ij = -T_ii X.
  for (int d = 1; d < 4; ++d) {
    const int nb = 4 - d;
    for (int o = tid; o < nb * 256; o += 256) {
      const int bb = o >> 8, r = (o >> 4) & 15, cc = o & 15;
      const int bj = bb, bi = bb + d;
      float s = 0.0f;
      for (int m = 16 * bj; m < 16 * bi; ++m) s += af[(16 * bi + r) * RF + m] * tf[m * RF + 16 * bj + cc];
      xf[bb * 272 + r * 17 + cc] = s;
    }
    __syncthreads();
    for (int o = tid; o < nb * 256; o += 256) {
      const int bb = o >> 8, r = (o >> 4) & 15, cc = o & 15;
      const int bj = bb, bi = bb + d;
      float s = 0.0f;
#pragma unroll
      for (int m = 0; m < 16; ++m) s += tf[(16 * bi + r) * RF + 16 * bi + m] * xf[bb * 272 + m * 17 + cc];
      tf[(16 * bi + r) * RF + 16 * bj + cc] = -s;
    }
    __syncthreads();
  }

  // bf16 operands: T; (diag(beta Gam) K)^T, (diag(beta) V)^T and
  // K^T diag(Gam_last / Gam), each transposed to [dim][token].
  for (int idx = tid; idx < C * C; idx += 256) {
    const int r = idx >> 6, cc = idx & 63;
    tb[r * RT + cc] = (__bf16)tf[r * RF + cc];
  }
  {
    const float glast = gam_s[C - 1];  // padding repeats the last token's value
    for (int task = tid; task < (C / 2) * (DK / 8); task += 256) {
      const int m = 2 * (task >> 4), kc = task & 15;
      const bf16x8 k0 = *reinterpret_cast<const bf16x8 *>(kl + m * RB + 8 * kc);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8 *>(kl + (m + 1) * RB + 8 * kc);
      const bf16x8 v0 = *reinterpret_cast<const bf16x8 *>(vl + m * RB + 8 * kc);
      const bf16x8 v1 = *reinterpret_cast<const bf16x8 *>(vl + (m + 1) * RB + 8 * kc);
      const float fk0 = beta_s[m] * big_s[m], fk1 = beta_s[m + 1] * big_s[m + 1];
      const float fv0 = beta_s[m], fv1 = beta_s[m + 1];
      const float fd0 = expf(glast - gam_s[m]), fd1 = expf(glast - gam_s[m + 1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = 8 * kc + e;
        *reinterpret_cast<bf16x2 *>(kts + row * RT + m) =
            bf16x2{(__bf16)(fk0 * (float)k0[e]), (__bf16)(fk1 * (float)k1[e])};
        *reinterpret_cast<bf16x2 *>(vts + row * RT + m) =
            bf16x2{(__bf16)(fv0 * (float)v0[e]), (__bf16)(fv1 * (float)v1[e])};
        *reinterpret_cast<bf16x2 *>(kdl + row * C + m) =
            bf16x2{(__bf16)(fd0 * (float)k0[e]), (__bf16)(fd1 * (float)k1[e])};
      }
    }
  }
  __syncthreads();

  // K^T diag(Gam_last / Gam) to the workspace, 16 bytes at a time
  for (int idx = tid; idx < DK * (C / 8); idx += 256) {
    const int r = idx >> 3, cc = idx & 7;
    *reinterpret_cast<bf16x8 *>(kd_out + r * C + cc * 8) = *reinterpret_cast<const bf16x8 *>(kdl + r * C + cc * 8);
  }
  // W = T (diag(beta Gam) K), U = T (diag(beta) V): wave w -> columns
  // 32w .. 32w+31 of both, all 64 rows (two 32-row blocks).
  {
    f32x16 wacc[2] = {(f32x16)(0.0f), (f32x16)(0.0f)};
    f32x16 uacc[2] = {(f32x16)(0.0f), (f32x16)(0.0f)};
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      const bf16x8 bw = *reinterpret_cast<const bf16x8 *>(kts + (32 * wave + l32) * RT + 16 * ks + 8 * g);
      const bf16x8 bu = *reinterpret_cast<const bf16x8 *>(vts + (32 * wave + l32) * RT + 16 * ks + 8 * g);
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const bf16x8 at = *reinterpret_cast<const bf16x8 *>(tb + (32 * ib + l32) * RT + 16 * ks + 8 * g);
        wacc[ib] = mfma(at, bw, wacc[ib]);
        uacc[ib] = mfma(at, bu, uacc[ib]);
      }
    }
    const int col = 32 * wave + l32;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int i = 32 * ib + acc_row(e, g);
        w_out[i * DK + col] = (__bf16)wacc[ib][e];
        u_out[i * DV + col] = (__bf16)uacc[ib][e];
      }
  }
}

// Registers holding one chunk's workspace rows and queries on their way to LDS.
struct ChunkRegs {
  bf16x8 w[4], q[4], kd[4], p[2], u;
  float gam;
};

__global__ __launch_bounds__(256, 1) void gdn_scan(const GdnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 wl[2][C * RB];
  __shared__ __attribute__((aligned(16))) __bf16 qsl[2][C * RB];
  __shared__ __attribute__((aligned(16))) __bf16 pl[2][C * RT];
  __shared__ __attribute__((aligned(16))) __bf16 kdl[2][DK * RT];
  __shared__ __attribute__((aligned(16))) __bf16 ul[2][C * RU];
  __shared__ float gl[2][C];
  __shared__ __attribute__((aligned(16))) __bf16 sb[kSliceRows * RB];   // S rows [v][k], bf16
  __shared__ __attribute__((aligned(16))) __bf16 upt[kSliceRows * RT];  // U'^T [v][t], bf16

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  constexpr int SLICES = DV / kSliceRows;
  const int s = blockIdx.x % SLICES;
  const int bh = blockIdx.x / SLICES;
  const int h = bh % a.h;
  const int b = bh / a.h;
  const int nchunks = a.chunk_start[b + 1] - a.chunk_start[b];
  const int seq_len = a.seq_len[b];
  const int seq0 = a.seq_start[b];
  const size_t state_off = ((size_t)(a.seq_base + b) * a.h + h) * DV * DK;

  // State slice S^T[k][v], k = 32 wave + acc_row, v = 32 s + l32.
  f32x16 st = (f32x16)(0.0f);
  if (a.s0 != nullptr) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 x = *reinterpret_cast<const f32x4 *>(a.s0 + state_off + (size_t)(32 * s + l32) * DK +
                                                       32 * wave + 8 * q4 + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) st[4 * q4 + e] = x[e];
    }
  }

  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q);
  auto load_chunk = [&](int c, ChunkRegs &r) {
    const size_t item = (size_t)(a.chunk_start[b] + c) * a.h + h;
    const __bf16 *w = reinterpret_cast<const __bf16 *>(a.ws_w) + item * C * DK;
    const __bf16 *u = reinterpret_cast<const __bf16 *>(a.ws_u) + item * C * DV;
    const __bf16 *p = reinterpret_cast<const __bf16 *>(a.ws_p) + item * C * C;
    const __bf16 *kd = reinterpret_cast<const __bf16 *>(a.ws_kd) + item * DK * C;
    const int t0 = seq0 + c * C;
    const int n = min(C, seq_len - c * C);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx >> 4, cc = idx & 15;
      r.w[i] = *reinterpret_cast<const bf16x8 *>(w + row * DK + cc * 8);
      r.q[i] = row < n ? *reinterpret_cast<const bf16x8 *>(Q + ((size_t)(t0 + row) * a.h + h) * DK + cc * 8)
                       : (bf16x8)((__bf16)0.0f);
      const int krow = idx >> 3, kc = idx & 7;
      r.kd[i] = *reinterpret_cast<const bf16x8 *>(kd + krow * C + kc * 8);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      r.p[i] = *reinterpret_cast<const bf16x8 *>(p + (idx >> 3) * C + (idx & 7) * 8);
    }
    r.u = *reinterpret_cast<const bf16x8 *>(u + (tid >> 2) * DV + kSliceRows * s + (tid & 3) * 8);
    r.gam = tid < C ? a.ws_gam[item * C + tid] : 0.0f;
  };
  auto store_chunk = [&](int buf, const ChunkRegs &r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx >> 4, cc = idx & 15;
      *reinterpret_cast<bf16x8 *>(&wl[buf][row * RB + cc * 8]) = r.w[i];
      *reinterpret_cast<bf16x8 *>(&qsl[buf][row * RB + cc * 8]) = r.q[i];
      *reinterpret_cast<bf16x8 *>(&kdl[buf][(idx >> 3) * RT + (idx & 7) * 8]) = r.kd[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      *reinterpret_cast<bf16x8 *>(&pl[buf][(idx >> 3) * RT + (idx & 7) * 8]) = r.p[i];
    }
    *reinterpret_cast<bf16x8 *>(&ul[buf][(tid >> 2) * RU + (tid & 3) * 8]) = r.u;
    if (tid < C) gl[buf][tid] = r.gam;
  };
  // bf16 copy of the state slice as S rows [v][k] (B operand of W S^T, Q S^T)
  auto store_state = [&]() {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (__bf16)st[4 * q4 + e];
      *reinterpret_cast<bf16x4 *>(&sb[l32 * RB + 32 * wave + 8 * q4 + 4 * g]) = x;
    }
  };

  ChunkRegs nxt;
  if (nchunks > 0) {
    load_chunk(0, nxt);
    store_chunk(0, nxt);
  }
  store_state();
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) load_chunk(c + 1, nxt);
    const int t0 = seq0 + c * C;
    const int n = min(C, seq_len - c * C);

    // waves 0, 1: X = W S^T (token rows 32 wave ..); waves 2, 3: Y = Q S^T
    const int tb = 32 * (wave & 1);
    const __bf16 *arow = (wave < 2 ? wl[buf] : qsl[buf]) + (tb + l32) * RB + 8 * g;
    f32x16 xy = (f32x16)(0.0f);
#pragma unroll
    for (int ks = 0; ks < DK / 16; ++ks) {
      const bf16x8 av = *reinterpret_cast<const bf16x8 *>(arow + 16 * ks);
      const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(&sb[l32 * RB + 16 * ks + 8 * g]);
      xy = mfma(av, bv, xy);
    }
    if (wave < 2) {
      // U' = U - X, stored transposed [v][t] in bf16
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = tb + 8 * q4 + 4 * g + e;
          x[e] = (__bf16)((float)ul[buf][t * RU + l32] - xy[4 * q4 + e]);
        }
        *reinterpret_cast<bf16x4 *>(&upt[l32 * RT + tb + 8 * q4 + 4 * g]) = x;
      }
    }
    __syncthreads();

    if (wave >= 2) {
      // O = diag(scale Gam) Q S^T + P U'
#pragma unroll
      for (int e = 0; e < 16; ++e) xy[e] *= a.scale * gl[buf][tb + acc_row(e, g)];
#pragma unroll
      for (int ks = 0; ks < C / 16; ++ks) {
        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&pl[buf][(tb + l32) * RT + 16 * ks + 8 * g]);
        const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(&upt[l32 * RT + 16 * ks + 8 * g]);
        xy = mfma(av, bv, xy);
      }
      __bf16 *orow = reinterpret_cast<__bf16 *>(a.out);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = tb + acc_row(e, g);
        if (t < n) orow[((size_t)(t0 + t) * a.h + h) * DV + kSliceRows * s + l32] = (__bf16)xy[e];
      }
    }
    // S^T <- Gam_last S^T + Kd U'
    const float glast = gl[buf][C - 1];
#pragma unroll
    for (int e = 0; e < 16; ++e) st[e] *= glast;
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&kdl[buf][(32 * wave + l32) * RT + 16 * ks + 8 * g]);
      const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(&upt[l32 * RT + 16 * ks + 8 * g]);
      st = mfma(av, bv, st);
    }
    store_state();
    if (c + 1 < nchunks) store_chunk(buf ^ 1, nxt);
    __syncthreads();
  }

  if (a.s_final != nullptr) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = st[4 * q4 + e];
      *reinterpret_cast<f32x4 *>(a.s_final + state_off + (size_t)(32 * s + l32) * DK + 32 * wave + 8 * q4 + 4 * g) = x;
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
    e = hipLaunchKernel(reinterpret_cast<const void *>(gdn_scan), dim3(a.n_seqs * a.h * (kDv / kSliceRows)),
                        dim3(256), args, 0, st);
  return static_cast<int>(e);
}

}  // namespace gdn
