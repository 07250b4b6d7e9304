/*
 * proj.h -- C ABI of the projections on either side of attention, for
 * MI355X (gfx950): int8 weights dequantized once, then the vendor GEMM.
 *
 * The paper "A Modern Multimodal Assistant on a 6 GB 2011 GPU" keeps its
 * language weights in 8 bits and, rather than hand-written GEMM tiles,
 * dequantizes them once and calls the vendor GEMM, which reached 64 % of the
 * FP32 peak where the best hand-written tile reached 37 % (abstract, result
 * (i); gist.science technical summary, Metodologia, GEMM efficiency).  The
 * pages give neither the quantization format nor the layer sizes; the plain
 * reading used here is symmetric int8 with one float scale per output row,
 * w[n][k] = scale[n] * q[n][k].  On MI355X the matrix cores run bf16 (2.5
 * PFLOP/s dense) against 157 TFLOP/s of fp32, so the weights are dequantized
 * to bf16 (round to nearest even) and the projection is the vendor bf16
 * GEMM with fp32 accumulation.
 *
 * Layout: row-major, contiguous.  x [T][K], w [N][K], y [T][N]:
 *     y[t][n] = sum_k x[t][k] * w[n][k]            (y = x w^T)
 * Device pointers must be 16-byte aligned (scale: 4-byte).
 *
 * Ownership and execution as for attn_prefill: the caller owns every buffer;
 * calls check all arguments on the host first, enqueue on `stream` and
 * return; status codes of attn_prefill.h.  proj_linear calls hipBLASLt with
 * one handle per calling thread and one plan per shape, created on first use
 * (the heuristic's first algorithm, which needs no GEMM workspace, so a
 * shape always runs the same algorithm and gives the same bits).
 */
#ifndef PROJ_H
#define PROJ_H

#include <stdint.h>

#include "attn_prefill.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * w[n][k] = bf16(scale[n] * q[n][k]) for n < N, k < K (one pass; run once
 * per weight matrix).
 *   q      device int8 [N][K]
 *   scale  device float32 [N], finite
 *   w      device bf16 [N][K], overlapping neither input
 * Returns ATTN_OK, ATTN_EINVAL for NULL or misaligned pointers (NULL allowed
 * when N * K = 0), N < 0, K < 0, overlap; ATTN_ELAUNCH on a launch failure.
 */
int proj_dequantize_int8(const int8_t *q, const float *scale, void *w, int64_t n,
                         int64_t k, void *stream);

/*
 * y = x w^T in bf16 with fp32 accumulation (vendor GEMM, hipBLASLt).
 *   x  device bf16 [T][K];  w  device bf16 [N][K];  y  device bf16 [T][N],
 *   overlapping neither input.  T, N >= 0, K >= 1, each < 2^31.
 * Returns ATTN_OK (T * N = 0 does nothing), ATTN_EINVAL for NULL/misaligned
 * pointers, negative sizes, K < 1 or overlap, ATTN_EUNSUPPORTED for sizes of
 * 2^31 or more, ATTN_ELAUNCH when the vendor library has no algorithm for
 * the shape or fails.
 */
int proj_linear(const void *x, const void *w, void *y, int64_t t, int64_t n, int64_t k,
                void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PROJ_H */
