// proj_api.cpp -- C ABI of the projections (include/proj.h): argument checks,
// the dequantization launch and the vendor GEMM call (rocBLAS, bf16 in and
// out, fp32 compute).  Host only.
#include <cstdint>

#include <rocblas/rocblas.h>

#include "proj.h"
#include "proj_launch.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// One handle per calling thread: rocBLAS handles bind a stream and are not
// meant to be shared between threads.  Created on first use, kept for the
// life of the process (tearing it down at thread exit could race the HIP
// runtime's own shutdown).
rocblas_handle thread_handle() {
  thread_local rocblas_handle h = nullptr;
  if (h == nullptr && rocblas_create_handle(&h) != rocblas_status_success) h = nullptr;
  return h;
}

}  // namespace

namespace proj {

int gemm_nt(const void *x, const void *w, void *y, int64_t t, int64_t n, int64_t k, bool f32_in,
            bool f32_out, void *stream) {
  rocblas_handle h = thread_handle();
  if (h == nullptr) return -1;
  if (rocblas_set_stream(h, static_cast<hipStream_t>(stream)) != rocblas_status_success) return -1;
  // Row-major y[T][N] = x[T][K] w[N][K]^T is, column-major, the N x T matrix
  // W^T X with W the K x N view of w (ld K) and X the K x T view of x (ld K).
  const rocblas_datatype in = f32_in ? rocblas_datatype_f32_r : rocblas_datatype_bf16_r;
  const rocblas_datatype out = f32_out ? rocblas_datatype_f32_r : in;
  const float alpha = 1.0f, beta = 0.0f;
  const rocblas_status st = rocblas_gemm_ex(
      h, rocblas_operation_transpose, rocblas_operation_none, static_cast<rocblas_int>(n),
      static_cast<rocblas_int>(t), static_cast<rocblas_int>(k), &alpha, w, in, static_cast<rocblas_int>(k), x, in,
      static_cast<rocblas_int>(k), &beta, y, out, static_cast<rocblas_int>(n), y, out,
      static_cast<rocblas_int>(n), rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? 0 : -1;
}

}  // namespace proj

extern "C" {

int proj_dequantize_int8(const int8_t *q, const float *scale, void *w, int64_t n, int64_t k,
                         void *stream) {
  if (n < 0 || k < 0) return ATTN_EINVAL;
  const uint64_t elems = static_cast<uint64_t>(n) * static_cast<uint64_t>(k);
  if (elems == 0) return ATTN_OK;
  if (q == nullptr || scale == nullptr || w == nullptr) return ATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(w, 16) || !aligned(scale, 4)) return ATTN_EINVAL;
  if (overlaps(w, elems * 2, q, elems) || overlaps(w, elems * 2, scale, static_cast<uint64_t>(n) * 4))
    return ATTN_EINVAL;
  return proj::launch_dequantize_int8(q, scale, w, n, k, stream) == 0 ? ATTN_OK : ATTN_ELAUNCH;
}

int proj_linear(const void *x, const void *w, void *y, int64_t t, int64_t n, int64_t k, void *stream) {
  if (t < 0 || n < 0 || k < 1) return ATTN_EINVAL;
  if (t == 0 || n == 0) return ATTN_OK;
  if (t >= (int64_t(1) << 31) || n >= (int64_t(1) << 31) || k >= (int64_t(1) << 31)) return ATTN_EUNSUPPORTED;
  if (x == nullptr || w == nullptr || y == nullptr) return ATTN_EINVAL;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return ATTN_EINVAL;
  const uint64_t xb = static_cast<uint64_t>(t) * k * 2, wb = static_cast<uint64_t>(n) * k * 2,
                 yb = static_cast<uint64_t>(t) * n * 2;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, w, wb)) return ATTN_EINVAL;
  return proj::gemm_nt(x, w, y, t, n, k, false, false, stream) == 0 ? ATTN_OK : ATTN_ELAUNCH;
}

}  // extern "C"
