// proj_launch.h -- the dequantization kernel's launch, shared by the host
// translation unit (proj_api.cpp) and the HIP one (proj_fwd.hip), and the
// library's internal vendor-GEMM calls.
#pragma once

#include <stdint.h>

namespace proj {

// w[n][k] = bf16(scale[n] * q[n][k]); returns 0 or a hipError_t value.
int launch_dequantize_int8(const int8_t *q, const float *scale, void *w, int64_t n, int64_t k,
                           void *stream);

// y[T][N] = x[T][K] w[N][K]^T by the vendor GEMM (hipBLASLt), bf16 in and
// out, fp32 accumulation.  Sizes already checked (each < 2^31, K >= 1).
// Returns 0 or -1.
int gemm_nt(const void *x, const void *w, void *y, int64_t t, int64_t n, int64_t k, void *stream);

// y[T][N] = x[T][K] w[N][K]^T + b[N] by the vendor GEMM (hipBLASLt, the bias
// added to the fp32 accumulator in its epilogue, the result rounded once to
// the inputs' type), all of one type: bf16, or fp32 when `f32`.  Row-major,
// contiguous.  Returns 0, or -1 when the library has no algorithm for the
// shape or refuses the call.
int gemm_nt_bias(const void *x, const void *w, const void *bias, void *y, int64_t t, int64_t n, int64_t k,
                 bool f32, void *stream);

}  // namespace proj
