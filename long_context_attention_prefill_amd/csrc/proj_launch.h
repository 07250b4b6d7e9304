// proj_launch.h -- the dequantization kernel's launch, shared by the host
// translation unit (proj_api.cpp) and the HIP one (proj_fwd.hip).
#pragma once

#include <stdint.h>

namespace proj {

// w[n][k] = bf16(scale[n] * q[n][k]); returns 0 or a hipError_t value.
int launch_dequantize_int8(const int8_t *q, const float *scale, void *w, int64_t n, int64_t k,
                           void *stream);

// y[T][N] = x[T][K] w[N][K]^T by the vendor GEMM, inputs bf16 (f32_in false)
// or fp32, output fp32 (f32_out) or the input type, fp32 accumulation.
// Sizes already checked (each < 2^31, K >= 1).  Returns 0 or -1.
int gemm_nt(const void *x, const void *w, void *y, int64_t t, int64_t n, int64_t k, bool f32_in,
            bool f32_out, void *stream);

}  // namespace proj
