// proj_launch.h -- the dequantization kernel's launch, shared by the host
// translation unit (proj_api.cpp) and the HIP one (proj_fwd.hip).
#pragma once

#include <stdint.h>

namespace proj {

// w[n][k] = bf16(scale[n] * q[n][k]); returns 0 or a hipError_t value.
int launch_dequantize_int8(const int8_t *q, const float *scale, void *w, int64_t n, int64_t k,
                           void *stream);

}  // namespace proj
