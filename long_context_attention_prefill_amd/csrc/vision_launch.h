// vision_launch.h -- the vision block's elementwise launches, shared by the
// host translation unit (vision_api.cpp) and the HIP one (vision_fwd.hip).
#pragma once

#include <stdint.h>

namespace vision {

// q, k, v [T][H][d] (dtype) = the three column blocks of qkv [T][3 H d] (fp32)
// plus the matching entries of bias [3 H d] (dtype), rounded once.
int launch_split_qkv(const float *qkv, const void *bias, void *q, void *k, void *v, int64_t t,
                     int32_t hd, bool f32, void *stream);
// out [T][n] (dtype) = y [T][n] (fp32) + bias [n] (dtype), rounded once.
int launch_add_bias(const float *y, const void *bias, void *out, int64_t t, int32_t n, bool f32,
                    void *stream);

}  // namespace vision
