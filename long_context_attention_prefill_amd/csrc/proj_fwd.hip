// proj_fwd.hip -- int8 weight dequantization for gfx950 (MI355X).
//
// The paper "A Modern Multimodal Assistant on a 6 GB 2011 GPU" keeps its
// language weights in 8 bits and dequantizes them once before the vendor
// GEMM (abstract, result (i); gist.science technical summary, Metodologia,
// GEMM efficiency).  Here: w[n][k] = bf16(scale[n] * q[n][k]), the product
// in fp32 and one round to nearest even to bf16.  The pass is bound by HBM
// (1 byte read, 2 written per weight): each thread turns 16 weights of one
// row (a 16-byte load) into two 16-byte stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "proj_launch.h"

namespace proj {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int8_t i8x16 __attribute__((ext_vector_type(16)));

// K a multiple of 16: 16 weights per thread, vector loads and stores.
__global__ __launch_bounds__(256) void dequant_vec16(const int8_t *__restrict__ q,
                                                     const float *__restrict__ scale,
                                                     __bf16 *__restrict__ w, int64_t n, int64_t k) {
  const int64_t per_row = k >> 4;
  const int64_t total = n * per_row;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = c / per_row;
    const float s = scale[row];
    const i8x16 v = *reinterpret_cast<const i8x16 *>(q + c * 16);
    bf16x8 lo, hi;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = (__bf16)(s * (float)v[e]);
      hi[e] = (__bf16)(s * (float)v[8 + e]);
    }
    *reinterpret_cast<bf16x8 *>(w + c * 16) = lo;
    *reinterpret_cast<bf16x8 *>(w + c * 16 + 8) = hi;
  }
}

// Any K: one weight per thread.
__global__ __launch_bounds__(256) void dequant_scalar(const int8_t *__restrict__ q,
                                                      const float *__restrict__ scale,
                                                      __bf16 *__restrict__ w, int64_t n, int64_t k) {
  const int64_t total = n * k;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x)
    w[i] = (__bf16)(scale[i / k] * (float)q[i]);
}

}  // namespace

int launch_dequantize_int8(const int8_t *q, const float *scale, void *w, int64_t n, int64_t k,
                           void *stream) {
  if (n == 0 || k == 0) return 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool vec = (k % 16) == 0;
  const int64_t work = vec ? n * (k / 16) : n * k;
  const int64_t blocks = std::min<int64_t>((work + 255) / 256, 256 * 64);
  if (vec)
    dequant_vec16<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(q, scale, static_cast<__bf16 *>(w), n, k);
  else
    dequant_scalar<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(q, scale, static_cast<__bf16 *>(w), n, k);
  return static_cast<int>(hipGetLastError());
}

}  // namespace proj
