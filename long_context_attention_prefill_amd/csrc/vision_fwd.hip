// vision_fwd.hip -- the vision attention block's elementwise passes on gfx950:
// bias add and head split after the QKV projection, bias add after the
// output projection.  Both read the vendor GEMM's fp32 result once and round
// once to the block's dtype; HBM-bound, four values per thread.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "vision_launch.h"

namespace vision {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ float as_f32(const T *p, int64_t i) { return (float)p[i]; }

template <typename T>
__device__ __forceinline__ void store4(T *p, int64_t i, f32x4 x);
template <>
__device__ __forceinline__ void store4<float>(float *p, int64_t i, f32x4 x) {
  *reinterpret_cast<f32x4 *>(p + i) = x;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16 *p, int64_t i, f32x4 x) {
  bf16x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (__bf16)x[e];
  *reinterpret_cast<bf16x4 *>(p + i) = y;
}

// qkv row t: [q (hd) | k (hd) | v (hd)]; the destination of column c.
template <typename T>
__global__ __launch_bounds__(256) void split_qkv(const float *__restrict__ qkv, const T *__restrict__ bias,
                                                 T *__restrict__ q, T *__restrict__ k, T *__restrict__ v,
                                                 int64_t t, int32_t hd) {
  const int64_t per_row = (3 * (int64_t)hd) / 4;
  const int64_t total = t * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / per_row;
    const int32_t c = (int32_t)(i - row * per_row) * 4;
    f32x4 x = *reinterpret_cast<const f32x4 *>(qkv + row * 3 * hd + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] += as_f32(bias, c + e);
    const int part = c / hd, col = c - part * hd;
    T *dst = part == 0 ? q : (part == 1 ? k : v);
    store4(dst, row * hd + col, x);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void add_bias(const float *__restrict__ y, const T *__restrict__ bias,
                                                T *__restrict__ out, int64_t t, int32_t n) {
  const int64_t per_row = n / 4;
  const int64_t total = t * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / per_row;
    const int32_t c = (int32_t)(i - row * per_row) * 4;
    f32x4 x = *reinterpret_cast<const f32x4 *>(y + row * n + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] += as_f32(bias, c + e);
    store4(out, row * n + c, x);
  }
}

unsigned blocks_for(int64_t work) { return (unsigned)std::min<int64_t>((work + 255) / 256, 256 * 64); }

}  // namespace

int launch_split_qkv(const float *qkv, const void *bias, void *q, void *k, void *v, int64_t t, int32_t hd,
                     bool f32, void *stream) {
  if (t == 0) return 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned nb = blocks_for(t * 3 * (int64_t)hd / 4);
  if (f32)
    split_qkv<float><<<nb, 256, 0, st>>>(qkv, static_cast<const float *>(bias), static_cast<float *>(q),
                                         static_cast<float *>(k), static_cast<float *>(v), t, hd);
  else
    split_qkv<__bf16><<<nb, 256, 0, st>>>(qkv, static_cast<const __bf16 *>(bias), static_cast<__bf16 *>(q),
                                          static_cast<__bf16 *>(k), static_cast<__bf16 *>(v), t, hd);
  return static_cast<int>(hipGetLastError());
}

int launch_add_bias(const float *y, const void *bias, void *out, int64_t t, int32_t n, bool f32, void *stream) {
  if (t == 0) return 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned nb = blocks_for(t * (int64_t)n / 4);
  if (f32)
    add_bias<float><<<nb, 256, 0, st>>>(y, static_cast<const float *>(bias), static_cast<float *>(out), t, n);
  else
    add_bias<__bf16><<<nb, 256, 0, st>>>(y, static_cast<const __bf16 *>(bias), static_cast<__bf16 *>(out), t, n);
  return static_cast<int>(hipGetLastError());
}

}  // namespace vision
