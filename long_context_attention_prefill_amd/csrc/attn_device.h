// attn_device.h -- device-side definitions shared by the gfx950 attention
// kernels (prefill in attn_fwd.hip, decode in attn_decode.hip): vector
// types, base-2 softmax constants, raw buffer descriptor constants and the
// padded, key-permuted LDS tile layout of the MFMA kernels.
#ifndef ATTN_DEVICE_H
#define ATTN_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;

// Softmax runs in base 2 on scores pre-multiplied by scale*log2(e).  The
// reference maximum is raised only when a row's new maximum exceeds it by
// more than this many doublings, so probabilities stay below 2^8 and the
// output/sum rescale is skipped on most tiles.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// ---------------------------------------------------------------------------
// LDS tile layout of the MFMA kernels.  A K or V tile row (one key, d bf16
// values = CH 16-byte chunks in memory) occupies CH + 1 16-byte slots in LDS
// (one slot of padding, filled with zeros by the same direct loads), and
// inside each 16-key MFMA step the keys are taken in the order
//     pi(x) = ((x >> 2) & 1) + 4 (x & 3) + 2 (x >> 3),   x = MFMA row mod 16,
// so that on gfx950's 64 banks x 4 bytes (b128 reads serve 16 lanes per
// cycle, b64 reads 32):
//   - the 16 K rows read together (rows pi(0..15)) start in 16 distinct
//     16-byte slots mod 256 bytes (odd row stride in slots), and
//   - the 4 V rows of each transposing read (ds_read_b64_tr_b16) are 4 rows,
//     i.e. 64 bytes mod 256, apart,
// both conflict-free, with every LDS address a per-lane base plus an
// immediate offset.
// ---------------------------------------------------------------------------

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Raw buffer descriptor word 3 for gfx9-family parts (32-bit data format).
constexpr int kBufferWord3 = 0x00020000;
// A buffer offset past any key range: the load returns zeros.
constexpr uint32_t kOutOfRange = 0x7ffffff0u;

template <int D>
struct FastLayout {
  static constexpr int CH = D / 8;            // 16-byte chunks of a row in memory
  static constexpr int KST = (D + 15) / 16;   // 16-wide MFMA k steps over the row
  // 16-byte slots per K or V row in LDS: the k steps' 2 KST chunks (those
  // past CH zero-filled, so a head dim that is not a multiple of 16 reads
  // zeros in its last step) plus one, an odd count
  static constexpr int SLOTS = 2 * KST + 1;
  static constexpr int ROWB = SLOTS * 16;
  static_assert(D % 8 == 0, "whole 16-byte chunks per row");
};

// Key (0..31 within a 32-key block) held by MFMA row m of S^T.
__device__ __forceinline__ int key_of_row(int m) {
  const int x = m & 15;
  return 16 * (m >> 4) + ((x >> 2) & 1) + 4 * (x & 3) + 2 * (x >> 3);
}

}  // namespace
}  // namespace attn

#endif  // ATTN_DEVICE_H
