// attn_decode.hip -- decode attention for gfx950 (MI355X): the newest token
// of each sequence attends to its whole key/value cache.  The cache is cut
// into chunks computed in parallel (one wave each) and merged exactly
// through their softmax references and sums; one chunk per sequence writes
// the output directly.  The result equals exact attention of that single
// query over its visible keys (bottom-right alignment: the query is the last
// position of its sequence).
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

// ---------------------------------------------------------------------------
// Decode: one query per sequence over its key/value cache.  Every wave is an
// independent worker on one item (sequence, KV head, block of up to 32 of
// that KV head's query heads, chunk of up to a.chunk visible keys): the
// block's query heads are the 32 query columns of S^T = K Q^T (unused columns
// carry zeros), so each K and V element the item streams is used by all its
// query heads.  Per 32-key tile, K fragments come straight from memory into
// registers (a range-checked buffer load per MFMA step: each lane reads 16
// bytes of the key row it multiplies, keys past the chunk read as zeros),
// one tile ahead; V reaches the wave's own double-buffered LDS region by
// direct loads in the prefill layout (rows of CH+1 16-byte slots, permuted
// keys) for the transposing reads.  A wave waits only on its own loads, and
// two workgroups share a CU.  The softmax is the online one with the
// prefill kernels' lazy rescale (the reference rises only by more than
// kRescaleSlack doublings).  With one chunk per (sequence, head block) the
// wave writes the output; otherwise it writes its unnormalised output,
// reference and sum to the workspace and decode_merge combines the chunks.
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256, 2) void decode_bf16_partial(const DecodeArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(D == 64 || D == 128, "decode covers head_dim 64 and 128");
  using L = FastLayout<D>;
  constexpr int BN = kDecodeTile;
  constexpr int CH = L::CH;
  constexpr int KST = D / 16;
  constexpr int DB = D / 32;
  constexpr int NLOADS = (BN * L::SLOTS + 63) / 64;  // wave-wide V loads per tile
  constexpr int TILE = NLOADS * 1024;                // V tile bytes, with zero-filled spill
  // one array per buffer half, indexed by wave: a direct load into one half
  // is then visibly unrelated to reads of the other
  __shared__ __attribute__((aligned(1024))) char v_lds0[4][TILE];
  __shared__ __attribute__((aligned(1024))) char v_lds1[4][TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __builtin_assume(wave >= 0 && wave < 4);
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int item = blockIdx.x * 4 + wave;
  if (item >= a.total_items) return;  // a whole wave; no barrier follows

  int seq = 0;
  while (seq + 1 < a.n_seqs && a.item_start[seq + 1] <= item) ++seq;
  const int rem = item - a.item_start[seq];
  const int splits = a.splits[seq];
  const int gh = rem / splits;
  const int split = rem - gh * splits;
  const int kvh = gh / a.head_blocks;
  const int hb = gh - kvh * a.head_blocks;
  const int k0 = split * a.chunk;                       // within the visible keys
  const int k1 = min(k0 + a.chunk, a.k_count[seq]);
  const float c = a.c == 0.0f ? 0x1p-126f : a.c;

  // query head of this lane's column
  const int hr = hb * 32 + l32;                         // head within the KV group
  const bool col_ok = l32 < a.rows && hr < a.group;
  const int h = kvh * a.group + hr;
  bf16x8 qf[KST];
  {
    const __bf16 *qrow = reinterpret_cast<const __bf16 *>(a.q) + ((size_t)seq * a.hq + (col_ok ? h : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      qf[kk] = col_ok ? *reinterpret_cast<const bf16x8 *>(qrow + 16 * kk + 8 * g) : (bf16x8)((__bf16)0.0f);
  }

  const int rowbytes = a.hkv * D * 2;
  uint32_t ld_off[NLOADS];
#pragma unroll
  for (int j = 0; j < NLOADS; ++j) {
    const int p = j * 64 + lane;
    const int r = p / L::SLOTS, cs = p % L::SLOTS;
    ld_off[j] = (cs < CH && r < BN) ? (uint32_t)(r * rowbytes + cs * 16) : kOutOfRange;
  }
  const size_t base = ((size_t)(a.k_begin[seq]) * a.hkv + kvh) * D * 2;
  const char *kseq = reinterpret_cast<const char *>(a.k) + base;
  const char *vseq = reinterpret_cast<const char *>(a.v) + base;
  // keys kt .. kt+31, rows past k1 out of range
  auto tile_rsrc = [&](const char *src, int kt) {
    const int nrows = min(k1 - kt, BN);
    const int rec = max(0, (nrows - 1) * rowbytes + D * 2);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(src + (size_t)kt * rowbytes), (short)0,
                                             rec, kBufferWord3);
  };
  auto issue_v = [&](auto buf_tag, int kt) {
    char *lds = decltype(buf_tag)::value == 0 ? v_lds0[wave] : v_lds1[wave];
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(vseq, kt);
#pragma unroll
    for (int j = 0; j < NLOADS; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(lds + j * 1024), 16, ld_off[j], 0, 0, 0);
  };
  // K fragment kk of MFMA row l32 (key key_of_row(l32), the order the V
  // reads expect): 16 bytes at column 16 kk + 8 g
  const uint32_t kvoff = (uint32_t)(key_of_row(l32) * rowbytes + 16 * g);
  auto load_k = [&](bf16x8 (&kf)[KST], int kt) {
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(kseq, kt);
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      kf[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, kvoff + kk * 32, 0, 0));
  };
  const int vread = (g + 4 * ((lane & 15) >> 2)) * L::ROWB + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16)(0.0f);
  float m_run = kNegInf, l_run = 0.0f;  // reference (exp2 units) and this lane's share of the sum
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 kfa[KST], kfb[KST];

  // One tile: K in kf, V in buffer BUF; the next tile's K goes to kn and its
  // V to the other buffer while this one is computed.
  auto step = [&](auto buf_tag, bf16x8 (&kf)[KST], bf16x8 (&kn)[KST], int kt) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_tag)::value;
    const char *vb = (BUF == 0 ? v_lds0[wave] : v_lds1[wave]) + vread;
    const bool more = kt + BN < k1;
    if (more) {
      issue_v(std::integral_constant<int, BUF ^ 1>{}, kt + BN);
      load_k(kn, kt + BN);
    }
    f32x16 sc = (f32x16)(0.0f);
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], sc, 0, 0, 0);
    // x = c * s in exp2 units; on the chunk's last tile keys past k1 are void.
    // Entry j of lane half g holds key kt + 16 (j >> 3) + 2 ((j >> 2) & 1) + 4 (j & 3) + g.
    float mx = kNegInf;
    if (kt + BN <= k1) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sc[j] *= c;
        mx = fmaxf(mx, sc[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kt + 16 * (j >> 3) + 2 * ((j >> 2) & 1) + 4 * (j & 3) + g;
        sc[j] = key < k1 ? sc[j] * c : kNegInf;
        mx = fmaxf(mx, sc[j]);
      }
    }
    mx = fmaxf(mx, xor32(mx));
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack)) {
      const float m_new = mx > m_run + kRescaleSlack ? mx : m_run;
      const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    bf16x8 pf[BN / 16];
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[ks][e] = (__bf16)fast_exp2(sc[8 * ks + e] - m_run);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {pf[ks][2 * e], pf[ks][2 * e + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
      }
    }
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char *vp = vb + ks * 16 * L::ROWB + db * 64;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vp));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vp + 2 * L::ROWB));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[db], 0, 0, 0);
      }
    // the next tile's loads complete before it is computed, and this V
    // buffer's reads complete before the tile after next overwrites it
    __builtin_amdgcn_s_waitcnt(0);
  };

  issue_v(std::integral_constant<int, 0>{}, k0);
  load_k(kfa, k0);
  __builtin_amdgcn_s_waitcnt(0);
  int kt = k0;
  for (; kt + BN < k1; kt += 2 * BN) {
    step(std::integral_constant<int, 0>{}, kfa, kfb, kt);
    step(std::integral_constant<int, 1>{}, kfb, kfa, kt + BN);
  }
  if (kt < k1) step(std::integral_constant<int, 0>{}, kfa, kfb, kt);

  const float l_tot = l_run + xor32(l_run);
  if (!col_ok) return;
  if (a.direct) {
    const float inv = 1.0f / l_tot;
    __bf16 *orow = reinterpret_cast<__bf16 *>(a.out) + ((size_t)seq * a.hq + h) * D;
    if (a.lse != nullptr && g == 0) a.lse[(size_t)seq * a.hq + h] = (m_run + log2f(l_tot)) * kLn2;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[db][4 * jj + e] * inv);
        *reinterpret_cast<bf16x4 *>(orow + 32 * db + 8 * jj + 4 * g) = w;
      }
  } else {
    const size_t row = (size_t)item * a.rows + l32;
    float *orow = a.ws_o + row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[db][4 * jj + e];
        *reinterpret_cast<f32x4 *>(orow + 32 * db + 8 * jj + 4 * g) = w;
      }
    if (g == 0) {
      a.ws_ml[2 * row] = m_run;
      a.ws_ml[2 * row + 1] = l_tot;
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// Merge of the chunks of one (sequence, query head): with references m_s and
// sums l_s, m = max m_s, l = sum l_s 2^(m_s - m), out = sum o_s 2^(m_s - m) / l.
// A workgroup takes CB output columns of one (sequence, head): its 256
// threads find m and l together (wave reductions, then one exchange), then
// each thread owns four columns and every (256 / (CB / 4))-th chunk, eight
// independent loads at a time, and the partial sums meet in LDS.  With few
// (sequence, head) pairs (small batches, hence many chunks each) CB = 32
// spreads one pair over D / 32 workgroups; otherwise CB = D.
template <int D, int CB>
__global__ __launch_bounds__(256) void decode_merge(const DecodeArgs a) {
  static_assert(D % CB == 0 && CB % 32 == 0, "whole column blocks");
  constexpr int CPL = CB / 4;  // threads per chunk row (four columns each)
  constexpr int NG = 256 / CPL;  // chunk groups
  constexpr int U = 8;           // loads in flight per thread
  __shared__ float red[2][4];
  __shared__ f32x4 part[NG][CPL];
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int cb = blockIdx.x % (D / CB);
  const int sh = blockIdx.x / (D / CB);
  const int seq = sh / a.hq;
  const int h = sh - seq * a.hq;
  const int kvh = h / a.group;
  const int hr = h - kvh * a.group;
  const int hb = hr >> 5;
  const int r = hr & 31;
  const int splits = a.splits[seq];
  const size_t first = (size_t)a.item_start[seq] + (size_t)(kvh * a.head_blocks + hb) * splits;
  auto ml = [&](int s) { return reinterpret_cast<const float2 *>(a.ws_ml)[(first + s) * a.rows + r]; };

  float m = kNegInf;
  for (int s = t; s < splits; s += 256) m = fmaxf(m, ml(s).x);
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) m = fmaxf(m, __shfl_xor(m, w));
  if ((t & 63) == 0) red[0][wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float l = 0.0f;
  for (int s = t; s < splits; s += 256) {
    const float2 e = ml(s);
    l += e.y * fast_exp2(e.x - m);
  }
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) l += __shfl_xor(l, w);
  if ((t & 63) == 0) red[1][wave] = l;

  const int col = cb * CB + 4 * (t % CPL), grp = t / CPL;
  f32x4 acc = (f32x4)(0.0f);
  for (int s0 = grp; s0 < splits; s0 += U * NG) {
    f32x4 ov[U];
    float ms[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * NG;
      ov[u] = (f32x4)(0.0f);
      ms[u] = kNegInf;
      if (s < splits) {
        ov[u] = *reinterpret_cast<const f32x4 *>(a.ws_o + ((first + s) * a.rows + r) * D + col);
        ms[u] = ml(s).x;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += ov[u] * fast_exp2(ms[u] - m);
  }
  part[grp][t % CPL] = acc;
  __syncthreads();
  l = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  if (t < CPL) {
    f32x4 sum = part[0][t];
#pragma unroll
    for (int g = 1; g < NG; ++g) sum += part[g][t];
    const float inv = 1.0f / l;
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (__bf16)(sum[e] * inv);
    *reinterpret_cast<bf16x4 *>(reinterpret_cast<__bf16 *>(a.out) + ((size_t)seq * a.hq + h) * D + col) = o;
  }
  if (a.lse != nullptr && cb == 0 && t == 0) a.lse[(size_t)seq * a.hq + h] = (m + log2f(l)) * kLn2;
}

// (sequence, head) pairs from which each pair gets one merge workgroup
constexpr int kMergeWideFrom = 256;

}  // namespace

// The decode workspace of attn_decode_noalloc: one copy per device (each
// device's code object holds its own), alive until the process ends.  Host
// code never uses the array's name as an address: decode_scratch() looks up
// each device's copy once, with that device current, and hands out that
// address.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices] = {};
}  // namespace

int decode_scratch(void *stream, void **ptr) {
  int dev = 0;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                   : hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return static_cast<int>(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return static_cast<int>(e);
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return static_cast<int>(e);
    if (p == nullptr) return static_cast<int>(hipErrorInvalidSymbol);
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return 0;
}

int launch_decode_bf16(const DecodeArgs &a, int head_dim, void *stream) {
  if (a.total_items == 0) return 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void *args[] = {const_cast<DecodeArgs *>(&a)};
  const dim3 grid((a.total_items + 3) / 4);
  const int pairs = a.n_seqs * a.hq;
  const bool wide = pairs >= kMergeWideFrom;
  const void *partial, *merge;
  switch (head_dim) {
    case 64:
      partial = reinterpret_cast<const void *>(decode_bf16_partial<64>);
      merge = wide ? reinterpret_cast<const void *>(decode_merge<64, 64>)
                   : reinterpret_cast<const void *>(decode_merge<64, 32>);
      break;
    case 128:
      partial = reinterpret_cast<const void *>(decode_bf16_partial<128>);
      merge = wide ? reinterpret_cast<const void *>(decode_merge<128, 128>)
                   : reinterpret_cast<const void *>(decode_merge<128, 32>);
      break;
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  hipError_t e = hipLaunchKernel(partial, grid, dim3(256), args, 0, st);
  if (e == hipSuccess && !a.direct) {
    const dim3 merge_grid(pairs * (wide ? 1 : head_dim / 32));
    e = hipLaunchKernel(merge, merge_grid, dim3(256), args, 0, st);
  }
  return static_cast<int>(e);
}

}  // namespace attn
