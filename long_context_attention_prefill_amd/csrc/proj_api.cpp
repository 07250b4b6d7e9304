// proj_api.cpp -- C ABI of the projections (include/proj.h): argument checks,
// the dequantization launch and the vendor GEMM calls (hipBLASLt, fp32
// compute; a bias, when there is one, rides in the GEMM's epilogue).  Host
// only.
#include <cstdint>
#include <vector>

#include <hipblaslt/hipblaslt.h>

#include "proj.h"
#include "proj_launch.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// hipBLASLt plans, per calling thread and device (handles and descriptors
// are not shared between threads, and a handle and its algorithms belong to
// one device), created on first use of a shape and kept for the life of the
// process (tearing them down at thread exit could race the HIP runtime's own
// shutdown); a biased plan gets its bias pointer on every call.
struct LtPlan {
  int64_t t, n, k;
  bool f32;
  bool bias;
  bool ok;
  hipblasLtMatmulDesc_t desc;
  hipblasLtMatrixLayout_t la, lb, lc;
  hipblasLtMatmulAlgo_t algo;
};

struct LtState {
  int device = -1;
  hipblasLtHandle_t handle = nullptr;
  std::vector<LtPlan> plans;
};

constexpr size_t kMaxLtPlans = 64;

LtState *lt_state() {
  thread_local std::vector<LtState *> per_device;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  for (LtState *st : per_device)
    if (st->device == dev) return st;
  LtState *st = new LtState();
  st->device = dev;
  if (hipblasLtCreate(&st->handle) != HIPBLAS_STATUS_SUCCESS) st->handle = nullptr;
  per_device.push_back(st);
  return st;
}

void lt_destroy(LtPlan &p) {
  if (p.la != nullptr) hipblasLtMatrixLayoutDestroy(p.la);
  if (p.lb != nullptr) hipblasLtMatrixLayoutDestroy(p.lb);
  if (p.lc != nullptr) hipblasLtMatrixLayoutDestroy(p.lc);
  if (p.desc != nullptr) hipblasLtMatmulDescDestroy(p.desc);
}

// Row-major y[T][N] = x[T][K] w[N][K]^T (+ b) is, column-major, the N x T
// matrix op(W) X (+ b) with W the K x N view of w (transposed), X the K x T
// view of x and b broadcast along the T columns (the epilogue's bias runs
// along rows).
const LtPlan *lt_plan(LtState *st, int64_t t, int64_t n, int64_t k, bool f32, bool bias) {
  for (const LtPlan &p : st->plans)
    if (p.t == t && p.n == n && p.k == k && p.f32 == f32 && p.bias == bias) return &p;
  if (st->plans.size() >= kMaxLtPlans) {
    lt_destroy(st->plans.front());
    st->plans.erase(st->plans.begin());
  }
  LtPlan p{};
  p.t = t;
  p.n = n;
  p.k = k;
  p.f32 = f32;
  p.bias = bias;
  const hipDataType dt = f32 ? HIP_R_32F : HIP_R_16BF;
  bool good = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  const hipblasLtEpilogue_t ep = bias ? HIPBLASLT_EPILOGUE_BIAS : HIPBLASLT_EPILOGUE_DEFAULT;
  const int32_t bias_type = dt;
  good = good &&
         hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &ep, sizeof(ep)) == HIPBLAS_STATUS_SUCCESS &&
         (!bias || hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type,
                                                   sizeof(bias_type)) == HIPBLAS_STATUS_SUCCESS);
  good = good && hipblasLtMatrixLayoutCreate(&p.la, dt, k, n, k) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatrixLayoutCreate(&p.lb, dt, k, t, k) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatrixLayoutCreate(&p.lc, dt, n, t, n) == HIPBLAS_STATUS_SUCCESS;
  if (good) {
    // the heuristic's first choice, with no workspace: a fixed algorithm per
    // shape, so repeated calls give the same bits
    hipblasLtMatmulPreference_t pref = nullptr;
    uint64_t ws = 0;
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    good = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
           hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof(ws)) ==
               HIPBLAS_STATUS_SUCCESS &&
           hipblasLtMatmulAlgoGetHeuristic(st->handle, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &found) ==
               HIPBLAS_STATUS_SUCCESS &&
           found > 0;
    if (pref != nullptr) hipblasLtMatmulPreferenceDestroy(pref);
    if (good) p.algo = res[0].algo;
  }
  p.ok = good;
  st->plans.push_back(p);
  return &st->plans.back();
}

}  // namespace

namespace proj {

namespace {

int gemm(const void *x, const void *w, const void *bias, void *y, int64_t t, int64_t n, int64_t k, bool f32,
         void *stream) {
  LtState *st = lt_state();
  if (st == nullptr || st->handle == nullptr) return -1;
  const LtPlan *p = lt_plan(st, t, n, k, f32, bias != nullptr);
  if (!p->ok) return -1;
  if (bias != nullptr &&
      hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)) !=
          HIPBLAS_STATUS_SUCCESS)
    return -1;
  const float alpha = 1.0f, beta = 0.0f;
  return hipblasLtMatmul(st->handle, p->desc, &alpha, w, p->la, x, p->lb, &beta, y, p->lc, y, p->lc, &p->algo,
                         nullptr, 0, static_cast<hipStream_t>(stream)) == HIPBLAS_STATUS_SUCCESS
             ? 0
             : -1;
}

}  // namespace

int gemm_nt(const void *x, const void *w, void *y, int64_t t, int64_t n, int64_t k, void *stream) {
  return gemm(x, w, nullptr, y, t, n, k, false, stream);
}

int gemm_nt_bias(const void *x, const void *w, const void *bias, void *y, int64_t t, int64_t n, int64_t k,
                 bool f32, void *stream) {
  return bias == nullptr ? -1 : gemm(x, w, bias, y, t, n, k, f32, stream);
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
  return proj::gemm_nt(x, w, y, t, n, k, stream) == 0 ? ATTN_OK : ATTN_ELAUNCH;
}

}  // extern "C"
