// Dense projections over whole token rows: the full-width [C, C] reading of
// the static projection W_p and the output projection W^O.
//
// Sources: SALAD structured summary (paper.rainbus.top/paper/2601.16515),
// method steps 4 (projection of the linear branch's output) and 7 (output
// projection).
//
// Both are plain GEMMs, [rows, C] x [C, C] with rows = B*N in the tens of
// thousands and C = H*d in the thousands, so they go to hipBLASLt (MFMA
// kernels tuned per shape) rather than a hand-written kernel.  One handle
// per device, created on first use; per device and shape the descriptors and
// the library's first-ranked algorithm (among those needing no workspace)
// are built once and reused.  A lock serialises lookups and launches, since
// a handle is not safe to share between threads.
#include <hipblaslt/hipblaslt.h>

#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace salad {

namespace {

constexpr int kMaxDevices = 64;

struct GemmPlan {
  int bf16;
  long long rows;
  int C;
  hipblasLtMatmulDesc_t desc;
  hipblasLtMatrixLayout_t la, lb, ld;
  hipblasLtMatmulAlgo_t algo;
};

struct DeviceBlas {
  hipblasLtHandle_t handle = nullptr;
  std::vector<GemmPlan> plans;
};

std::mutex g_blas_lock;
DeviceBlas g_dev[kMaxDevices];

const char *blas_message(hipblasStatus_t st) {
  switch (st) {
    case HIPBLAS_STATUS_SUCCESS: return nullptr;
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "hipBLASLt: not initialised";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "hipBLASLt: allocation failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "hipBLASLt: invalid value";
    case HIPBLAS_STATUS_ARCH_MISMATCH: return "hipBLASLt: architecture mismatch";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "hipBLASLt: execution failed";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "hipBLASLt: not supported for these types";
    default: return "hipBLASLt: call failed";
  }
}

#define BLAS_TRY(x)                                          \
  do {                                                       \
    if (const char *_m = blas_message(x)) return _m;         \
  } while (0)

// Row-major out[rows, C] = a[rows, C] W[C, C] (+ beta out).  In the
// library's column-major terms the row-major matrices are their transposes:
// out^T [C, rows] = W^T [C, C] a^T [C, rows], i.e. m = C, n = rows, k = C,
// no transposition, every leading dimension C.  C and D are the same
// matrix (in place).
const char *make_plan(hipblasLtHandle_t h, int bf16, long long rows, int C, GemmPlan *pl) {
  const hipDataType t = bf16 ? HIP_R_16BF : HIP_R_32F;
  pl->bf16 = bf16;
  pl->rows = rows;
  pl->C = C;
  BLAS_TRY(hipblasLtMatmulDescCreate(&pl->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F));
  const hipblasOperation_t op = HIPBLAS_OP_N;
  BLAS_TRY(hipblasLtMatmulDescSetAttribute(pl->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op, sizeof op));
  BLAS_TRY(hipblasLtMatmulDescSetAttribute(pl->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op, sizeof op));
  BLAS_TRY(hipblasLtMatrixLayoutCreate(&pl->la, t, C, C, C));
  BLAS_TRY(hipblasLtMatrixLayoutCreate(&pl->lb, t, C, rows, C));
  BLAS_TRY(hipblasLtMatrixLayoutCreate(&pl->ld, t, C, rows, C));
  hipblasLtMatmulPreference_t pref;
  BLAS_TRY(hipblasLtMatmulPreferenceCreate(&pref));
  const size_t no_ws = 0;
  hipblasLtMatmulHeuristicResult_t res[8];
  int n = 0;
  hipblasStatus_t st = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                             &no_ws, sizeof no_ws);
  if (st == HIPBLAS_STATUS_SUCCESS)
    st = hipblasLtMatmulAlgoGetHeuristic(h, pl->desc, pl->la, pl->lb, pl->ld, pl->ld, pref, 8, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  BLAS_TRY(st);
  for (int i = 0; i < n; ++i)
    if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize == 0) {
      pl->algo = res[i].algo;
      return nullptr;
    }
  return "hipBLASLt: no algorithm without workspace for this shape";
}

}  // namespace

const char *gemm_rows(int bf16, long long rows, int C, const void *a, const void *w, float beta,
                      void *out, hipStream_t st) {
  if (rows == 0) return nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return "gemm: no current HIP device";
  std::lock_guard<std::mutex> lock(g_blas_lock);
  DeviceBlas &d = g_dev[dev];
  if (!d.handle) BLAS_TRY(hipblasLtCreate(&d.handle));
  const GemmPlan *pl = nullptr;
  for (const GemmPlan &p : d.plans)
    if (p.bf16 == bf16 && p.rows == rows && p.C == C) pl = &p;
  if (!pl) {
    GemmPlan np;
    if (const char *m = make_plan(d.handle, bf16, rows, C, &np)) return m;
    d.plans.push_back(np);
    pl = &d.plans.back();
  }
  const float alpha = 1.f;
  return blas_message(hipblasLtMatmul(d.handle, pl->desc, &alpha, w, pl->la, a, pl->lb, &beta, out, pl->ld,
                                      out, pl->ld, &pl->algo, nullptr, 0, st));
}

}  // namespace salad
