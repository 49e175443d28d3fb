// Dense projections around the attention core (ZGCM-1 paper summaries: onedev.kr "How it works": the gated
// layer is o_proj(A_SWA(q, k, v) (.) sigmoid(g_proj(h))), with q/k/v/g projections of the hidden state h).
// These are plain GEMMs, run on hipBLASLt: y[T][N] = x[T][K] . W[N][K]^T (a linear layer's forward, W stored
// out_features x in_features), fp32 accumulation, bf16 result; operands bf16, or E4M3 with per-tensor scales.
//
// hipBLASLt is column-major: the row-major y[T][N] is the column-major N x T matrix D = op(A) op(B) with A = W
// read as the column-major K x N matrix (transposed: op(A) = W, N x K) and B = x read as the column-major
// K x T matrix (not transposed).
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "linear.h"

namespace zg {
namespace {

constexpr size_t kBlasWorkspace = 64ull << 20;   // hipBLASLt workspace per device

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo{};
};

struct DeviceBlas {
  hipblasLtHandle_t handle = nullptr;
  void* ws = nullptr;
  std::map<std::tuple<int, int64_t, int32_t, int32_t>, Plan> plans;   // (fp8?, T, K, N)
};

std::mutex g_mu;
std::map<int, DeviceBlas> g_dev;

// Handle, workspace and plan for this device and shape, created on first use and kept until the process
// ends.  Returns a hipblasStatus_t value (0 = success).
int get_plan(bool fp8, int64_t T, int32_t K, int32_t N, DeviceBlas** dev_out, Plan** plan_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return HIPBLAS_STATUS_NOT_INITIALIZED;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceBlas& d = g_dev[dev];
  if (!d.handle) {
    hipblasStatus_t s = hipblasLtCreate(&d.handle);
    if (s != HIPBLAS_STATUS_SUCCESS) { d.handle = nullptr; return s; }
    if (hipMalloc(&d.ws, kBlasWorkspace) != hipSuccess) {
      hipblasLtDestroy(d.handle);
      d.handle = nullptr;
      d.ws = nullptr;
      return HIPBLAS_STATUS_ALLOC_FAILED;
    }
  }
  const auto key = std::make_tuple(fp8 ? 1 : 0, T, K, N);
  auto it = d.plans.find(key);
  if (it == d.plans.end()) {
    Plan p;
    hipblasStatus_t s = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
    const int32_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof opT);
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof opN);
    const hipDataType in = fp8 ? HIP_R_8F_E4M3 : HIP_R_16BF;
    if (fp8 && s == HIPBLAS_STATUS_SUCCESS) {
      // placeholder scale pointers so the heuristic sees a scaled FP8 problem; each call sets its own
      static float one = 1.0f;
      const void* pa = &one;
      s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_A_SCALE_POINTER, &pa, sizeof pa);
      if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_B_SCALE_POINTER, &pa, sizeof pa);
    }
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&p.la, in, (uint64_t)K, (uint64_t)N, (int64_t)K);
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&p.lb, in, (uint64_t)K, (uint64_t)T, (int64_t)K);
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&p.ld, HIP_R_16BF, (uint64_t)N, (uint64_t)T, (int64_t)N);
    hipblasLtMatmulPreference_t pref = nullptr;
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatmulPreferenceCreate(&pref);
    const uint64_t wsb = kBlasWorkspace;
    if (s == HIPBLAS_STATUS_SUCCESS)
      s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof wsb);
    hipblasLtMatmulHeuristicResult_t res[1];
    int n = 0;
    if (s == HIPBLAS_STATUS_SUCCESS)
      s = hipblasLtMatmulAlgoGetHeuristic(d.handle, p.desc, p.la, p.lb, p.ld, p.ld, pref, 1, res, &n);
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (s == HIPBLAS_STATUS_SUCCESS && n < 1) s = HIPBLAS_STATUS_NOT_SUPPORTED;
    if (s != HIPBLAS_STATUS_SUCCESS) {
      if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
      if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
      if (p.ld) hipblasLtMatrixLayoutDestroy(p.ld);
      if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
      return s;
    }
    p.algo = res[0].algo;
    it = d.plans.emplace(key, p).first;
  }
  *dev_out = &d;
  *plan_out = &it->second;
  return HIPBLAS_STATUS_SUCCESS;
}

}  // namespace

int linear_bf16_run(const void* x, const void* w, void* y, int64_t T, int32_t K, int32_t N, hipStream_t st) {
  DeviceBlas* d = nullptr;
  Plan* p = nullptr;
  int s = get_plan(false, T, K, N, &d, &p);
  if (s != HIPBLAS_STATUS_SUCCESS) return s;
  const float alpha = 1.0f, beta = 0.0f;
  return hipblasLtMatmul(d->handle, p->desc, &alpha, w, p->la, x, p->lb, &beta, y, p->ld, y, p->ld, &p->algo, d->ws,
                         kBlasWorkspace, st);
}

int linear_fp8_run(const void* xq, const void* wq, void* y, int64_t T, int32_t K, int32_t N, const float* x_scale_inv,
                   const float* w_scale_inv, hipStream_t st) {
  DeviceBlas* d = nullptr;
  Plan* p = nullptr;
  int s = get_plan(true, T, K, N, &d, &p);
  if (s != HIPBLAS_STATUS_SUCCESS) return s;
  // the scale pointers live in the shared plan: set them and enqueue under the lock
  std::lock_guard<std::mutex> lk(g_mu);
  const void* pa = w_scale_inv;   // A = W
  const void* pb = x_scale_inv;   // B = x
  s = hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_A_SCALE_POINTER, &pa, sizeof pa);
  if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_B_SCALE_POINTER, &pb, sizeof pb);
  if (s != HIPBLAS_STATUS_SUCCESS) return s;
  const float alpha = 1.0f, beta = 0.0f;
  return hipblasLtMatmul(d->handle, p->desc, &alpha, wq, p->la, xq, p->lb, &beta, y, p->ld, y, p->ld, &p->algo, d->ws,
                         kBlasWorkspace, st);
}

const char* blas_status_name(int s) {
  switch (s) {
    case HIPBLAS_STATUS_SUCCESS: return "success";
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "not initialized";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "allocation failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "invalid value";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "execution failed";
    case HIPBLAS_STATUS_INTERNAL_ERROR: return "internal error";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "not supported";
    case HIPBLAS_STATUS_ARCH_MISMATCH: return "architecture mismatch";
    default: return "hipBLASLt error";
  }
}

}  // namespace zg
