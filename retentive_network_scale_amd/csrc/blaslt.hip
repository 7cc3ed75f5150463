// Plain bf16 GEMMs through hipBLASLt: the gated layer's projections ("Retentive
// Network" paper summary, Sec. 2.2: X W_Q, X W_K, X W_V, X W_G and the output
// projection) and the block's FFN (gelu(X W_1) W_2).  These products carry no
// fused arithmetic beyond a residual add -- the layer reads its operands back
// through strides and applies swish in the retention epilogue -- so a library GEMM
// is used for them; everything specific to retention runs in this library's own
// kernels.
//
//   C[t][n] = sum_k X[t][k] W[n][k] (+ R[t][n])   (row-major, bf16 in, bf16 or
//                                                  fp32 out, fp32 accumulate;
//                                                  R optional, bf16 out only)
//
// In hipBLASLt's column-major terms this is C^T (N x T, ld ldc) = W (N x K) * X^T
// (K x T), with W given as its stored K x N column-major transpose: a "TN" product.
// One handle per device and one plan (descriptors + chosen algorithm) per shape
// are created on first use and kept until the process ends.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "launch.hpp"

namespace ret {
namespace {

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
  size_t ws = 0;
  bool ok = false;
};

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<std::tuple<int, int, int, int, int, size_t, bool>, Plan> g_plans;

// Builds (or finds) the plan for this device and shape; nullptr when hipBLASLt has no algorithm for it.
const Plan *get_plan(int dev, hipblasLtHandle_t *handle, int T, int N, int K, int ldc, size_t ws_bytes,
                     bool out_f32) {
  std::lock_guard<std::mutex> lock(g_mu);
  auto hit = g_handles.find(dev);
  if (hit == g_handles.end()) {
    hipblasLtHandle_t h = nullptr;
    if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return nullptr;
    hit = g_handles.emplace(dev, h).first;
  }
  *handle = hit->second;
  const auto key = std::make_tuple(dev, T, N, K, ldc, ws_bytes, out_f32);
  auto pit = g_plans.find(key);
  if (pit != g_plans.end()) return pit->second.ok ? &pit->second : nullptr;
  Plan p;
  bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)) ==
                 HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, T, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.lc, out_f32 ? HIP_R_32F : HIP_R_16BF, N, T, ldc) ==
                 HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t max_ws = ws_bytes;
    hipblasLtMatmulHeuristicResult_t res[1];
    int n = 0;
    ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &max_ws,
                                               sizeof(max_ws)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulAlgoGetHeuristic(*handle, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &n) ==
             HIPBLAS_STATUS_SUCCESS &&
         n > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize <= ws_bytes;
    if (ok) {
      p.algo = res[0].algo;
      p.ws = res[0].workspaceSize;
    }
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  }
  p.ok = ok;
  auto ins = g_plans.emplace(key, p).first;
  return ok ? &ins->second : nullptr;
}

}  // namespace

hipError_t blaslt_gemm_nt(const uint16_t *X, const uint16_t *W, void *C, int T, int N, int K, int ldc, void *ws,
                          size_t ws_bytes, hipStream_t st, const uint16_t *R, bool out_f32) {
  if (R && out_f32) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  hipblasLtHandle_t handle = nullptr;
  const Plan *p = get_plan(dev, &handle, T, N, K, ldc, ws_bytes, out_f32);
  if (!p) return hipErrorNotSupported;
  const float alpha = 1.0f, beta = R ? 1.0f : 0.0f;
  const void *Cin = R ? (const void *)R : (const void *)C;
  const hipblasStatus_t s = hipblasLtMatmul(handle, p->desc, &alpha, W, p->la, X, p->lb, &beta, Cin, p->lc, C,
                                            p->lc, &p->algo, p->ws ? ws : nullptr, p->ws, st);
  return s == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace ret
