// shared_blas.cpp -- the bf16 shared expert of prefill-sized batches as two
// plain dense GEMMs in hipBLASLt (the Kimi-K2.6 catalog entry's MoE paragraph:
// one always-on shared expert; QUANT: kept in higher precision, so it is an
// ordinary bf16 MLP):
//
//   g|u [T, 2I] fp32 = x [T, H] . Ws13^T      (then SwiGLU in swiglu_kernel)
//   s   [T, H]  fp32 = hs [T, I] . Ws2^T
//
// Weights are row-major [rows, K] and activations row-major [T, K]; in the
// library's column-major terms D' [rows, T] = W'^T [rows, K] . A' [K, T] with
// W' = the weights seen as [K, rows], A' = the activations seen as [K, T].
// bf16 inputs, fp32 accumulation and fp32 output. The handle is created once
// per device on first use; plans (descriptors and the heuristic's algorithm)
// are cached per shape.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "internal.h"

namespace moe {
namespace {

struct Plan {
  bool ok = false;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t w = nullptr, a = nullptr, d = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<std::tuple<int, int64_t, int64_t, int64_t>, Plan> g_plans;

bool make_plan(hipblasLtHandle_t h, int64_t rows, int64_t T, int64_t K, Plan& p) {
  if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
    return false;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  if (hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) !=
          HIPBLAS_STATUS_SUCCESS)
    return false;
  if (hipblasLtMatrixLayoutCreate(&p.w, HIP_R_16BF, K, rows, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, K, T, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.d, HIP_R_32F, rows, T, rows) != HIPBLAS_STATUS_SUCCESS)
    return false;
  hipblasLtMatmulPreference_t pref;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return false;
  const uint64_t max_ws = kSharedBlasWorkspace;
  hipblasLtMatmulHeuristicResult_t res[1];
  int n = 0;
  const bool found =
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                            &max_ws, sizeof(max_ws)) == HIPBLAS_STATUS_SUCCESS &&
      hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.w, p.a, p.d, p.d, pref, 1, res, &n) ==
          HIPBLAS_STATUS_SUCCESS &&
      n > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize <= max_ws;
  hipblasLtMatmulPreferenceDestroy(pref);
  if (!found) return false;
  p.algo = res[0].algo;
  p.ws = res[0].workspaceSize;
  return true;
}

}  // namespace

hipError_t launch_shared_blas(const uint16_t* weights, const uint16_t* act, float* out,
                              int64_t rows, int64_t T, int64_t K, void* workspace,
                              hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  Plan* plan = nullptr;
  hipblasLtHandle_t h = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto hit = g_handles.find(dev);
    if (hit == g_handles.end()) {
      if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return hipErrorNotSupported;
      g_handles[dev] = h;
    } else {
      h = hit->second;
    }
    const auto key = std::make_tuple(dev, rows, T, K);
    auto it = g_plans.find(key);
    if (it == g_plans.end()) {
      Plan p;
      p.ok = make_plan(h, rows, T, K, p);
      it = g_plans.emplace(key, p).first;
    }
    plan = &it->second;
  }
  if (!plan->ok) return hipErrorNotSupported;
  const float alpha = 1.0f, beta = 0.0f;
  const hipblasStatus_t st =
      hipblasLtMatmul(h, plan->desc, &alpha, weights, plan->w, act, plan->a, &beta, out, plan->d,
                      out, plan->d, &plan->algo, workspace, plan->ws, stream);
  return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace moe
