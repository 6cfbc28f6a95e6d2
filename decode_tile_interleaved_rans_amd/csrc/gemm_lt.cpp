// The plain BF16 GEMM of the compressed linear forward's decoded slices through hipBLASLt, the
// ROCm GEMM library, at prefill sizes: its tuned kernels run the same MFMA work faster than the
// library's own 256 x 256 kernel there (4096 x 8192 x 8192: 363 against 441 us). The decode, the
// part this library adds, stays in its own kernels; the product of a decoded slice with X is an
// ordinary GEMM.
//
// Y[M][N] = X[M][K] W[N][K]^T (+ bias) in hipBLASLt's column-major terms: D (N x M, leading
// dimension ldy) = op(A) B with A = W seen as K x N (ld ldw) and op(A) = A^T, B = X seen as K x M
// (ld ldx), fp32 accumulation and scale, BF16 D; the bias epilogue adds bias[n] to row n of D.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "gemm.h"

namespace ep {
namespace {

struct LtPlan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
    bool ok = false;
};

using LtKey = std::tuple<int, int, int, int, int, int, int, bool, size_t>;

std::mutex g_mu;                                   // guards the maps and each plan's bias attribute
std::map<int, hipblasLtHandle_t> g_handles;        // per device, kept until the process ends
std::map<LtKey, LtPlan> g_plans;

LtPlan make_plan(hipblasLtHandle_t h, const GemmArgs& g, size_t ws_bytes) {
    LtPlan p;
    if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return p;
    const int32_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta);
    hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb);
    if (g.bias) {
        const uint32_t epi = HIPBLASLT_EPILOGUE_BIAS;
        const int32_t bt = HIP_R_16BF;
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof epi);
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt, sizeof bt);
        const void* bp = g.bias;
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bp, sizeof bp);
    }
    if (hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, (uint64_t)g.K, (uint64_t)g.N, g.ldw) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, (uint64_t)g.K, (uint64_t)g.M, g.ldx) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.d, HIP_R_16BF, (uint64_t)g.N, (uint64_t)g.M, g.ldy) != HIPBLAS_STATUS_SUCCESS)
        return p;
    hipblasLtMatmulPreference_t pref = nullptr;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return p;
    const uint64_t ws = ws_bytes;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof ws);
    hipblasLtMatmulHeuristicResult_t res[1];
    int n = 0;
    const hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.a, p.b, p.d, p.d, pref, 1, res, &n);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (st != HIPBLAS_STATUS_SUCCESS || n < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS || res[0].workspaceSize > ws_bytes)
        return p;
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    p.ok = true;
    return p;
}

}  // namespace

hipError_t lt_gemm(const GemmArgs& g, void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_mu);
    hipblasLtHandle_t& h = g_handles[dev];
    if (!h && hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) {
        h = nullptr;
        return hipErrorNotSupported;
    }
    const LtKey key{dev, g.M, g.N, g.K, g.ldx, g.ldw, g.ldy, g.bias != nullptr, ws_bytes};
    auto it = g_plans.find(key);
    if (it == g_plans.end()) it = g_plans.emplace(key, make_plan(h, g, ws_bytes)).first;
    LtPlan& p = it->second;
    if (!p.ok) return hipErrorNotSupported;
    if (g.bias) {                                  // the slice's bias (the plan is per shape)
        const void* bp = g.bias;
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bp, sizeof bp);
    }
    const float alpha = 1.0f, beta = 0.0f;
    const hipblasStatus_t st = hipblasLtMatmul(h, p.desc, &alpha, g.W, p.a, g.X, p.b, &beta, g.Y, p.d, g.Y, p.d,
                                               &p.algo, p.ws ? workspace : nullptr, p.ws, stream);
    return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace ep
