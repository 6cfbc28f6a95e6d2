// The plain BF16 GEMM of the compressed linear forward's decoded slices through hipBLASLt, the
// ROCm GEMM library, at prefill sizes: its tuned kernels run the same MFMA work faster than the
// library's own 256 x 256 kernel there (4096 x 8192 x 8192: 363 against 441 us). The decode, the
// part this library adds, stays in its own kernels; the product of a decoded slice with X is an
// ordinary GEMM.
//
// Y[M][N] = X[M][K] W[N][K]^T (+ bias) in hipBLASLt's column-major terms: D (N x M, leading
// dimension ldy) = op(A) B with A = W seen as K x N (ld ldw) and op(A) = A^T, B = X seen as K x M
// (ld ldx), fp32 accumulation and scale, BF16 D; the bias epilogue adds bias[n] to row n of D.
// FP8 (the FP8 forward's slices): A and B hold OCP E4M3 codes, and the outer-vector scale mode
// multiplies element (n, m) of the product by the weight row scale s_w[n] (A's vector) and the
// activation row scale s_x[m] (B's vector) before the bias.
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
    uint64_t tick = 0;         // last use, for eviction
};

// Plans kept at most: a caller whose row count varies from call to call (serving with variable
// token counts) would otherwise add a plan, and a heuristic query, per distinct M for ever.
constexpr size_t kMaxPlans = 128;

void destroy(LtPlan& p) {
    if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
    if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
    if (p.d) hipblasLtMatrixLayoutDestroy(p.d);
    if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
    p = LtPlan{};
}

using LtKey = std::tuple<int, int, int, int, int, int, int, bool, bool, size_t>;

struct LtShape {
    int M, N, K, ldx, ldw, ldy;
    bool bias, f8;
};

std::mutex g_mu;                                   // guards the maps and each plan's pointer attributes
std::map<int, hipblasLtHandle_t> g_handles;        // per device, kept until the process ends
std::map<LtKey, LtPlan> g_plans;
uint64_t g_tick = 0;

// Pointers a call sets on the shared descriptor (under the lock): bias and the FP8 scale vectors.
void set_pointers(hipblasLtMatmulDesc_t d, const void* bias, const void* sa, const void* sb) {
    if (bias) hipblasLtMatmulDescSetAttribute(d, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof bias);
    if (sa) hipblasLtMatmulDescSetAttribute(d, HIPBLASLT_MATMUL_DESC_A_SCALE_POINTER, &sa, sizeof sa);
    if (sb) hipblasLtMatmulDescSetAttribute(d, HIPBLASLT_MATMUL_DESC_B_SCALE_POINTER, &sb, sizeof sb);
}

LtPlan make_plan(hipblasLtHandle_t h, const LtShape& g, size_t ws_bytes, const void* bias, const void* sa,
                 const void* sb) {
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
    }
    if (g.f8) {
        const int32_t mode = HIPBLASLT_MATMUL_MATRIX_SCALE_OUTER_VEC_32F;
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_A_SCALE_MODE, &mode, sizeof mode);
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_B_SCALE_MODE, &mode, sizeof mode);
    }
    set_pointers(p.desc, bias, sa, sb);
    const hipDataType in = g.f8 ? HIP_R_8F_E4M3 : HIP_R_16BF;
    if (hipblasLtMatrixLayoutCreate(&p.a, in, (uint64_t)g.K, (uint64_t)g.N, g.ldw) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.b, in, (uint64_t)g.K, (uint64_t)g.M, g.ldx) != HIPBLAS_STATUS_SUCCESS ||
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

hipError_t run(const LtShape& s, const void* W, const void* X, void* Y, const void* bias, const void* sa,
               const void* sb, void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (s.M <= 0 || s.N <= 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_mu);
    hipblasLtHandle_t& h = g_handles[dev];
    if (!h && hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) {
        h = nullptr;
        return hipErrorNotSupported;
    }
    const LtKey key{dev, s.M, s.N, s.K, s.ldx, s.ldw, s.ldy, s.bias, s.f8, ws_bytes};
    auto it = g_plans.find(key);
    if (it == g_plans.end()) {
        if (g_plans.size() >= kMaxPlans) {
            // the least recently used plan goes; descriptors are host objects that a queued
            // matmul no longer reads once hipblasLtMatmul has returned
            auto lru = g_plans.begin();
            for (auto j = g_plans.begin(); j != g_plans.end(); ++j)
                if (j->second.tick < lru->second.tick) lru = j;
            destroy(lru->second);
            g_plans.erase(lru);
        }
        it = g_plans.emplace(key, make_plan(h, s, ws_bytes, bias, sa, sb)).first;
    }
    LtPlan& p = it->second;
    p.tick = ++g_tick;
    if (!p.ok) return hipErrorNotSupported;
    set_pointers(p.desc, bias, sa, sb);            // this call's vectors (the plan is per shape)
    const float alpha = 1.0f, beta = 0.0f;
    const hipblasStatus_t st = hipblasLtMatmul(h, p.desc, &alpha, W, p.a, X, p.b, &beta, Y, p.d, Y, p.d, &p.algo,
                                               p.ws ? workspace : nullptr, p.ws, stream);
    return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace

hipError_t lt_gemm(const GemmArgs& g, void* workspace, size_t ws_bytes, hipStream_t stream) {
    const LtShape s{g.M, g.N, g.K, g.ldx, g.ldw, g.ldy, g.bias != nullptr, false};
    return run(s, g.W, g.X, g.Y, g.bias, nullptr, nullptr, workspace, ws_bytes, stream);
}

hipError_t lt_gemm_f8(const GemmF8Args& g, void* workspace, size_t ws_bytes, hipStream_t stream) {
    const LtShape s{g.M, g.N, g.K, g.ldx, g.ldw, g.ldy, g.bias != nullptr, true};
    return run(s, g.W, g.X, g.Y, g.bias, g.sw, g.sx, workspace, ws_bytes, stream);
}

}  // namespace ep
