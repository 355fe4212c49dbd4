// Dense projections of the RNN layer: the skinny MFMA kernel of gemv.hip for few rows (decode
// steps), hipBLASLt for the prefill's long products.
//
// The layer around the mixer ("Hybrid Linear Attention Done Right", Appendix A, Eq. 18) has two
// plain GEMMs: x [W_q | W_k | W_v | W_z] in front of the mixer and the output projection W_o^T
// behind it.  Both are written here as D[M][N] = A[M][K] W[N][K]^T with row-major operands (K
// contiguous in both, the "TN" form the MFMA GEMMs of hipBLASLt stream best) and fp32
// accumulation; D is stored in the activation dtype.
//
// One hipBLASLt handle is created per device on first use, and the descriptors plus the
// heuristic's first algorithm are cached per (device, M, N, K, dtype, workspace limit), so a
// steady-state call costs one hipblasLtMatmul.  Both caches live until the process ends; access
// is serialised by a mutex, the GEMMs themselves are enqueued outside it.
#include <hipblaslt/hipblaslt.h>

#include <mutex>
#include <vector>

#include "lt_internal.h"

namespace lt {
namespace {

struct GemmPlan {
    int device;
    int64_t M, N, K;
    int dtype;
    size_t ws_limit;
    hipblasLtMatmulDesc_t desc;
    hipblasLtMatrixLayout_t a, b, c;
    hipblasLtMatmulAlgo_t algo;
    size_t ws_need;
};

std::mutex g_mutex;
std::vector<std::pair<int, hipblasLtHandle_t>> g_handles;
std::vector<GemmPlan> g_plans;

hipblasLtHandle_t handle_for(int device) {
    for (auto& e : g_handles)
        if (e.first == device) return e.second;
    hipblasLtHandle_t h = nullptr;
    if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return nullptr;
    g_handles.emplace_back(device, h);
    return h;
}

void destroy(GemmPlan& p) {
    if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
    if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
    if (p.c) hipblasLtMatrixLayoutDestroy(p.c);
    if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
}

// Column-major view used by hipBLASLt: D^T (N x M, ld N) = op(W) (N x K) * op(A) (K x M), where
// W row-major [N][K] is the column-major K x N matrix transposed (TRANSA = T) and A row-major
// [M][K] is the column-major K x M matrix as is (TRANSB = N).
lt_status make_plan(hipblasLtHandle_t h, GemmPlan& p) {
    const hipDataType t = p.dtype == LT_BF16 ? HIP_R_16BF : HIP_R_32F;
    if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
        return LT_ERR_HIP;
    const int32_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
    if (hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof opT) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof opN) !=
            HIPBLAS_STATUS_SUCCESS)
        return LT_ERR_HIP;
    if (hipblasLtMatrixLayoutCreate(&p.a, t, p.K, p.N, p.K) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.b, t, p.K, p.M, p.K) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.c, t, p.N, p.M, p.N) != HIPBLAS_STATUS_SUCCESS)
        return LT_ERR_HIP;
    hipblasLtMatmulPreference_t pref = nullptr;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return LT_ERR_HIP;
    const uint64_t limit = p.ws_limit;
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    hipblasStatus_t st = hipblasLtMatmulPreferenceSetAttribute(
        pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &limit, sizeof limit);
    if (st == HIPBLAS_STATUS_SUCCESS)
        st = hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.a, p.b, p.c, p.c, pref, 1, res, &found);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (st != HIPBLAS_STATUS_SUCCESS && st != HIPBLAS_STATUS_NOT_SUPPORTED) return LT_ERR_HIP;
    if (found < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS) return LT_ERR_UNSUPPORTED;
    p.algo = res[0].algo;
    p.ws_need = res[0].workspaceSize;
    return LT_OK;
}

}  // namespace

size_t gemm_workspace_limit() { return size_t(32) << 20; }

lt_status gemm_xwt(const void* A, const void* W, void* D, int64_t M, int64_t N, int64_t K,
                   int dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (launch_gate() != hipSuccess) return LT_ERR_HIP;
    if (M <= kSkinnyMaxRows) {
        if (N > 0x7fffffffLL || K > 0x7fffffffLL) return LT_ERR_UNSUPPORTED;
        return launch_skinny_gemm(A, W, D, (int)M, (int)N, (int)K, (int)K, (int)K, (int)N, dtype,
                                  stream) == hipSuccess
                   ? LT_OK
                   : LT_ERR_HIP;
    }
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return LT_ERR_HIP;
    hipblasLtHandle_t h;
    GemmPlan plan;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        h = handle_for(device);
        if (h == nullptr) return LT_ERR_HIP;
        const GemmPlan* hit = nullptr;
        for (const auto& p : g_plans)
            if (p.device == device && p.M == M && p.N == N && p.K == K && p.dtype == dtype &&
                p.ws_limit == ws_bytes) {
                hit = &p;
                break;
            }
        if (hit) {
            plan = *hit;
        } else {
            GemmPlan p{};
            p.device = device; p.M = M; p.N = N; p.K = K; p.dtype = dtype; p.ws_limit = ws_bytes;
            const lt_status st = make_plan(h, p);
            if (st != LT_OK) {
                destroy(p);
                return st;
            }
            g_plans.push_back(p);
            plan = p;
        }
    }
    const float alpha = 1.0f, beta = 0.0f;
    if (hipblasLtMatmul(h, plan.desc, &alpha, W, plan.a, A, plan.b, &beta, D, plan.c, D, plan.c,
                        &plan.algo, ws, plan.ws_need, stream) != HIPBLAS_STATUS_SUCCESS)
        return LT_ERR_HIP;
    return LT_OK;
}

}  // namespace lt
