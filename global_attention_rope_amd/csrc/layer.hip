// layer.hip — the attention layer with its projections: q/k/v projections, the hybrid attention
// prefill of this library, and the output projection with the value rescale folded into it.
//
// Pages: "Add Xiaomi MiMo-V2", section "Additional useful info" (the value head dim is separate
// from the QK head dim, so the output projection maps Hq * v_head_dim back to the hidden size; the
// values are rescaled by sqrt(hidden / (heads * v_head_dim))).  By linearity the rescale of the
// attention output equals the same scale of the output projection, so it rides on the last GEMM's
// alpha.  The projections are plain dense products and run on hipBLASLt (bf16 operands, fp32
// accumulation); the attention between them is this library's own kernels.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <math.h>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "mimo_attn.h"
#include "kernels.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kGemmWorkspace = (size_t)32 << 20;   // hipBLASLt scratch inside the workspace

std::mutex g_lt_mu;
hipblasLtHandle_t g_lt[kMaxDevices];

int layer_fail(int code, const char* fmt, ...) {
    char msg[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    return mimo::set_error(code, msg);
}

// One hipBLASLt handle per device, created on first use and kept until the process ends.
hipblasLtHandle_t lt_handle() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_lt_mu);
    if (!g_lt[dev] && hipblasLtCreate(&g_lt[dev]) != HIPBLAS_STATUS_SUCCESS) g_lt[dev] = nullptr;
    return g_lt[dev];
}

// Row-major Y[M, N] = alpha * X[M, K] * W[K, N], bf16 operands and result, fp32 accumulation.
// (In hipBLASLt's column-major terms: Y^T = W^T * X^T, W^T being W's row-major storage.)
hipblasStatus_t gemm_rm(hipblasLtHandle_t h, int64_t M, int64_t N, int64_t K, const void* X,
                        const void* W, void* Y, float alpha, void* ws, size_t ws_bytes,
                        hipStream_t st) {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    hipblasStatus_t rc = hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
    const hipblasOperation_t op = HIPBLAS_OP_N;
    const uint64_t wsb = ws_bytes;
    if (rc == HIPBLAS_STATUS_SUCCESS)
        rc = hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op, sizeof op);
    if (rc == HIPBLAS_STATUS_SUCCESS)
        rc = hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op, sizeof op);
    if (rc == HIPBLAS_STATUS_SUCCESS) rc = hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, N, K, N);
    if (rc == HIPBLAS_STATUS_SUCCESS) rc = hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, K, M, K);
    if (rc == HIPBLAS_STATUS_SUCCESS) rc = hipblasLtMatrixLayoutCreate(&lc, HIP_R_16BF, N, M, N);
    if (rc == HIPBLAS_STATUS_SUCCESS) rc = hipblasLtMatmulPreferenceCreate(&pref);
    if (rc == HIPBLAS_STATUS_SUCCESS)
        rc = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                   &wsb, sizeof wsb);
    hipblasLtMatmulHeuristicResult_t res;
    int found = 0;
    if (rc == HIPBLAS_STATUS_SUCCESS)
        rc = hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, lc, lc, pref, 1, &res, &found);
    if (rc == HIPBLAS_STATUS_SUCCESS && found < 1) rc = HIPBLAS_STATUS_NOT_SUPPORTED;
    const float beta = 0.0f;
    if (rc == HIPBLAS_STATUS_SUCCESS)
        rc = hipblasLtMatmul(h, desc, &alpha, W, la, X, lb, &beta, Y, lc, Y, lc, &res.algo, ws,
                             ws_bytes, st);
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (lc) hipblasLtMatrixLayoutDestroy(lc);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (desc) hipblasLtMatmulDescDestroy(desc);
    return rc;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

struct LayerBuffers {
    size_t q, k, v, attn, gemm, attn_ws, total;   // byte offsets (total: bytes)
};

LayerBuffers layer_buffers(const mimo_attn_params* p, int32_t S) {
    const size_t T = (size_t)p->batch * S;
    LayerBuffers L;
    L.q = 0;
    L.k = L.q + align256(T * p->num_q_heads * p->qk_head_dim * 2);
    L.v = L.k + align256(T * p->num_kv_heads * p->qk_head_dim * 2);
    L.attn = L.v + align256(T * p->num_kv_heads * p->v_head_dim * 2);
    L.gemm = L.attn + align256(T * p->num_q_heads * p->v_head_dim * 2);
    L.attn_ws = L.gemm + kGemmWorkspace;
    L.total = L.attn_ws + align256(mimo_attn_prefill_workspace_size(p, S));
    return L;
}

}  // namespace

extern "C" {

size_t mimo_attn_layer_workspace_size(const mimo_attn_params* p, int32_t hidden, int32_t seq_len) {
    if (mimo_attn_check_params(p) != MIMO_OK || hidden < 1 || seq_len < 0 ||
        p->dtype != MIMO_BF16)
        return 0;
    return layer_buffers(p, seq_len).total;
}

int mimo_attn_layer_prefill(const mimo_attn_params* p, int32_t hidden, int32_t seq_len,
                            const void* x, const void* w_q, const void* w_k, const void* w_v,
                            const void* w_o, int32_t out_dim, const int32_t* start_pos,
                            const float* sinks, void* out, void* k_cache, void* v_cache,
                            int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                            void* stream) {
    int rc = mimo_attn_check_params(p);
    if (rc != MIMO_OK) return rc;   // (message already set)
    if (p->dtype != MIMO_BF16)
        return layer_fail(MIMO_ERR_UNSUPPORTED, "the layer entry point is compiled for bf16 only");
    if (hidden < 1 || out_dim < 1 || seq_len < 0)
        return layer_fail(MIMO_ERR_INVALID_ARG, "hidden %d, out_dim %d, seq_len %d", hidden,
                          out_dim, seq_len);
    if (p->batch == 0 || seq_len == 0) {
        mimo::clear_error();
        return MIMO_OK;
    }
    if (!x || !w_q || !w_k || !w_v || !w_o || !start_pos || !out)
        return layer_fail(MIMO_ERR_INVALID_ARG, "x, weights, start_pos and out must be non-NULL");
    const LayerBuffers L = layer_buffers(p, seq_len);
    if (!workspace || workspace_bytes < L.total)
        return layer_fail(MIMO_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", L.total,
                          workspace ? workspace_bytes : (size_t)0);
    hipblasLtHandle_t h = lt_handle();
    if (!h) return layer_fail(MIMO_ERR_HIP, "hipBLASLt handle could not be created");
    hipStream_t st = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    void *q = ws + L.q, *k = ws + L.k, *v = ws + L.v, *attn = ws + L.attn;
    void* gws = ws + L.gemm;
    const int64_t T = (int64_t)p->batch * seq_len;
    const int64_t nq = (int64_t)p->num_q_heads * p->qk_head_dim;
    const int64_t nk = (int64_t)p->num_kv_heads * p->qk_head_dim;
    const int64_t nv = (int64_t)p->num_kv_heads * p->v_head_dim;
    const int64_t na = (int64_t)p->num_q_heads * p->v_head_dim;
    const struct {
        const void* w;
        void* y;
        int64_t n;
    } proj[3] = {{w_q, q, nq}, {w_k, k, nk}, {w_v, v, nv}};
    for (const auto& pr : proj) {
        const hipblasStatus_t s = gemm_rm(h, T, pr.n, hidden, x, pr.w, pr.y, 1.0f, gws,
                                          kGemmWorkspace, st);
        if (s != HIPBLAS_STATUS_SUCCESS)
            return layer_fail(MIMO_ERR_HIP, "projection GEMM failed (hipBLASLt status %d)", (int)s);
    }
    // attention without the value rescale, which the output projection applies
    mimo_attn_params pa = *p;
    pa.v_scale = 1.0f;
    rc = mimo_attn_prefill(&pa, seq_len, q, k, v, start_pos, sinks, attn, k_cache, v_cache,
                           cache_capacity, ws + L.attn_ws, L.total - L.attn_ws, stream);
    if (rc != MIMO_OK) return rc;   // (message already set)
    const hipblasStatus_t s =
        gemm_rm(h, T, out_dim, na, attn, w_o, out, p->v_scale, gws, kGemmWorkspace, st);
    if (s != HIPBLAS_STATUS_SUCCESS)
        return layer_fail(MIMO_ERR_HIP, "output GEMM failed (hipBLASLt status %d)", (int)s);
    mimo::clear_error();
    return MIMO_OK;
}

}  // extern "C"
