// layer.hip — the attention layer with its projections: q/k/v projections, the hybrid attention
// prefill of this library, and the output projection with the value rescale folded into it.
//
// Pages: "Add Xiaomi MiMo-V2", section "Additional useful info" (the value head dim is separate
// from the QK head dim, so the output projection maps Hq * v_head_dim back to the hidden size; the
// values are rescaled by sqrt(hidden / (heads * v_head_dim))).  By linearity the rescale of the
// attention output equals the same scale of the output projection, so it rides on the last
// product's alpha.  Every product runs on this library's bf16 MFMA kernel (csrc/gemm_bf16.hip).
//
// With the model's rotated width (64 of 192 dims) or none, the key projection's epilogue rotates
// the keys in fp32 and writes them straight into the attention's rotated-key layout and into the
// KV cache, and the value projection's epilogue stores the cache's values: no separate rotation
// pass and no second trip of the keys through memory.  Other rotated widths take the plain
// projection and the prefill's own key-rotation pass.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "mimo_attn.h"
#include "kernels.h"

namespace {

int layer_fail(int code, const char* fmt, ...) {
    char msg[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    return mimo::set_error(code, msg);
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

struct LayerBuffers {
    size_t q, k, v, attn, attn_ws, total;   // byte offsets (total: bytes)
};

// q [T, Hq*dqk], k [T, Hkv*dqk] (projected, before rotation), v [T, Hkv*dv], attention output
// [T, Hq*dv], then the prefill workspace (the rotated keys, [B, Hkv, S, dqk]).
LayerBuffers layer_buffers(const mimo_attn_params* p, int32_t S) {
    const size_t T = (size_t)p->batch * S;
    LayerBuffers L;
    L.q = 0;
    L.k = L.q + align256(T * p->num_q_heads * p->qk_head_dim * 2);
    L.v = L.k + align256(T * p->num_kv_heads * p->qk_head_dim * 2);
    L.attn = L.v + align256(T * p->num_kv_heads * p->v_head_dim * 2);
    L.attn_ws = L.attn + align256(T * p->num_q_heads * p->v_head_dim * 2);
    L.total = L.attn_ws + align256(mimo_attn_prefill_workspace_size(p, S));
    return L;
}

// Products sharing X[M, K] (row-major): part p is Y_p[M, N_p] = alpha * X W_p[K, N_p] with the
// plain epilogue until set otherwise.
mimo::GemmArgs gemm_args(int64_t M, int64_t K, const void* X, float alpha) {
    mimo::GemmArgs g;
    memset(&g, 0, sizeof g);
    g.A = (const uint16_t*)X;
    g.lda = K;
    g.M = (int32_t)M;
    g.K = (int32_t)K;
    g.alpha = alpha;
    return g;
}

void add_part(mimo::GemmArgs& g, const void* W, void* Y, int64_t N, int epilogue) {
    mimo::GemmPart& p = g.part[g.nparts++];
    p.B = (const uint16_t*)W;
    p.C = (uint16_t*)Y;
    p.ldb = p.ldc = N;
    p.N = (int32_t)N;
    p.epilogue = epilogue;
    p.code_inv = 1.0f;
}

int gemm_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MIMO_OK;
    return layer_fail(MIMO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
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
    // every argument check comes before the first launch, so an error enqueues nothing
    if ((k_cache == nullptr) != (v_cache == nullptr))
        return layer_fail(MIMO_ERR_INVALID_ARG, "k_cache and v_cache must both be set or both be NULL");
    const bool swa = p->layer_kind == MIMO_LAYER_SWA;
    if (k_cache) {
        if (cache_capacity < 1)
            return layer_fail(MIMO_ERR_INVALID_ARG, "cache_capacity must be >= 1");
        if (swa && cache_capacity != p->window)
            return layer_fail(MIMO_ERR_INVALID_ARG, "ring cache capacity %d must equal window %d",
                              cache_capacity, p->window);
    }
    const int64_t nq = (int64_t)p->num_q_heads * p->qk_head_dim;
    const int64_t nk = (int64_t)p->num_kv_heads * p->qk_head_dim;
    const int64_t nv = (int64_t)p->num_kv_heads * p->v_head_dim;
    const int64_t na = (int64_t)p->num_q_heads * p->v_head_dim;
    if (hidden % 64 || out_dim % 8)
        return layer_fail(MIMO_ERR_UNSUPPORTED,
                          "the projection kernel needs hidden %% 64 == 0 and out_dim %% 8 == 0 "
                          "(hidden %d, out_dim %d)", hidden, out_dim);
    const int64_t T = (int64_t)p->batch * seq_len;
    if (T > 0x7fffffffLL || (int64_t)seq_len * p->num_q_heads * p->batch > ((int64_t)1 << 40))
        return layer_fail(MIMO_ERR_INVALID_ARG, "problem too large");
    const LayerBuffers L = layer_buffers(p, seq_len);
    if (!workspace || workspace_bytes < L.total)
        return layer_fail(MIMO_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", L.total,
                          workspace ? workspace_bytes : (size_t)0);
    hipStream_t st = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    void *q = ws + L.q, *k = ws + L.k, *v = ws + L.v, *attn = ws + L.attn;
    void* kws = ws + L.attn_ws;   // rotated keys [B, Hkv, S, dqk]
    const bool fp8 = p->cache_dtype == MIMO_CACHE_FP8_E4M3;

    mimo_attn_params pa = *p;
    pa.v_scale = 1.0f;   // the output projection applies it
    mimo::GemmArgs g = gemm_args(T, hidden, x, 1.0f);
    add_part(g, w_q, q, nq, mimo::kGemmPlain);
    if (p->rope_dims != 0 && p->rope_dims != 64) {
        // other rotated widths: plain projections, then the prefill's own key-rotation pass
        add_part(g, w_k, k, nk, mimo::kGemmPlain);
        add_part(g, w_v, v, nv, mimo::kGemmPlain);
        rc = gemm_status(mimo::launch_gemm_bf16(g, st), "q/k/v projections");
        if (rc != MIMO_OK) return rc;
        rc = mimo_attn_prefill(&pa, seq_len, q, k, v, start_pos, sinks, attn, k_cache, v_cache,
                               cache_capacity, kws, L.total - L.attn_ws, stream);
        if (rc != MIMO_OK) return rc;   // (message already set)
    } else {
        // one launch for the three products; the key part's epilogue rotates the keys and writes
        // them in the attention's layout and the cache, the value part's the cache's values
        add_part(g, w_k, kws, nk, mimo::kGemmKey);
        add_part(g, w_v, v, nv, mimo::kGemmValue);
        g.part[1].cache = k_cache;
        g.part[2].cache = v_cache;
        g.part[1].code_inv = fp8 ? 1.0f / p->k_cache_scale : 1.0f;
        g.part[2].code_inv = fp8 ? 1.0f / p->v_cache_scale : 1.0f;
        g.S = seq_len;
        g.heads = p->num_kv_heads;
        g.dqk = p->qk_head_dim;
        g.dv = p->v_head_dim;
        g.start_pos = start_pos;
        g.cap = cache_capacity;
        g.ring_window = swa ? p->window : 0;
        g.cache_i0 = (swa && seq_len > p->window) ? seq_len - p->window : 0;   // ring: last W
        g.cache_fp8 = fp8;
        g.rope_dims = p->rope_dims;
        mimo::rope_omega_rev(p->rope_theta, p->rope_dims, g.omega_rev, 32);
        rc = gemm_status(mimo::launch_gemm_bf16(g, st), "q/k/v projections");
        if (rc != MIMO_OK) return rc;
        // the attention over the rotated keys (the prefill kernel rotates the queries itself)
        mimo::PrefillArgs a;
        memset(&a, 0, sizeof a);
        a.q = (const uint16_t*)q;
        a.k = (const uint16_t*)kws;
        a.v = (const uint16_t*)v;
        a.start_pos = start_pos;
        a.sinks = sinks;
        a.out = (uint16_t*)attn;
        a.k_sb = (int64_t)p->num_kv_heads * seq_len * p->qk_head_dim;
        a.k_sh = (int64_t)seq_len * p->qk_head_dim;
        a.k_sj = p->qk_head_dim;
        a.v_sb = (int64_t)seq_len * nv;
        a.v_sh = p->v_head_dim;
        a.v_sj = nv;
        a.kpos_rel = 1;
        a.max_start = -1;
        a.B = p->batch;
        a.S = seq_len;
        a.Hq = p->num_q_heads;
        a.Hkv = p->num_kv_heads;
        a.rope_dims = p->rope_dims;
        a.window = p->window;
        const float tau = p->softmax_scale != 0.0f ? p->softmax_scale
                                                   : (float)(1.0 / sqrt((double)p->qk_head_dim));
        a.score_scale_log2 = tau * 1.4426950408889634f;
        a.v_scale = 1.0f;
        mimo::rope_omega_rev(p->rope_theta, p->rope_dims, a.omega_rev, mimo::kMaxRopeHalfArgs);
        rc = gemm_status(mimo::launch_prefill_bf16(a, swa, sinks != nullptr, st), "prefill (bf16)");
        if (rc != MIMO_OK) return rc;
    }
    mimo::GemmArgs go = gemm_args(T, na, attn, p->v_scale);
    add_part(go, w_o, out, out_dim, mimo::kGemmPlain);
    rc = gemm_status(mimo::launch_gemm_bf16(go, st), "output projection");
    if (rc != MIMO_OK) return rc;
    mimo::clear_error();
    return MIMO_OK;
}

}  // extern "C"
