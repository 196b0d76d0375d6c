// abi.hip — the C ABI of libmimo_attn.so: host-side validation, workspace sizing and dispatch.
//
// Declarations, argument meaning, layouts, ownership and error behaviour: include/mimo_attn.h.
// Layer definition: "Add Xiaomi MiMo-V2" (transformers PR 45144), "Additional useful info";
// "add Xiaomi MiMo v2 (mimo_v2_flash)" (mlxcel issue 842), "Architecture, verified against
// upstream" and "Implementation plan".
#include <math.h>
#include <stdarg.h>

#include <mutex>
#include <stdio.h>
#include <string.h>

#include "mimo_attn.h"
#include "kernels.h"
#include "verify.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return MIMO_OK;
}

}  // namespace

// The thread-local error message, shared by every entry point of the library.
namespace mimo {
int set_error(int code, const char* msg) {
    snprintf(g_err, sizeof g_err, "%s", msg);
    return code;
}
void clear_error() { g_err[0] = '\0'; }

void rope_omega_rev(double theta, int rope_dims, double* out, int n) {
    const double two_pi = 6.283185307179586476925286766559;
    for (int d = 0; d < n; ++d)
        out[d] = d < rope_dims / 2 ? pow(theta, -2.0 * (double)d / (double)rope_dims) / two_pi : 0.0;
}
}  // namespace mimo

namespace {

constexpr int kBf16Dqk = 192, kBf16Dv = 128, kF32MaxDim = 256, kMaxDecodeGroup = 16;

// Frequencies of the rotated slice, omega_d = theta^(-2d/r) for d < r/2, in revolutions per
// position (omega_d / 2pi) as the kernels take them.
void fill_omega(const mimo_attn_params* p, double* omega_rev) {
    mimo::rope_omega_rev(p->rope_theta, p->rope_dims, omega_rev, mimo::kMaxRopeHalfArgs);
}

bool fp8_cache(const mimo_attn_params* p) { return p->cache_dtype == MIMO_CACHE_FP8_E4M3; }

// Bytes per cache element.
int cache_elem_bytes(const mimo_attn_params* p) {
    return fp8_cache(p) ? 1 : (p->dtype == MIMO_BF16 ? 2 : 4);
}

float score_scale(const mimo_attn_params* p) {
    return p->softmax_scale != 0.0f ? p->softmax_scale : (float)(1.0 / sqrt((double)p->qk_head_dim));
}

int check(const mimo_attn_params* p) {
    if (!p) return fail(MIMO_ERR_INVALID_ARG, "params is NULL");
    if (p->cache_dtype != MIMO_CACHE_SAME && p->cache_dtype != MIMO_CACHE_FP8_E4M3)
        return fail(MIMO_ERR_INVALID_ARG, "cache_dtype %d is neither MIMO_CACHE_SAME (0) nor "
                    "MIMO_CACHE_FP8_E4M3 (2)", p->cache_dtype);
    if (p->cache_dtype == MIMO_CACHE_FP8_E4M3) {
        if (!(p->k_cache_scale > 0.0f && isfinite(p->k_cache_scale) && p->v_cache_scale > 0.0f &&
              isfinite(p->v_cache_scale)))
            return fail(MIMO_ERR_INVALID_ARG, "fp8 caches need finite scales > 0 (k %g, v %g)",
                        (double)p->k_cache_scale, (double)p->v_cache_scale);
        if (p->dtype != MIMO_BF16)
            return fail(MIMO_ERR_UNSUPPORTED, "fp8 caches are compiled for bf16 layers only");
    }
    if (p->batch < 0) return fail(MIMO_ERR_INVALID_ARG, "batch %d < 0", p->batch);
    if (p->num_q_heads < 1 || p->num_kv_heads < 1)
        return fail(MIMO_ERR_INVALID_ARG, "head counts must be >= 1 (Hq %d, Hkv %d)",
                    p->num_q_heads, p->num_kv_heads);
    if (p->num_q_heads % p->num_kv_heads)
        return fail(MIMO_ERR_INVALID_ARG, "num_kv_heads %d does not divide num_q_heads %d",
                    p->num_kv_heads, p->num_q_heads);
    if (p->qk_head_dim < 1 || p->v_head_dim < 1)
        return fail(MIMO_ERR_INVALID_ARG, "head dims must be >= 1 (dqk %d, dv %d)", p->qk_head_dim,
                    p->v_head_dim);
    if (p->rope_dims < 0 || p->rope_dims > p->qk_head_dim || (p->rope_dims & 1))
        return fail(MIMO_ERR_INVALID_ARG, "rope_dims %d must be even and in [0, qk_head_dim %d]",
                    p->rope_dims, p->qk_head_dim);
    if (p->rope_dims / 2 > mimo::kMaxRopeHalfArgs)
        return fail(MIMO_ERR_UNSUPPORTED, "rope_dims %d above %d", p->rope_dims,
                    2 * mimo::kMaxRopeHalfArgs);
    if (p->layer_kind != MIMO_LAYER_GLOBAL && p->layer_kind != MIMO_LAYER_SWA)
        return fail(MIMO_ERR_INVALID_ARG, "layer_kind %d is neither GLOBAL (0) nor SWA (1)",
                    p->layer_kind);
    if (p->layer_kind == MIMO_LAYER_SWA && p->window < 1)
        return fail(MIMO_ERR_INVALID_ARG, "sliding-window layer needs window >= 1 (got %d)",
                    p->window);
    if (p->layer_kind == MIMO_LAYER_GLOBAL && p->window != 0)
        return fail(MIMO_ERR_INVALID_ARG, "global layer needs window == 0 (got %d)", p->window);
    if (p->rope_dims > 0 && !(p->rope_theta > 0.0 && isfinite(p->rope_theta)))
        return fail(MIMO_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
    if (!isfinite(p->v_scale)) return fail(MIMO_ERR_INVALID_ARG, "v_scale must be finite");
    if (!(p->softmax_scale >= 0.0f) || !isfinite(p->softmax_scale))
        return fail(MIMO_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    if (p->dtype == MIMO_BF16) {
        if (p->qk_head_dim != kBf16Dqk || p->v_head_dim != kBf16Dv)
            return fail(MIMO_ERR_UNSUPPORTED, "bf16 kernels cover (dqk, dv) = (192, 128), got (%d, %d)",
                        p->qk_head_dim, p->v_head_dim);
        if (p->rope_dims % 16)
            return fail(MIMO_ERR_UNSUPPORTED, "bf16 kernels need rope_dims %% 16 == 0 (got %d)",
                        p->rope_dims);
    } else if (p->dtype == MIMO_F32) {
        if (p->qk_head_dim > kF32MaxDim || p->v_head_dim > kF32MaxDim)
            return fail(MIMO_ERR_UNSUPPORTED, "fp32 kernels cover head dims <= %d", kF32MaxDim);
    } else {
        return fail(MIMO_ERR_INVALID_ARG, "dtype %d is neither MIMO_F32 (0) nor MIMO_BF16 (1)",
                    p->dtype);
    }
    return MIMO_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MIMO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// bf16 prefill keeps the keys rotated once in [B, Hkv, S, dqk] (both layer kinds).
size_t prefill_ws(const mimo_attn_params* p, int32_t S) {
    if (p->dtype != MIMO_BF16) return 0;
    return (size_t)p->batch * p->num_kv_heads * (size_t)S * p->qk_head_dim * 2;
}

// Decode split size: slots per workgroup.
//  * a sliding ring of at most 1024 slots is one split;
//  * a small grid (at most two rounds of 256-slot splits on the chip) is cut into as many splits
//    as make one workgroup per CU (256), at least 128 slots each, rounded up to whole tiles;
//  * otherwise a power of two >= 1024 (fp8 caches, half the bytes per slot: >= 2048), large
//    enough to keep the grid (B * Hkv * splits) within 4096 workgroups and the splits per
//    sequence within what the combine kernel merges.
// A workgroup's fixed work (query rotation, new token, wave merge, partial record) is paid per
// split: in graph-replayed global decodes over 32767-slot caches, 256-slot splits at batch 4-8
// streamed 4.3-4.4 TB/s and 1024-slot ones 5.1-5.3; at batch 1-2 one round of 256 workgroups beat
// 512 (batch 1: 3.6 -> 4.2 TB/s, mixed lengths 2.3 -> 3.1); at batch 64 over lengths up to 32768
// 2048-slot splits streamed 2-6% faster than 1024-slot ones and 4096-slot ones lost on mixed
// lengths.

// Split size (key rows per workgroup) for n_max key rows per query and `pairs` (query block, KV
// head) pairs; `one_split_upto`: a key range up to this many rows is never split.
int64_t chunk_policy(int64_t n_max, int64_t pairs, int64_t one_split_upto, bool fp8) {
    if (n_max <= one_split_upto) return n_max < 1 ? 1 : n_max;
    if (pairs * ((n_max + 255) / 256) <= 2 * mimo::kResidentDecodeGroups) {
        int64_t ns = mimo::kResidentDecodeGroups / 2 / pairs;   // one per CU
        if (ns < 1) ns = 1;
        if (ns > (n_max + 127) / 128) ns = (n_max + 127) / 128;
        return ((n_max + ns - 1) / ns + 31) / 32 * 32;
    }
    // (more than 4096 pairs: one split each, the whole range)
    int64_t chunk = fp8 ? 2048 : 1024;
    while (chunk < n_max && (pairs * ((n_max + chunk - 1) / chunk) > 4096 ||
                             (n_max + chunk - 1) / chunk > mimo::decode_max_splits()))
        chunk *= 2;
    return chunk;
}

struct SplitGeometry {
    int64_t n_max;   // key rows of the longest query
    int chunk, nsplit;
};

SplitGeometry split_geometry(int64_t n_max, int64_t pairs, int64_t one_split_upto, bool fp8) {
    SplitGeometry g;
    g.n_max = n_max;
    g.chunk = (int)chunk_policy(n_max, pairs, one_split_upto, fp8);
    g.nsplit = (int)((n_max + g.chunk - 1) / g.chunk);
    return g;
}

// Decode: keys 0..max_position (linear) or the window's slots (ring, never split up to 1024).
SplitGeometry decode_geometry(const mimo_attn_params* p, int32_t max_position) {
    const bool swa = p->layer_kind == MIMO_LAYER_SWA;
    const int64_t n_max = swa ? (int64_t)(p->window < max_position + 1 ? p->window : max_position + 1)
                              : (int64_t)max_position + 1;
    return split_geometry(n_max, (int64_t)p->batch * p->num_kv_heads, swa ? 1024 : 0,
                          fp8_cache(p));
}

size_t partials_bytes(const mimo_attn_params* p, int64_t queries, int nsplit) {
    if (nsplit <= 1) return 0;
    return (size_t)queries * p->num_q_heads * (size_t)nsplit * (p->v_head_dim + 2) * sizeof(float);
}

size_t decode_ws(const mimo_attn_params* p, int32_t max_position) {
    if (p->dtype != MIMO_BF16) return 0;
    return partials_bytes(p, p->batch, decode_geometry(p, max_position).nsplit);
}

// Extend of at most this many new tokens per sequence runs the multi-token tile kernel: the
// (query head, token) pairs of a KV group are the query columns of one workgroup, so each key
// tile is read once for all of them.
constexpr int kVerifyMaxTokens = 16;

int pow2_at_least(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

bool verify_tokens(const mimo_attn_params* p, int32_t S) {
    return S >= 1 && S <= kVerifyMaxTokens &&
           mimo::verify_tile_waves(p->num_q_heads / p->num_kv_heads, pow2_at_least(S)) > 0 &&
           (int64_t)p->batch * S <= 65535 && p->batch <= 65535;   // (combine grid, kernel grid)
}

// Multi-token extend: key rows of the longest query — global: positions 0..max_start + S - 1
// of the cache; sliding: the W + S rows of the workspace (never split up to 1024 rows).
// Splits of whole 64-row tiles: enough (sequence, KV head, split) workgroups to fill the chip
// once (two resident per CU), at least 256 rows each, and at most kVerifyMaxSplitRows rows each:
// the tile kernel's grid is split-major, so with mixed lengths the workgroups that start last
// are the longest sequences' last splits, and no workgroup runs much longer than the others (B64,
// 4 tokens after 1024-32768 positions, fp8 cache: 0.54 ms with two splits of 16384 rows, 0.455
// with splits of 4096; 2048- and 8192-row splits lost at this batch).
constexpr int64_t kVerifyMaxSplitRows = 4096;

SplitGeometry verify_geometry(const mimo_attn_params* p, int32_t S, int32_t max_start) {
    const bool swa = p->layer_kind == MIMO_LAYER_SWA;
    const int64_t n_max = swa ? (int64_t)p->window + S : (int64_t)max_start + S;
    const int64_t pairs = (int64_t)p->batch * p->num_kv_heads;
    int64_t ns = (512 + pairs - 1) / pairs;
    if (ns < (n_max + kVerifyMaxSplitRows - 1) / kVerifyMaxSplitRows)
        ns = (n_max + kVerifyMaxSplitRows - 1) / kVerifyMaxSplitRows;
    if (ns > (n_max + 255) / 256) ns = (n_max + 255) / 256;
    if (ns > mimo::decode_max_splits()) ns = mimo::decode_max_splits();
    if (ns < 1) ns = 1;
    int64_t chunk = ((n_max + ns - 1) / ns + 63) / 64 * 64;
    SplitGeometry g;
    g.n_max = n_max;
    g.chunk = (int)chunk;
    g.nsplit = (int)((n_max + chunk - 1) / chunk);
    return g;
}

// Rows per (sequence, KV head) of the bf16 key/value rows an extend lays out in its workspace:
// sliding layers window + S (the ring's content in position order, then the new tokens); global
// layers with an fp8 cache: a few new tokens S (the multi-token kernel reads the cached codes in
// place), more max_start + S (row = position: the cached rows widened to bf16, then the new
// tokens); global layers with a bf16 cache none (they attend straight from the cache).
int64_t extend_rows(const mimo_attn_params* p, int32_t S, int32_t max_start) {
    if (p->dtype != MIMO_BF16) return 0;
    if (p->layer_kind == MIMO_LAYER_SWA) return (int64_t)p->window + S;
    if (!fp8_cache(p)) return 0;
    return verify_tokens(p, S) ? (int64_t)S : (int64_t)max_start + S;
}

// bf16 extend workspace: those rows (K then V, 256-byte aligned), then the split partials of a
// multi-token extend.
size_t extend_rows_ws(const mimo_attn_params* p, int32_t S, int32_t max_start) {
    const size_t b = (size_t)p->batch * p->num_kv_heads * (size_t)extend_rows(p, S, max_start) *
                     (p->qk_head_dim + p->v_head_dim) * 2;
    return (b + 255) / 256 * 256;
}

size_t extend_ws(const mimo_attn_params* p, int32_t S, int32_t max_start) {
    if (p->dtype != MIMO_BF16) return 0;
    size_t n = extend_rows_ws(p, S, max_start);
    if (verify_tokens(p, S))
        n += partials_bytes(p, (int64_t)p->batch * S, verify_geometry(p, S, max_start).nsplit);
    return n;
}

}  // namespace

extern "C" {

int mimo_attn_abi_version(void) { return MIMO_ATTN_ABI_VERSION; }

const char* mimo_attn_last_error(void) { return g_err; }

int mimo_attn_check_params(const mimo_attn_params* p) {
    const int rc = check(p);
    return rc == MIMO_OK ? ok() : rc;
}

size_t mimo_attn_prefill_workspace_size(const mimo_attn_params* p, int32_t seq_len) {
    if (check(p) != MIMO_OK || seq_len < 0) return 0;
    return prefill_ws(p, seq_len);
}

size_t mimo_attn_extend_workspace_size(const mimo_attn_params* p, int32_t seq_len,
                                       int32_t max_start) {
    if (check(p) != MIMO_OK || seq_len < 0 || max_start < 0) return 0;
    return extend_ws(p, seq_len, max_start);
}

size_t mimo_attn_decode_workspace_size(const mimo_attn_params* p, int32_t max_position) {
    if (check(p) != MIMO_OK || max_position < 0) return 0;
    return decode_ws(p, max_position);
}

int mimo_attn_prefill(const mimo_attn_params* p, int32_t seq_len, const void* q, const void* k,
                      const void* v, const int32_t* start_pos, const float* sinks, void* out,
                      void* k_cache, void* v_cache, int32_t cache_capacity, void* workspace,
                      size_t workspace_bytes, void* stream) {
    int rc = check(p);
    if (rc != MIMO_OK) return rc;
    if (seq_len < 0) return fail(MIMO_ERR_INVALID_ARG, "seq_len %d < 0", seq_len);
    if (p->batch == 0 || seq_len == 0) return ok();
    if (!q || !k || !v || !start_pos || !out)
        return fail(MIMO_ERR_INVALID_ARG, "q, k, v, start_pos and out must be non-NULL");
    if ((k_cache == nullptr) != (v_cache == nullptr))
        return fail(MIMO_ERR_INVALID_ARG, "k_cache and v_cache must both be set or both be NULL");
    const bool has_cache = k_cache != nullptr;
    const bool swa = p->layer_kind == MIMO_LAYER_SWA;
    if (has_cache) {
        if (cache_capacity < 1) return fail(MIMO_ERR_INVALID_ARG, "cache_capacity must be >= 1");
        if (swa && cache_capacity != p->window)
            return fail(MIMO_ERR_INVALID_ARG, "ring cache capacity %d must equal window %d",
                        cache_capacity, p->window);
    }
    if ((int64_t)seq_len * p->num_q_heads * p->batch > ((int64_t)1 << 40))
        return fail(MIMO_ERR_INVALID_ARG, "problem too large");
    const size_t need = prefill_ws(p, seq_len);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MIMO_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    hipStream_t st = (hipStream_t)stream;

    mimo::RopeKVArgs ra;
    memset(&ra, 0, sizeof ra);
    ra.k = k;
    ra.v = v;
    ra.start_pos = start_pos;
    ra.B = p->batch;
    ra.S = seq_len;
    ra.Hkv = p->num_kv_heads;
    ra.dqk = p->qk_head_dim;
    ra.dv = p->v_head_dim;
    ra.rope_dims = p->rope_dims;
    ra.cap = cache_capacity;
    ra.ring_window = swa ? p->window : 0;
    ra.ws_rows = seq_len;
    ra.max_start = -1;
    ra.cache_fp8 = fp8_cache(p);
    ra.k_inv = fp8_cache(p) ? 1.0f / p->k_cache_scale : 1.0f;
    ra.v_inv = fp8_cache(p) ? 1.0f / p->v_cache_scale : 1.0f;
    // the ring only keeps the last `window` tokens
    ra.cache_i0 = (swa && seq_len > p->window) ? seq_len - p->window : 0;
    if (has_cache) {
        ra.k_dst = k_cache;
        ra.v_dst = v_cache;
    }
    fill_omega(p, ra.omega_rev);

    if (p->dtype == MIMO_F32) {
        mimo::F32PrefillArgs fa;
        memset(&fa, 0, sizeof fa);
        fa.q = (const float*)q;
        fa.k = (const float*)k;
        fa.v = (const float*)v;
        fa.start_pos = start_pos;
        fa.sinks = sinks;
        fa.out = (float*)out;
        fa.B = p->batch;
        fa.S = seq_len;
        fa.Hq = p->num_q_heads;
        fa.Hkv = p->num_kv_heads;
        fa.dqk = p->qk_head_dim;
        fa.dv = p->v_head_dim;
        fa.rope_dims = p->rope_dims;
        fa.window = p->window;
        fa.layer_kind = p->layer_kind;
        fa.score_scale = score_scale(p);
        fa.v_scale = p->v_scale;
        fill_omega(p, fa.omega_rev);
        rc = hip_status(mimo::launch_prefill_f32(fa, st), "prefill (fp32)");
        if (rc != MIMO_OK || !has_cache) return rc;
        ra.i0 = ra.cache_i0;
        return hip_status(mimo::launch_rope_kv_f32(ra, st), "cache store (fp32)");
    }

    mimo::PrefillArgs pa;
    memset(&pa, 0, sizeof pa);
    pa.q = (const uint16_t*)q;
    pa.v = (const uint16_t*)v;
    pa.start_pos = start_pos;
    pa.sinks = sinks;
    pa.out = (uint16_t*)out;
    pa.B = p->batch;
    pa.S = seq_len;
    pa.Hq = p->num_q_heads;
    pa.Hkv = p->num_kv_heads;
    pa.rope_dims = p->rope_dims;
    pa.window = p->window;
    pa.score_scale_log2 = score_scale(p) * 1.4426950408889634f;
    pa.v_scale = p->v_scale;
    pa.v_sb = (int64_t)seq_len * p->num_kv_heads * p->v_head_dim;   // v [B,S,Hkv,dv]
    pa.v_sh = p->v_head_dim;
    pa.v_sj = (int64_t)p->num_kv_heads * p->v_head_dim;
    pa.kpos_rel = 1;   // key row j is token j
    pa.max_start = -1;
    fill_omega(p, pa.omega_rev);
    // rotate K once into the workspace (and store the cache), then attend
    ra.k_ws = workspace;
    rc = hip_status(mimo::launch_rope_kv_bf16(ra, st), "key rotation (bf16)");
    if (rc != MIMO_OK) return rc;
    const int64_t dqk = p->qk_head_dim;
    pa.k = (const uint16_t*)workspace;
    pa.k_sb = (int64_t)p->num_kv_heads * seq_len * dqk;
    pa.k_sh = (int64_t)seq_len * dqk;
    pa.k_sj = dqk;
    return hip_status(mimo::launch_prefill_bf16(pa, swa, sinks != nullptr, st), "prefill (bf16)");
}

int mimo_attn_extend(const mimo_attn_params* p, int32_t seq_len, const void* q, const void* k,
                     const void* v, const int32_t* start_pos, int32_t max_start,
                     const float* sinks, void* out, void* k_cache, void* v_cache,
                     int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                     void* stream) {
    int rc = check(p);
    if (rc != MIMO_OK) return rc;
    if (seq_len < 0) return fail(MIMO_ERR_INVALID_ARG, "seq_len %d < 0", seq_len);
    if (max_start < 0) return fail(MIMO_ERR_INVALID_ARG, "max_start %d < 0", max_start);
    if ((int64_t)max_start + seq_len > 0x7fffffffLL)
        return fail(MIMO_ERR_INVALID_ARG, "max_start %d + seq_len %d overflows int32 positions",
                    max_start, seq_len);
    if (p->dtype != MIMO_BF16)
        return fail(MIMO_ERR_UNSUPPORTED, "extend is compiled for bf16 layers only");
    const bool swa = p->layer_kind == MIMO_LAYER_SWA;
    const bool fp8 = fp8_cache(p);
    if (swa && cache_capacity != p->window)
        return fail(MIMO_ERR_INVALID_ARG, "ring cache capacity %d must equal window %d",
                    cache_capacity, p->window);
    if (!swa && (int64_t)max_start + seq_len > (int64_t)cache_capacity)
        return fail(MIMO_ERR_INVALID_ARG,
                    "linear cache capacity %d must hold max_start %d + seq_len %d positions",
                    cache_capacity, max_start, seq_len);
    if (p->batch == 0 || seq_len == 0) return ok();
    if (!q || !k || !v || !start_pos || !out || !k_cache || !v_cache)
        return fail(MIMO_ERR_INVALID_ARG,
                    "q, k, v, start_pos, out, k_cache and v_cache must be non-NULL");
    if ((int64_t)seq_len * p->num_q_heads * p->batch > ((int64_t)1 << 40))
        return fail(MIMO_ERR_INVALID_ARG, "problem too large");
    const size_t need = extend_ws(p, seq_len, max_start);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MIMO_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    hipStream_t st = (hipStream_t)stream;
    const int64_t Hkv = p->num_kv_heads, dqk = p->qk_head_dim, dv = p->v_head_dim;

    mimo::RopeKVArgs ra;
    memset(&ra, 0, sizeof ra);
    ra.k = k;
    ra.v = v;
    ra.start_pos = start_pos;
    ra.k_dst = k_cache;
    ra.v_dst = v_cache;
    ra.B = p->batch;
    ra.S = seq_len;
    ra.Hkv = p->num_kv_heads;
    ra.dqk = p->qk_head_dim;
    ra.dv = p->v_head_dim;
    ra.rope_dims = p->rope_dims;
    ra.cap = cache_capacity;
    ra.ring_window = swa ? p->window : 0;
    ra.max_start = max_start;
    if (fp8) {   // the new tokens are stored as codes
        ra.cache_fp8 = 1;
        ra.k_inv = 1.0f / p->k_cache_scale;
        ra.v_inv = 1.0f / p->v_cache_scale;
    }
    fill_omega(p, ra.omega_rev);

    mimo::PrefillArgs pa;
    memset(&pa, 0, sizeof pa);
    pa.q = (const uint16_t*)q;
    pa.start_pos = start_pos;
    pa.sinks = sinks;
    pa.out = (uint16_t*)out;
    pa.max_start = max_start;
    pa.B = p->batch;
    pa.S = seq_len;
    pa.Hq = p->num_q_heads;
    pa.Hkv = p->num_kv_heads;
    pa.rope_dims = p->rope_dims;
    pa.window = p->window;
    pa.score_scale_log2 = score_scale(p) * 1.4426950408889634f;
    pa.v_scale = p->v_scale;
    fill_omega(p, pa.omega_rev);

    // a few new tokens run the multi-token tile kernel, more the prefill kernel
    const bool few = verify_tokens(p, seq_len);
    const int64_t rows = extend_rows(p, seq_len, max_start);
    uint16_t* kws = (uint16_t*)workspace;
    uint16_t* vws = kws + (int64_t)p->batch * Hkv * rows * dqk;
    mimo::CacheRowsArgs ua;   // cached rows -> workspace rows by position (widened if fp8)
    memset(&ua, 0, sizeof ua);
    ua.k_cache = k_cache;
    ua.v_cache = v_cache;
    ua.start_pos = start_pos;
    ua.k_ws = kws;
    ua.v_ws = vws;
    ua.B = p->batch;
    ua.Hkv = p->num_kv_heads;
    ua.dqk = p->qk_head_dim;
    ua.dv = p->v_head_dim;
    ua.cap = cache_capacity;
    ua.ws_rows = (int32_t)rows;
    ua.max_start = max_start;
    if (fp8) {
        ua.cache_fp8 = 1;
        ua.k_scale = p->k_cache_scale;
        ua.v_scale = p->v_cache_scale;
    }
    if (swa) {
        // workspace rows r < W: the ring's positions start - W + r (in position order; from a bf16
        // ring the tile kernel reads those in place); rows W + i: the new tokens, rotated.  The
        // ring itself is refreshed only after it is read.
        if (!few || fp8) {
            ua.W = p->window;
            ua.rows = p->window;
            rc = hip_status(mimo::launch_cache_rows_bf16(ua, st), "ring unroll (bf16)");
            if (rc != MIMO_OK) return rc;
        }
        ra.k_ws = kws;
        ra.v_ws = vws;
        ra.ws_rows = (int32_t)rows;
        ra.ws_row0 = p->window;
        ra.cache_i0 = seq_len > p->window ? seq_len - p->window : 0;
        pa.k = kws;
        pa.v = vws;
        pa.k_sb = Hkv * rows * dqk;
        pa.k_sh = rows * dqk;
        pa.v_sb = Hkv * rows * dv;
        pa.v_sh = rows * dv;
        pa.kpos_rel = 1;
        pa.kpos_off = -p->window;   // key row j sits at position start - W + j
    } else if (fp8 && few) {
        // workspace row t = new token t, rotated (the tokens also go to the cache, as codes); the
        // multi-token kernel reads the cached positions' codes in place
        ra.k_ws = kws;
        ra.v_ws = vws;
        ra.ws_rows = (int32_t)rows;
        ra.ws_row0 = 0;
        pa.k = kws;
        pa.v = vws;
        pa.k_sb = Hkv * rows * dqk;
        pa.k_sh = rows * dqk;
        pa.v_sb = Hkv * rows * dv;
        pa.v_sh = rows * dv;
        pa.kpos_rel = 0;
        pa.kpos_off = 0;
    } else if (fp8) {
        // workspace row j = position j: the cached rows before each start widened to bf16, then
        // the new tokens, rotated (which also go to the cache, as codes)
        ua.W = 0;
        ua.rows = max_start;
        rc = hip_status(mimo::launch_cache_rows_bf16(ua, st), "cache widening (fp8)");
        if (rc != MIMO_OK) return rc;
        ra.k_ws = kws;
        ra.v_ws = vws;
        ra.ws_rows = (int32_t)rows;
        ra.ws_row0 = 0;
        ra.ws_rel = 1;
        pa.k = kws;
        pa.v = vws;
        pa.k_sb = Hkv * rows * dqk;
        pa.k_sh = rows * dqk;
        pa.v_sb = Hkv * rows * dv;
        pa.v_sh = rows * dv;
        pa.kpos_rel = 0;
        pa.kpos_off = 0;
    } else {
        // new tokens go to the linear cache first; key row j of the cache is position j
        pa.k = (const uint16_t*)k_cache;
        pa.v = (const uint16_t*)v_cache;
        pa.k_sb = Hkv * cache_capacity * dqk;
        pa.k_sh = (int64_t)cache_capacity * dqk;
        pa.v_sb = Hkv * cache_capacity * dv;
        pa.v_sh = (int64_t)cache_capacity * dv;
        pa.kpos_rel = 0;
        pa.kpos_off = 0;
    }
    pa.k_sj = dqk;
    pa.v_sj = dv;
    // (multi-token sliding extend: the ring is stored after the attention, which reads it)
    mimo::RopeKVArgs ra_first = ra;
    if (few && swa) ra_first.k_dst = ra_first.v_dst = nullptr;
    rc = hip_status(mimo::launch_rope_kv_bf16(ra_first, st), "key rotation (bf16)");
    if (rc != MIMO_OK) return rc;
    if (!few)
        return hip_status(mimo::launch_prefill_bf16(pa, swa, sinks != nullptr, st), "extend (bf16)");

    // a few new tokens: the multi-token tile kernel over the same key rows
    const SplitGeometry geo = verify_geometry(p, seq_len, max_start);
    mimo::VerifyArgs va;
    memset(&va, 0, sizeof va);
    va.q = (const uint16_t*)q;
    va.k = pa.k;
    va.v = pa.v;
    va.start_pos = start_pos;
    va.sinks = sinks;
    va.out = (uint16_t*)out;
    va.partial = (float*)((uint8_t*)workspace + extend_rows_ws(p, seq_len, max_start));
    if (swa && !fp8) {
        va.ring_k = (const uint16_t*)k_cache;
        va.ring_v = (const uint16_t*)v_cache;
        va.ring_w = p->window;
    }
    if (!swa && fp8) {
        // cached positions read as codes, in place: the scales ride on the score and output scales
        va.code_k = (const uint8_t*)k_cache;
        va.code_v = (const uint8_t*)v_cache;
        va.code_cap = cache_capacity;
        va.code_k_scale = p->k_cache_scale;
        va.code_v_scale = p->v_cache_scale;
    }
    va.k_sb = pa.k_sb;
    va.k_sh = pa.k_sh;
    va.v_sb = pa.v_sb;
    va.v_sh = pa.v_sh;
    va.B = p->batch;
    va.T = seq_len;
    va.TP = pow2_at_least(seq_len);
    va.Hq = p->num_q_heads;
    va.Hkv = p->num_kv_heads;
    va.rope_dims = p->rope_dims;
    va.window = p->window;
    va.kpos_rel = pa.kpos_rel;
    va.kpos_off = pa.kpos_off;
    va.max_start = max_start;
    va.chunk = geo.chunk;
    va.nsplit = geo.nsplit;
    va.score_scale_log2 = pa.score_scale_log2;
    va.v_scale = p->v_scale;
    if (va.code_k) {   // (the cache scales of codes read in place)
        va.score_scale_log2 *= p->k_cache_scale;
        va.v_scale *= p->v_cache_scale;
    }
    fill_omega(p, va.omega_rev);
    rc = hip_status(mimo::launch_verify_tiles_bf16(va, swa, sinks != nullptr, st), "extend (bf16)");
    if (rc != MIMO_OK) return rc;
    if (swa) {   // now store the new tokens in the ring
        mimo::RopeKVArgs rs = ra;
        rs.k_ws = rs.v_ws = nullptr;
        rc = hip_status(mimo::launch_rope_kv_bf16(rs, st), "ring store (bf16)");
        if (rc != MIMO_OK) return rc;
    }
    if (geo.nsplit <= 1) return rc;
    mimo::DecodeArgs da;   // the combine's view of the partials
    memset(&da, 0, sizeof da);
    da.positions = start_pos;
    da.sinks = sinks;
    da.out = (uint16_t*)out;
    da.partial = va.partial;
    da.B = p->batch;
    da.Hq = p->num_q_heads;
    da.Hkv = p->num_kv_heads;
    da.window = p->window;
    da.max_position = max_start;
    da.chunk = geo.chunk;
    da.nsplit = geo.nsplit;
    da.q_per_seq = seq_len;
    da.kpos_rel = pa.kpos_rel;
    da.kpos_off = pa.kpos_off;
    da.v_scale = va.v_scale;
    return hip_status(mimo::launch_verify_combine(da, swa, sinks != nullptr, st), "extend combine");
}

}  // extern "C"

namespace {

// Scratch of the allocation-free decode (mimo_attn_decode_noalloc): the split partials live in
// this file-scope device array instead of a caller workspace.  Each device that runs the library
// holds its own copy until the process ends.  Host code never passes the array's name to a kernel
// (on the host it only stands in for the symbol): its device address, looked up once per device
// with that device current, is what the kernels get.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MIMO_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MIMO_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(MIMO_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MIMO_OK;
}

int decode_impl(const mimo_attn_params* p, const void* q, const void* k_new, const void* v_new,
                const int32_t* positions, int32_t max_position, void* k_cache, void* v_cache,
                int32_t cache_capacity, const float* sinks, void* out, void* workspace,
                size_t workspace_bytes, void* stream, bool noalloc) {
    int rc = check(p);
    if (rc != MIMO_OK) return rc;
    if (max_position < 0) return fail(MIMO_ERR_INVALID_ARG, "max_position %d < 0", max_position);
    if (p->batch == 0) return ok();
    if (!q || !k_new || !v_new || !positions || !k_cache || !v_cache || !out)
        return fail(MIMO_ERR_INVALID_ARG,
                    "q, k_new, v_new, positions, k_cache, v_cache and out must be non-NULL");
    const bool swa = p->layer_kind == MIMO_LAYER_SWA;
    if (swa && cache_capacity != p->window)
        return fail(MIMO_ERR_INVALID_ARG, "ring cache capacity %d must equal window %d",
                    cache_capacity, p->window);
    if (!swa && (int64_t)cache_capacity <= (int64_t)max_position)
        return fail(MIMO_ERR_INVALID_ARG, "linear cache capacity %d must exceed max_position %d",
                    cache_capacity, max_position);
    // bf16 decode addresses a cache slice through a buffer resource with a 32-bit byte bound
    if (p->dtype == MIMO_BF16 &&
        (int64_t)cache_capacity * p->qk_head_dim * cache_elem_bytes(p) > 0xffffffffLL)
        return fail(MIMO_ERR_UNSUPPORTED, "cache_capacity %d: a cache slice must stay below 4 GiB",
                    cache_capacity);
    hipStream_t st = (hipStream_t)stream;
    if (p->dtype == MIMO_F32) {
        mimo::F32DecodeArgs fa;
        memset(&fa, 0, sizeof fa);
        fa.q = (const float*)q;
        fa.k_new = (const float*)k_new;
        fa.v_new = (const float*)v_new;
        fa.positions = positions;
        fa.k_cache = (float*)k_cache;
        fa.v_cache = (float*)v_cache;
        fa.sinks = sinks;
        fa.out = (float*)out;
        fa.B = p->batch;
        fa.Hq = p->num_q_heads;
        fa.Hkv = p->num_kv_heads;
        fa.dqk = p->qk_head_dim;
        fa.dv = p->v_head_dim;
        fa.rope_dims = p->rope_dims;
        fa.window = p->window;
        fa.layer_kind = p->layer_kind;
        fa.cap = cache_capacity;
        fa.max_position = max_position;
        fa.score_scale = score_scale(p);
        fa.v_scale = p->v_scale;
        fill_omega(p, fa.omega_rev);
        return hip_status(mimo::launch_decode_f32(fa, st), "decode (fp32)");
    }
    if (p->num_q_heads / p->num_kv_heads > kMaxDecodeGroup)
        return fail(MIMO_ERR_UNSUPPORTED, "bf16 decode packs at most %d query heads per KV head",
                    kMaxDecodeGroup);
    const size_t need = decode_ws(p, max_position);
    if (noalloc) {
        if (need > kNoAllocScratchBytes)
            return fail(MIMO_ERR_WORKSPACE,
                        "allocation-free decode: the split partials need %zu bytes, above its "
                        "%zu-byte scratch (use mimo_attn_decode with a workspace)",
                        need, kNoAllocScratchBytes);
        workspace = nullptr;
        workspace_bytes = 0;
        if (need > 0) {
            rc = scratch_address(&workspace);
            if (rc != MIMO_OK) return rc;
            workspace_bytes = kNoAllocScratchBytes;
        }
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(MIMO_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    mimo::DecodeArgs da;
    memset(&da, 0, sizeof da);
    da.q = (const uint16_t*)q;
    da.k_new = (const uint16_t*)k_new;
    da.v_new = (const uint16_t*)v_new;
    da.positions = positions;
    da.k_cache = k_cache;
    da.v_cache = v_cache;
    da.sinks = sinks;
    da.out = (uint16_t*)out;
    da.partial = (float*)workspace;
    da.B = p->batch;
    da.Hq = p->num_q_heads;
    da.Hkv = p->num_kv_heads;
    da.rope_dims = p->rope_dims;
    da.window = p->window;
    da.cap = cache_capacity;
    da.max_position = max_position;
    const SplitGeometry geo = decode_geometry(p, max_position);
    da.chunk = geo.chunk;
    da.nsplit = geo.nsplit;
    da.score_scale_log2 = score_scale(p) * 1.4426950408889634f;
    da.v_scale = p->v_scale;
    if (fp8_cache(p)) {
        // codes are attended as their e4m3 values; the scales multiply scores and output
        da.cache_fp8 = 1;
        da.k_inv = 1.0f / p->k_cache_scale;
        da.v_inv = 1.0f / p->v_cache_scale;
        da.score_scale_log2 *= p->k_cache_scale;
        da.v_scale *= p->v_cache_scale;
    }
    fill_omega(p, da.omega_rev);
    return hip_status(mimo::launch_decode_bf16(da, swa, sinks != nullptr, st), "decode (bf16)");
}

}  // namespace

extern "C" {

int mimo_attn_decode(const mimo_attn_params* p, const void* q, const void* k_new,
                     const void* v_new, const int32_t* positions, int32_t max_position,
                     void* k_cache, void* v_cache, int32_t cache_capacity, const float* sinks,
                     void* out, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(p, q, k_new, v_new, positions, max_position, k_cache, v_cache,
                       cache_capacity, sinks, out, workspace, workspace_bytes, stream, false);
}

int mimo_attn_decode_noalloc(const mimo_attn_params* p, const void* q, const void* k_new,
                             const void* v_new, const int32_t* positions, int32_t max_position,
                             void* k_cache, void* v_cache, int32_t cache_capacity,
                             const float* sinks, void* out, void* stream) {
    return decode_impl(p, q, k_new, v_new, positions, max_position, k_cache, v_cache,
                       cache_capacity, sinks, out, nullptr, 0, stream, true);
}

size_t mimo_attn_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

}  // extern "C"
