// attn_f32.hip — fp32 vector-ALU prefill and decode for small head dims (dqk, dv <= 256).
//
// Same layer definition as the bf16 MFMA kernels (pages: "Add Xiaomi MiMo-V2", "Additional
// useful info"; "add Xiaomi MiMo v2 (mimo_v2_flash)", "Architecture, verified against upstream"
// and "Implementation plan"), computed fully in fp32.  These layers are tiny (e.g. 4 heads of
// dim 32), so one thread owns one query row (prefill) and one wave owns one query head (decode).
#include "device_common.h"
#include "kernels.h"

namespace mimo {
namespace {

constexpr int MAXD = 256;

// rotate x (length dim) at pos into y
__device__ __forceinline__ void rotate_f32(const float* x, float* y, int dim, int r, int32_t pos,
                                           const double* omega) {
    const int half = r >> 1;
    for (int d = 0; d < half; ++d) {
        float c, s;
        rope_cos_sin_rev(pos, omega[d], c, s);
        y[d] = x[d] * c - x[d + half] * s;
        y[d + half] = x[d + half] * c + x[d] * s;
    }
    for (int d = r; d < dim; ++d) y[d] = x[d];
}

__global__ __launch_bounds__(64) void prefill_f32_kernel(const F32PrefillArgs a) {
    const int i = blockIdx.x * 64 + threadIdx.x, h = blockIdx.y, b = blockIdx.z;
    if (i >= a.S) return;
    const int g = h / (a.Hq / a.Hkv);
    const int32_t p0 = a.start_pos[b];
    float qr[MAXD], kr[MAXD], acc[MAXD];
    rotate_f32(a.q + (((int64_t)b * a.S + i) * a.Hq + h) * a.dqk, qr, a.dqk, a.rope_dims, p0 + i,
               a.omega_rev);
    for (int e = 0; e < a.dv; ++e) acc[e] = 0.0f;
    const bool swa = a.layer_kind == 1;
    const int lo = swa ? max(0, i - a.window + 1) : 0;
    const float sink = a.sinks ? a.sinks[h] : -INFINITY;
    float m = sink, l = a.sinks ? 1.0f : 0.0f;  // the sink: logit s_h, no value
    for (int j = lo; j <= i; ++j) {
        const int64_t row = ((int64_t)b * a.S + j) * a.Hkv + g;
        rotate_f32(a.k + row * a.dqk, kr, a.dqk, a.rope_dims, p0 + j, a.omega_rev);
        float z = 0.0f;
        for (int d = 0; d < a.dqk; ++d) z = fmaf(qr[d], kr[d], z);
        z *= a.score_scale;
        const float m_new = fmaxf(m, z);
        const float alpha = (m == -INFINITY) ? 0.0f : expf(m - m_new);
        const float p = expf(z - m_new);
        l = l * alpha + p;
        const float* vrow = a.v + row * a.dv;
        for (int e = 0; e < a.dv; ++e) acc[e] = acc[e] * alpha + p * vrow[e];
        m = m_new;
    }
    float* o = a.out + (((int64_t)b * a.S + i) * a.Hq + h) * a.dv;
    const float inv = l > 0.0f ? a.v_scale / l : 0.0f;
    for (int e = 0; e < a.dv; ++e) o[e] = acc[e] * inv;
}

// One wave per (query head, sequence); lanes split the visible slots, then merge by shuffles.
__global__ __launch_bounds__(64) void decode_f32_kernel(const F32DecodeArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int G = a.Hq / a.Hkv, g = h / G;
    const int32_t pos = a.positions[b];
    const bool swa = a.layer_kind == 1;
    float* o = a.out + ((int64_t)b * a.Hq + h) * a.dv;
    if (pos < 0 || pos > a.max_position || (!swa && pos >= a.cap)) {
        for (int e = lane; e < a.dv; e += 64) o[e] = 0.0f;
        return;
    }
    const int n_valid = swa ? min(a.window, pos + 1) : pos + 1;
    const int slot_new = swa ? pos % a.window : pos;
    const int64_t row0 = ((int64_t)b * a.Hkv + g) * a.cap;
    float qr[MAXD], kn[MAXD], acc[MAXD];
    rotate_f32(a.q + ((int64_t)b * a.Hq + h) * a.dqk, qr, a.dqk, a.rope_dims, pos, a.omega_rev);
    rotate_f32(a.k_new + ((int64_t)b * a.Hkv + g) * a.dqk, kn, a.dqk, a.rope_dims, pos, a.omega_rev);
    const float* vn = a.v_new + ((int64_t)b * a.Hkv + g) * a.dv;
    for (int e = 0; e < a.dv; ++e) acc[e] = 0.0f;
    float m = -INFINITY, l = 0.0f;
    for (int j = lane; j < n_valid; j += 64) {
        const float* kr = (j == slot_new) ? kn : a.k_cache + (row0 + j) * a.dqk;
        const float* vr = (j == slot_new) ? vn : a.v_cache + (row0 + j) * a.dv;
        float z = 0.0f;
        for (int d = 0; d < a.dqk; ++d) z = fmaf(qr[d], kr[d], z);
        z *= a.score_scale;
        const float m_new = fmaxf(m, z);
        const float alpha = (m == -INFINITY) ? 0.0f : expf(m - m_new);
        const float p = expf(z - m_new);
        l = l * alpha + p;
        for (int e = 0; e < a.dv; ++e) acc[e] = acc[e] * alpha + p * vr[e];
        m = m_new;
    }
    // merge lanes; the sink joins once
    float M = m;
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float sink = a.sinks ? a.sinks[h] : -INFINITY;
    M = fmaxf(M, sink);
    const float f = (m == -INFINITY) ? 0.0f : expf(m - M);
    float L = l * f;
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    if (a.sinks) L += expf(sink - M);
    const float inv = L > 0.0f ? a.v_scale / L : 0.0f;
    for (int e = 0; e < a.dv; ++e) {
        float x = acc[e] * f;
        for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
        if (lane == 0) o[e] = x * inv;
    }
    // append the new token (one wave per KV head does it; nobody reads this slot from memory)
    if (h % G == 0) {
        for (int d = lane; d < a.dqk; d += 64) a.k_cache[(row0 + slot_new) * a.dqk + d] = kn[d];
        for (int e = lane; e < a.dv; e += 64) a.v_cache[(row0 + slot_new) * a.dv + e] = vn[e];
    }
}

}  // namespace

hipError_t launch_prefill_f32(const F32PrefillArgs& a, hipStream_t st) {
    if (a.B == 0 || a.S == 0) return hipSuccess;
    prefill_f32_kernel<<<dim3((a.S + 63) / 64, a.Hq, a.B), 64, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode_f32(const F32DecodeArgs& a, hipStream_t st) {
    if (a.B == 0) return hipSuccess;
    decode_f32_kernel<<<dim3(a.Hq, a.B), 64, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace mimo
