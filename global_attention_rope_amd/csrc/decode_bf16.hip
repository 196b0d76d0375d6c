// decode_bf16.hip — single-token decode of the hybrid attention layer against its KV cache.
//
// Pages: "Add Xiaomi MiMo-V2", section "Additional useful info" (per-kind theta and KV groups,
// decoupled V dim, value rescale, SWA-only sink); "add Xiaomi MiMo v2 (mimo_v2_flash)", section
// "Implementation plan" (sliding layers keep a rotating cache of the window).
//
// Per (sequence b, KV head g, split s) one workgroup:
//   * rotates the query heads of group g (<= 16) at the new token's position and keeps Q^T as the
//     B operand of v_mfma_f32_16x16x32_bf16 (heads are the 16-wide N dimension);
//   * the split that owns the new token's slot rotates k_new, stores it and v_new into the cache
//     (linear: slot = position; ring: slot = position % window) and substitutes them for that
//     slot in its own tile loads, so no workgroup reads a slot another one is writing;
//   * each wave streams 32-slot tiles: S^T = K * Q^T (rotated keys come from the cache), online
//     softmax per head in the log2 domain, O^T += V^T * P^T;
//   * the four waves are merged through LDS; with one split the sink is folded in and the bf16
//     output is written, otherwise (max, sum, O) partials go to the workspace and a combine kernel
//     merges the splits and adds the sink exactly once.
#include "device_common.h"
#include "kernels.h"

namespace mimo {
namespace {

constexpr int DQK = 192;
constexpr int DV = 128;
constexpr int NW = 4;
constexpr int TILE = 32;                 // slots per wave iteration
constexpr int PSTRIDE = DV + 2;          // floats per partial record: O[128], m, l

__device__ __forceinline__ u32x4 rotate8_dec(const u32x4& w, const u32x4& pw, int d0, int half,
                                             int32_t pos, const double* omega) {
    float x[8], y[8];
    unpack8(w, x);
    unpack8(pw, y);
    const bool lower = d0 < half;
    const int f0 = lower ? d0 : d0 - half;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        float c, s;
        rope_cos_sin(pos, omega[f0 + t], c, s);
        x[t] = lower ? (x[t] * c - y[t] * s) : (x[t] * c + y[t] * s);
    }
    return pack8(x);
}

template <bool SWA, bool SINK, bool SPLIT>
__global__ __launch_bounds__(256) void decode_bf16_kernel(const DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t Qs[16 * DQK];
    __shared__ __attribute__((aligned(16))) uint16_t Kn[DQK];
    __shared__ __attribute__((aligned(16))) uint16_t Vn[DV];
    __shared__ float red_m[NW][16], red_l[NW][16];
    __shared__ float red_o[NW][16][DV + 1];

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, gq = lane >> 4;
    const int G = a.Hq / a.Hkv;
    const int32_t pos = a.positions[b];
    const bool pos_ok = pos >= 0 && pos <= a.max_position && (SWA || pos < a.cap);
    if (!pos_ok) {
        if (!SPLIT && s == 0) {  // defined result: zero output, nothing appended
            for (int e = tid; e < G * DV; e += 256)
                a.out[((int64_t)b * a.Hq + g * G + e / DV) * DV + e % DV] = 0;
        }
        return;
    }
    const int n_valid = SWA ? min(a.window, pos + 1) : pos + 1;
    const int slot_new = SWA ? pos % a.window : pos;
    const int k_begin = s * a.chunk;
    if (k_begin >= n_valid) return;
    const int k_end = min(n_valid, k_begin + a.chunk);
    const bool own_new = slot_new >= k_begin && slot_new < k_end;
    const int r = a.rope_dims, half = r >> 1;
    const int64_t cache_row0 = ((int64_t)b * a.Hkv + g) * a.cap;

    // ---- rotated queries of this group -> LDS (heads >= G are zero).
    for (int c = tid; c < 16 * (DQK / 8); c += 256) {
        const int hh = c / (DQK / 8), col = c % (DQK / 8);
        u32x4 wv = u32x4{0u, 0u, 0u, 0u};
        if (hh < G) {
            const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + g * G + hh) * DQK;
            wv = *(const u32x4*)(qrow + col * 8);
            if (col * 8 < r) {
                const int d0 = col * 8;
                const int pd = d0 < half ? d0 + half : d0 - half;
                wv = rotate8_dec(wv, *(const u32x4*)(qrow + pd), d0, half, pos, a.omega);
            }
        }
        *(u32x4*)(Qs + hh * DQK + col * 8) = wv;
    }
    // ---- the new token: rotate, keep in LDS, append to the cache.
    if (own_new && tid < DQK / 8 + DV / 8) {
        if (tid < DQK / 8) {
            const uint16_t* krow = a.k_new + ((int64_t)b * a.Hkv + g) * DQK;
            const int d0 = tid * 8;
            u32x4 wv = *(const u32x4*)(krow + d0);
            if (d0 < r) {
                const int pd = d0 < half ? d0 + half : d0 - half;
                wv = rotate8_dec(wv, *(const u32x4*)(krow + pd), d0, half, pos, a.omega);
            }
            *(u32x4*)(Kn + d0) = wv;
            *(u32x4*)(a.k_cache + (cache_row0 + slot_new) * DQK + d0) = wv;
        } else {
            const int d0 = (tid - DQK / 8) * 8;
            const u32x4 wv = *(const u32x4*)(a.v_new + ((int64_t)b * a.Hkv + g) * DV + d0);
            *(u32x4*)(Vn + d0) = wv;
            *(u32x4*)(a.v_cache + (cache_row0 + slot_new) * DV + d0) = wv;
        }
    }
    __syncthreads();

    bf16x8 Qb[DQK / 32];
#pragma unroll
    for (int c = 0; c < DQK / 32; ++c) Qb[c] = *(const bf16x8*)(Qs + l16 * DQK + 32 * c + 8 * gq);

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 O[DV / 16];
#pragma unroll
    for (int db = 0; db < DV / 16; ++db) O[db] = f32x4{};

    const uint16_t* kc = a.k_cache + cache_row0 * DQK;
    const uint16_t* vc = a.v_cache + cache_row0 * DV;

    for (int t0 = k_begin + wave * TILE; t0 < k_end; t0 += NW * TILE) {
        // S^T (16 slots x 16 heads) for the two 16-slot blocks of the tile.
        f32x4 Sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int j = t0 + kb * 16 + l16;
            u32x4 kw[DQK / 32];
#pragma unroll
            for (int c = 0; c < DQK / 32; ++c) {
                u32x4 wv = u32x4{0u, 0u, 0u, 0u};
                if (j < k_end) {
                    wv = (j == slot_new) ? *(const u32x4*)(Kn + 32 * c + 8 * gq)
                                         : *(const u32x4*)(kc + (int64_t)j * DQK + 32 * c + 8 * gq);
                }
                kw[c] = wv;
            }
            f32x4 acc = f32x4{};
#pragma unroll
            for (int c = 0; c < DQK / 32; ++c) acc = mfma16x16x32(as_bf16x8(kw[c]), Qb[c], acc);
            Sacc[kb] = acc;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = t0 + kb * 16 + 4 * gq + i;
                const float sc = j < k_end ? Sacc[kb][i] * a.score_scale_log2 : -INFINITY;
                Sacc[kb][i] = sc;
                mx = fmaxf(mx, sc);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = exp2f(Sacc[kb][i] - m_use);
                Sacc[kb][i] = p;
                psum += p;
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int db = 0; db < DV / 16; ++db) O[db] *= alpha;
        // P^T: k-slot t of lane group gq is slot 4gq + t (t < 4) or 16 + 4gq + (t - 4).
        const bf16x8 Pb = as_bf16x8(u32x4{pack_bf16x2(Sacc[0][0], Sacc[0][1]),
                                          pack_bf16x2(Sacc[0][2], Sacc[0][3]),
                                          pack_bf16x2(Sacc[1][0], Sacc[1][1]),
                                          pack_bf16x2(Sacc[1][2], Sacc[1][3])});
        int jt[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) jt[t] = t0 + (t < 4 ? 4 * gq + t : 16 + 4 * gq + (t - 4));
#pragma unroll
        for (int db = 0; db < DV / 16; ++db) {
            const int d = db * 16 + l16;
            uint16_t e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int j = jt[t];
                e[t] = j < k_end ? (j == slot_new ? Vn[d] : vc[(int64_t)j * DV + d]) : (uint16_t)0;
            }
            const u32x4 vw = u32x4{(uint32_t)e[0] | ((uint32_t)e[1] << 16),
                                   (uint32_t)e[2] | ((uint32_t)e[3] << 16),
                                   (uint32_t)e[4] | ((uint32_t)e[5] << 16),
                                   (uint32_t)e[6] | ((uint32_t)e[7] << 16)};
            O[db] = mfma16x16x32(as_bf16x8(vw), Pb, O[db]);
        }
    }

    // ---- merge the waves of the workgroup.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (gq == 0) {
        red_m[wave][l16] = m_run;
        red_l[wave][l16] = l_run;
    }
#pragma unroll
    for (int db = 0; db < DV / 16; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[wave][l16][db * 16 + 4 * gq + i] = O[db][i];
    __syncthreads();

    for (int e = tid; e < 16 * DV; e += 256) {
        const int hh = e / DV, d = e % DV;
        if (hh >= G) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][hh]);
        const int h = g * G + hh;
        if (SPLIT) {
            const float Mu = (M == -INFINITY) ? 0.0f : M;
            float L = 0.0f, acc = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = exp2f(red_m[w][hh] - Mu);
                L += red_l[w][hh] * f;
                acc += red_o[w][hh][d] * f;
            }
            float* rec = a.partial + (((int64_t)b * a.Hq + h) * a.nsplit + s) * PSTRIDE;
            rec[d] = acc;
            if (d == 0) {
                rec[DV] = M;
                rec[DV + 1] = L;
            }
        } else {
            const float sk = SINK ? a.sinks[h] * kLog2e : -INFINITY;
            const float Ms = fmaxf(M, sk);
            const float Mu = (Ms == -INFINITY) ? 0.0f : Ms;
            float L = SINK ? exp2f(sk - Mu) : 0.0f, acc = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = exp2f(red_m[w][hh] - Mu);
                L += red_l[w][hh] * f;
                acc += red_o[w][hh][d] * f;
            }
            const float o = L > 0.0f ? a.v_scale * acc / L : 0.0f;
            a.out[((int64_t)b * a.Hq + h) * DV + d] = f32_to_bf16_bits(o);
        }
    }
}

// Merge the splits of one (sequence, query head); the sink joins the denominator once here.
template <bool SWA, bool SINK>
__global__ __launch_bounds__(128) void decode_combine_kernel(const DecodeArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int32_t pos = a.positions[b];
    uint16_t* o = a.out + ((int64_t)b * a.Hq + h) * DV;
    const bool pos_ok = pos >= 0 && pos <= a.max_position && (SWA || pos < a.cap);
    if (!pos_ok) {
        o[d] = 0;
        return;
    }
    const int n_valid = SWA ? min(a.window, pos + 1) : pos + 1;
    const int ns = (n_valid + a.chunk - 1) / a.chunk;
    const float* rec = a.partial + ((int64_t)b * a.Hq + h) * a.nsplit * PSTRIDE;
    const float sk = SINK ? a.sinks[h] * kLog2e : -INFINITY;
    float M = sk;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, rec[s * PSTRIDE + DV]);
    const float Mu = (M == -INFINITY) ? 0.0f : M;
    float L = SINK ? exp2f(sk - Mu) : 0.0f, acc = 0.0f;
    for (int s = 0; s < ns; ++s) {
        const float f = exp2f(rec[s * PSTRIDE + DV] - Mu);
        L += rec[s * PSTRIDE + DV + 1] * f;
        acc += rec[s * PSTRIDE + d] * f;
    }
    o[d] = f32_to_bf16_bits(L > 0.0f ? a.v_scale * acc / L : 0.0f);
}

template <bool SWA, bool SINK>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t st) {
    const dim3 grid(a.nsplit, a.Hkv, a.B);
    if (a.nsplit == 1) {
        decode_bf16_kernel<SWA, SINK, false><<<grid, 256, 0, st>>>(a);
        return hipGetLastError();
    }
    decode_bf16_kernel<SWA, SINK, true><<<grid, 256, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    decode_combine_kernel<SWA, SINK><<<dim3(a.Hq, a.B), DV, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, bool swa, bool sink, hipStream_t st) {
    if (a.B == 0) return hipSuccess;
    if (swa) return sink ? launch_typed<true, true>(a, st) : launch_typed<true, false>(a, st);
    return sink ? launch_typed<false, true>(a, st) : launch_typed<false, false>(a, st);
}

}  // namespace mimo
