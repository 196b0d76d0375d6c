// decode_bf16.hip — single-token decode of the hybrid attention layer against its KV cache.
//
// Pages: "Add Xiaomi MiMo-V2", section "Additional useful info" (per-kind theta and KV groups,
// decoupled V dim, value rescale, SWA-only sink); "add Xiaomi MiMo v2 (mimo_v2_flash)", section
// "Implementation plan" (sliding layers keep a rotating cache of the window).
//
// Per (sequence b, KV head g, split s) one workgroup of 4 waves:
//   * each wave issues the loads of its first 32-slot tile (K straight into MFMA operand layout,
//     V as coalesced 16-byte rows) early — on sliding layers before the position is even read —
//     so their latency overlaps the query rotation;
//   * the query heads of group g (<= 16) are rotated at the new token's position and kept as the
//     B operand of v_mfma_f32_16x16x32_bf16 (heads are the 16-wide N dimension);
//   * the split that owns the new token's slot rotates k_new, stores it and v_new into the cache
//     (linear: slot = position; ring: slot = position % window) and substitutes them for that
//     slot, so no workgroup reads a slot another one is writing;
//   * per tile: S^T = K * Q^T, online softmax per head in the log2 domain, V staged in a per-wave
//     LDS tile and read transposed with ds_read_b64_tr_b16, O^T += V^T * P^T; the next tile's
//     loads are in flight meanwhile (two waves per SIMD keep ~160 KB per CU in flight);
//   * the waves are merged through LDS; with one split the sink is folded in and the bf16 output
//     written, otherwise (max, sum, O) partials go to the workspace and the combine kernel merges
//     the splits in one pass (running maximum) and adds the sink exactly once.
#include "device_common.h"
#include "kernels.h"

namespace mimo {
namespace {

constexpr int DQK = 192;
constexpr int DV = 128;
constexpr int NW = 4;
constexpr int TILE = 32;                 // slots per wave iteration
constexpr int PSTRIDE = DV + 2;          // floats per partial record: O[128], m, l
constexpr int VT_PITCH = DV + 16;        // bf16 per V row in the per-wave LDS tile (288 bytes)
constexpr int KREG = 2 * (DQK / 32);     // 16-byte K operand loads per lane per tile (12)
constexpr int VREG = TILE * DV / 8 / 64; // 16-byte V loads per lane per tile (8)

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ u32x4 rotate8_dec(const u32x4& w, const u32x4& pw, int d0, int half,
                                             int32_t pos, const double* om) {
    float x[8], y[8];
    unpack8(w, x);
    unpack8(pw, y);
    const bool lower = d0 < half;
    const int f0 = lower ? d0 : d0 - half;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        float c, s;
        rope_cos_sin_rev(pos, om[f0 + t], c, s);
        x[t] = lower ? (x[t] * c - y[t] * s) : (x[t] * c + y[t] * s);
    }
    return pack8(x);
}

struct LdsDecode {
    uint16_t Qs[16 * DQK];
    uint16_t Kn[DQK];
    uint16_t Vn[DV];
    float red_m[NW][16], red_l[NW][16];
    union {
        uint16_t vt[NW][TILE * VT_PITCH];     // per-wave V tiles
        float red_o[NW][16][DV + 1];          // wave merge, after the slot loop
    } u;
};

template <bool SWA, bool SINK, bool SPLIT>
__global__ __launch_bounds__(256) void decode_bf16_kernel(const DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) LdsDecode sm;

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, gq = lane >> 4;
    const int G = a.Hq / a.Hkv;
    const int k_begin = s * a.chunk;
    const int64_t cache_row0 = ((int64_t)b * a.Hkv + g) * a.cap;
    const uint16_t* kc = a.k_cache + cache_row0 * DQK;
    const uint16_t* vc = a.v_cache + cache_row0 * DV;

    // ---- slot loads into registers, one tile ahead of the one being computed.  Slots past
    //      `limit` are not loaded; slots past the visible range and the new token's slot are fixed
    //      up when used.
    u32x4 kA[KREG], vA[VREG];
    auto fetch = [&](u32x4 (&kr)[KREG], u32x4 (&vr)[VREG], int t0, int limit) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int j = t0 + kb * 16 + l16;
#pragma unroll
            for (int c = 0; c < DQK / 32; ++c)
                kr[kb * (DQK / 32) + c] = j < limit ? *(const u32x4*)(kc + (int64_t)j * DQK + 32 * c + 8 * gq)
                                                    : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < VREG; ++it) {
            const int e = lane + 64 * it;
            const int j = t0 + e / (DV / 8);
            vr[it] = j < limit ? *(const u32x4*)(vc + (int64_t)j * DV + (e % (DV / 8)) * 8)
                               : u32x4{0u, 0u, 0u, 0u};
        }
    };
    const int stride = NW * TILE;
    int t0 = k_begin + wave * TILE;
    if (SWA) fetch(kA, vA, t0, a.cap);  // every ring slot is in bounds: start before the position is known

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
    if (k_begin >= n_valid) return;
    const int k_end = min(n_valid, k_begin + a.chunk);
    const bool own_new = slot_new >= k_begin && slot_new < k_end;
    const int r = a.rope_dims, half = r >> 1;
    if (!SWA) fetch(kA, vA, t0, k_end);

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
                wv = rotate8_dec(wv, *(const u32x4*)(qrow + pd), d0, half, pos, a.omega_rev);
            }
        }
        *(u32x4*)(sm.Qs + hh * DQK + col * 8) = wv;
    }
    // ---- the new token: rotate, keep in LDS, append to the cache.
    if (own_new && tid < DQK / 8 + DV / 8) {
        if (tid < DQK / 8) {
            const uint16_t* krow = a.k_new + ((int64_t)b * a.Hkv + g) * DQK;
            const int d0 = tid * 8;
            u32x4 wv = *(const u32x4*)(krow + d0);
            if (d0 < r) {
                const int pd = d0 < half ? d0 + half : d0 - half;
                wv = rotate8_dec(wv, *(const u32x4*)(krow + pd), d0, half, pos, a.omega_rev);
            }
            *(u32x4*)(sm.Kn + d0) = wv;
            *(u32x4*)(a.k_cache + (cache_row0 + slot_new) * DQK + d0) = wv;
        } else {
            const int d0 = (tid - DQK / 8) * 8;
            const u32x4 wv = *(const u32x4*)(a.v_new + ((int64_t)b * a.Hkv + g) * DV + d0);
            *(u32x4*)(sm.Vn + d0) = wv;
            *(u32x4*)(a.v_cache + (cache_row0 + slot_new) * DV + d0) = wv;
        }
    }
    __syncthreads();

    bf16x8 Qb[DQK / 32];
#pragma unroll
    for (int c = 0; c < DQK / 32; ++c) Qb[c] = *(const bf16x8*)(sm.Qs + l16 * DQK + 32 * c + 8 * gq);

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 O[DV / 16];
#pragma unroll
    for (int db = 0; db < DV / 16; ++db) O[db] = f32x4{};
    uint16_t* vt = sm.u.vt[wave];
    const float sc = a.score_scale_log2;

    // consume the tile held in (kr, vr) at slot t, refilling the registers with the next tile as
    // soon as the scores are formed
    auto consume = [&](u32x4 (&kr)[KREG], u32x4 (&vr)[VREG], int t) {
        if (own_new && slot_new >= t && slot_new < t + TILE) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                if (t + kb * 16 + l16 == slot_new) {
#pragma unroll
                    for (int c = 0; c < DQK / 32; ++c)
                        kr[kb * (DQK / 32) + c] = *(const u32x4*)(sm.Kn + 32 * c + 8 * gq);
                }
#pragma unroll
            for (int it = 0; it < VREG; ++it) {
                const int e = lane + 64 * it;
                if (t + e / (DV / 8) == slot_new) vr[it] = *(const u32x4*)(sm.Vn + (e % (DV / 8)) * 8);
            }
        }
        // V rows -> this wave's LDS tile (rows past the visible range as zeros)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < VREG; ++it) {
            const int e = lane + 64 * it;
            const int row = e / (DV / 8);
            *(u32x4*)(vt + row * VT_PITCH + (e % (DV / 8)) * 8) =
                (t + row < k_end) ? vr[it] : u32x4{0u, 0u, 0u, 0u};
        }
        // S^T (16 slots x 16 heads) for the two 16-slot blocks of the tile
        f32x4 Sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x4 acc = f32x4{};
#pragma unroll
            for (int c = 0; c < DQK / 32; ++c)
                acc = mfma16x16x32(as_bf16x8(kr[kb * (DQK / 32) + c]), Qb[c], acc);
            Sacc[kb] = acc;
        }
        fetch(kr, vr, t + stride, k_end);

        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = t + kb * 16 + 4 * gq + i;
                const float v = j < k_end ? Sacc[kb][i] * sc : -INFINITY;
                Sacc[kb][i] = v;
                mx = fmaxf(mx, v);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float psum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(Sacc[kb][i] - m_use);
                Sacc[kb][i] = p;
                psum += p;
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int db = 0; db < DV / 16; ++db) O[db] *= alpha;
        // P^T: k-slot t' of lane group gq is slot 4gq + t' (t' < 4) or 16 + 4gq + (t' - 4).
        const bf16x8 Pb = as_bf16x8(u32x4{pack_bf16x2(Sacc[0][0], Sacc[0][1]),
                                          pack_bf16x2(Sacc[0][2], Sacc[0][3]),
                                          pack_bf16x2(Sacc[1][0], Sacc[1][1]),
                                          pack_bf16x2(Sacc[1][2], Sacc[1][3])});
        __builtin_amdgcn_wave_barrier();
        // V^T operand: lane j of group gq points at V[key0 + j/4][16db + 4(j%4)] and receives
        // V[key0 + t'][16db + j], t' < 4, with key0 = 4gq (first read) and 16 + 4gq (second).
#pragma unroll
        for (int db = 0; db < DV / 16; ++db) {
            const int col = db * 16 + 4 * (l16 & 3);
            const int row = 4 * gq + (l16 >> 2);
            const bf16x4 v0 =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vt + row * VT_PITCH + col));
            const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(vt + (row + 16) * VT_PITCH + col));
            const bf16x8 A = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            O[db] = mfma16x16x32(A, Pb, O[db]);
        }
    };
    for (; t0 < k_end; t0 += stride) consume(kA, vA, t0);

    // ---- merge the waves of the workgroup (the V tiles are dead now; red_o reuses them).
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    __syncthreads();
    if (gq == 0) {
        sm.red_m[wave][l16] = m_run;
        sm.red_l[wave][l16] = l_run;
    }
#pragma unroll
    for (int db = 0; db < DV / 16; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.u.red_o[wave][l16][db * 16 + 4 * gq + i] = O[db][i];
    __syncthreads();

    for (int e = tid; e < 16 * DV; e += 256) {
        const int hh = e / DV, d = e % DV;
        if (hh >= G) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.red_m[w][hh]);
        const int h = g * G + hh;
        if (SPLIT) {
            const float Mu = (M == -INFINITY) ? 0.0f : M;
            float L = 0.0f, acc = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = fast_exp2(sm.red_m[w][hh] - Mu);
                L += sm.red_l[w][hh] * f;
                acc += sm.u.red_o[w][hh][d] * f;
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
            float L = SINK ? fast_exp2(sk - Mu) : 0.0f, acc = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = fast_exp2(sm.red_m[w][hh] - Mu);
                L += sm.red_l[w][hh] * f;
                acc += sm.u.red_o[w][hh][d] * f;
            }
            const float o = L > 0.0f ? a.v_scale * acc / L : 0.0f;
            a.out[((int64_t)b * a.Hq + h) * DV + d] = f32_to_bf16_bits(o);
        }
    }
}

// Merge the splits of one (sequence, query head); the sink joins the denominator once, here.  One
// thread per output dim; the records of up to 32 splits are loaded in one round trip, then merged
// against their common maximum (chunks of 32 are chained with a running maximum).
template <bool SWA, bool SINK>
__global__ __launch_bounds__(128) void decode_combine_kernel(const DecodeArgs a) {
    constexpr int CH = 32;
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int32_t pos = a.positions[b];
    uint16_t* o = a.out + ((int64_t)b * a.Hq + h) * DV;
    const bool pos_ok = pos >= 0 && pos <= a.max_position && (SWA || pos < a.cap);
    if (!pos_ok) {
        o[d] = 0;
        return;
    }
    const int n_valid = SWA ? min(a.window, pos + 1) : pos + 1;
    const int ns = (n_valid + a.chunk - 1) / a.chunk;   // every one of these splits wrote a record
    const float* rec = a.partial + ((int64_t)b * a.Hq + h) * a.nsplit * PSTRIDE;
    float M = SINK ? a.sinks[h] * kLog2e : -INFINITY;
    float L = SINK ? 1.0f : 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < ns; s0 += CH) {
        float m[CH], l[CH], x[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const bool ok = s0 + i < ns;
            const float* r = rec + (int64_t)(s0 + i) * PSTRIDE;
            m[i] = ok ? r[DV] : -INFINITY;
            l[i] = ok ? r[DV + 1] : 0.0f;
            x[i] = ok ? r[d] : 0.0f;
        }
        float Mc = M;
#pragma unroll
        for (int i = 0; i < CH; ++i) Mc = fmaxf(Mc, m[i]);
        const float Mu = (Mc == -INFINITY) ? 0.0f : Mc;
        const float f = fast_exp2(M - Mu);
        L *= f;
        acc *= f;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const float wgt = fast_exp2(m[i] - Mu);
            L += l[i] * wgt;
            acc += x[i] * wgt;
        }
        M = Mc;
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

int decode_max_splits() { return 1024; }

hipError_t launch_decode_bf16(const DecodeArgs& a, bool swa, bool sink, hipStream_t st) {
    if (a.B == 0) return hipSuccess;
    if (a.nsplit > decode_max_splits()) return hipErrorInvalidConfiguration;
    if (swa) return sink ? launch_typed<true, true>(a, st) : launch_typed<true, false>(a, st);
    return sink ? launch_typed<false, true>(a, st) : launch_typed<false, false>(a, st);
}

}  // namespace mimo
