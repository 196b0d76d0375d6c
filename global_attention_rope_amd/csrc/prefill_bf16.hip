// prefill_bf16.hip — flash-style prefill of the hybrid attention layer on gfx950 bf16 MFMA.
//
// Computes, for one layer (pages: "Add Xiaomi MiMo-V2", section "Additional useful info";
// "add Xiaomi MiMo v2 (mimo_v2_flash)", section "Architecture, verified against upstream"):
//   out[b,i,h,:] = v_scale * sum_j e^{z_ij} v_j / (e^{s_h} + sum_j e^{z_ij})
//   z_ij = tau * <rot(q_i, p_i), rot(k_j, p_j)>, keys j visible by the causal or window mask,
//   partial RoPE on the first r dims, GQA head h -> KV head h / (Hq / Hkv), optional sink s_h.
//
// Shape of the computation (qk head dim 192, v head dim 128):
//   * one workgroup = 4 waves = 128 query rows of one query head; each wave owns 32 rows;
//   * scores are formed transposed, S^T = K * Q^T, with v_mfma_f32_32x32x16_bf16: the MFMA
//     result column is the query, so every lane holds whole columns of S^T for "its" query and
//     the softmax row statistics need one exchange between lane l and l+32;
//   * rotated Q (bf16) lives in registers as the B operand for the whole kernel; the RoPE of Q is
//     applied while it is loaded;
//   * K tiles (64 keys x 192) are staged in LDS with a 400-byte row pitch (conflict-free 16-byte
//     reads); for sliding-window layers the raw K is rotated while it is staged;
//   * V tiles are staged transposed (V^T, 128 x 64 keys, 136-byte pitch) so that O^T = V^T * P^T
//     takes P^T straight from the score registers, with the key order of the score layout;
//   * online softmax in the log2 domain; the sink enters as the initial running maximum and a
//     running sum of 1 (it is one extra logit that carries no value);
//   * tiles outside the causal/window band are skipped; only tiles crossing the band edges are
//     masked element by element;
//   * workgroups are ordered heavy-first (late query blocks first on global layers) and grouped so
//     that the 8 workgroups the dispatcher sends to one XCD in a row share a KV head.
#include "device_common.h"
#include "kernels.h"

namespace mimo {
namespace {

constexpr int DQK = 192;
constexpr int DV = 128;
constexpr int BN = 64;               // keys per tile
constexpr int NWAVES = 4;
constexpr int QPW = 32;              // query rows per wave
constexpr int BM = NWAVES * QPW;     // query rows per workgroup
constexpr int K_PITCH = DQK + 8;     // bf16 per K row in LDS (400 bytes)
constexpr int VT_PITCH = BN + 4;     // bf16 per V^T row in LDS (136 bytes)
constexpr int KCH = DQK / 16;        // 16-wide k chunks of the QK contraction

// Rotate 8 consecutive dims [d0, d0+8) of a row held in w, given the 8 partner dims in pw
// (d0 +- r/2), at position pos.  r/2 is a multiple of 8 so the block never straddles r/2.
__device__ __forceinline__ u32x4 rotate8(const u32x4& w, const u32x4& pw, int d0, int half,
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

template <bool SWA, bool SINK, bool ROTK>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(const PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * K_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[DV * VT_PITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int S = a.S, Hq = a.Hq;
    const int nqblk = (S + BM - 1) / BM;
    const int total = a.B * Hq * nqblk;

    // Work item: XCD-grouped, heavy-first.
    const int id = blockIdx.x;
    int w = id;
    {
        const int xcd = id & 7, slot = id >> 3, grp = slot >> 3;
        if ((grp + 1) * 64 <= total) w = grp * 64 + xcd * 8 + (slot & 7);
    }
    const int h = w % Hq;
    const int b = (w / Hq) % a.B;
    const int qrank = w / (Hq * a.B);
    const int qblk = SWA ? qrank : (nqblk - 1 - qrank);
    const int kvh = h / (Hq / a.Hkv);
    const int32_t p0 = a.start_pos[b];
    const int r = a.rope_dims, half = r >> 1;

    const int q_first = qblk * BM + wave * QPW;              // this wave's first query row
    const int q_last = min(q_first + QPW, S) - 1;            // last valid row (< q_first if none)
    const int blk_first = qblk * BM;
    const int blk_last = min(blk_first + BM, S) - 1;

    // ---- Q^T operands, rotated, in registers.
    bf16x8 Qb[KCH];
    {
        const int qi = q_first + l32;
        const bool qok = qi < S;
        const uint16_t* qrow = a.q + (((int64_t)b * S + (qok ? qi : S - 1)) * Hq + h) * DQK;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int d0 = 16 * c + 8 * g;
            u32x4 wv = *(const u32x4*)(qrow + d0);
            if (d0 < r) {
                const int pd = d0 < half ? d0 + half : d0 - half;
                const u32x4 pw = *(const u32x4*)(qrow + pd);
                wv = rotate8(wv, pw, d0, half, p0 + qi, a.omega);
            }
            if (!qok) wv = u32x4{0u, 0u, 0u, 0u};
            Qb[c] = as_bf16x8(wv);
        }
    }

    const float sink_l2 = SINK ? a.sinks[h] * kLog2e : -INFINITY;
    float m_run = SINK ? sink_l2 : -INFINITY;
    float l_run = (SINK && g == 0) ? 1.0f : 0.0f;
    f32x16 O[DV / 32];
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) O[db] = f32x16{};

    const int kt_lo = SWA ? max(0, blk_first - a.window + 1) / BN : 0;
    const int kt_hi = blk_last / BN;
    const int64_t kbase = (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
    const int32_t koff = a.k_pos_off ? p0 : 0;

    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
        const int j0 = kt * BN;
        // ---- stage K (rotated when ROTK) into LDS: 64 rows x 24 chunks of 8.
#pragma unroll
        for (int it = 0; it < (BN * DQK / 8) / 256; ++it) {
            const int cidx = tid + it * 256;
            const int row = cidx / (DQK / 8), col = cidx % (DQK / 8);
            const int j = j0 + row;
            u32x4 wv = u32x4{0u, 0u, 0u, 0u};
            if (j < S) {
                const uint16_t* krow = a.k + kbase + (int64_t)(j + koff) * a.k_sj;
                wv = *(const u32x4*)(krow + col * 8);
                if (ROTK && col * 8 < r) {
                    const int d0 = col * 8;
                    const int pd = d0 < half ? d0 + half : d0 - half;
                    const u32x4 pw = *(const u32x4*)(krow + pd);
                    wv = rotate8(wv, pw, d0, half, p0 + j, a.omega);
                }
            }
            *(u32x4*)(Ks + row * K_PITCH + col * 8) = wv;
        }
        // ---- stage V^T into LDS: thread = (dv pair, group of 16 keys).
        {
            const int dp = tid & 63, kg = tid >> 6;
            uint32_t vals[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int j = j0 + kg * 16 + t;
                vals[t] = j < S ? *(const uint32_t*)(a.v + (((int64_t)b * S + j) * a.Hkv + kvh) * DV +
                                                     2 * dp)
                                : 0u;
            }
            uint16_t* r0 = Vt + (2 * dp) * VT_PITCH + kg * 16;
            uint16_t* r1 = r0 + VT_PITCH;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t a0 = vals[4 * t], a1 = vals[4 * t + 1], a2 = vals[4 * t + 2],
                               a3 = vals[4 * t + 3];
                *(u32x2*)(r0 + 4 * t) = u32x2{(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
                *(u32x2*)(r1 + 4 * t) =
                    u32x2{(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
            }
        }
        __syncthreads();

        // ---- does this wave see any key of the tile?
        const bool wave_live = q_first <= q_last && j0 <= q_last &&
                               (!SWA || j0 + BN - 1 > q_first - a.window);
        if (wave_live) {
            const bool full = (j0 + BN - 1 <= q_first) && (!SWA || q_last - j0 < a.window);
            f32x16 Sacc[2];
            Sacc[0] = f32x16{};
            Sacc[1] = f32x16{};
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 A = *(const bf16x8*)(Ks + (kb * 32 + l32) * K_PITCH + 16 * c + 8 * g);
                    Sacc[kb] = mfma32x32x16(A, Qb[c], Sacc[kb]);
                }
            }
            const int qi = q_first + l32;
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float s = Sacc[kb][i] * a.score_scale_log2;
                    if (!full) {
                        const int j = j0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                        const bool ok = j <= qi && j < S && (!SWA || qi - j < a.window);
                        s = ok ? s : -INFINITY;
                    }
                    Sacc[kb][i] = s;
                    mx = fmaxf(mx, s);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = exp2f(m_run - m_use);
            m_run = m_new;
            float psum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = exp2f(Sacc[kb][i] - m_use);
                    Sacc[kb][i] = p;
                    psum += p;
                }
            }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int db = 0; db < DV / 32; ++db) O[db] *= alpha;

            // P^T operands: 16-key chunk c = registers 8*(c%2) .. +8 of block c/2.
            bf16x8 Pb[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u32x4 pw;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    pw[t] = pack_bf16x2(Sacc[c >> 1][8 * (c & 1) + 2 * t],
                                        Sacc[c >> 1][8 * (c & 1) + 2 * t + 1]);
                Pb[c] = as_bf16x8(pw);
            }
            // O^T += V^T * P^T.  k-slot t of lane group g is key 16c + 4g + t (t < 4) or
            // 16c + 8 + 4g + (t - 4) (t >= 4), matching the score register order.
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int db = 0; db < DV / 32; ++db) {
                    const uint16_t* vr = Vt + (db * 32 + l32) * VT_PITCH + 16 * c + 4 * g;
                    const u32x2 lo = *(const u32x2*)vr;
                    const u32x2 hi = *(const u32x2*)(vr + 8);
                    const bf16x8 A = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
                    O[db] = mfma32x32x16(A, Pb[c], O[db]);
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: out = v_scale * O / l, bf16.
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
    const int qi = q_first + l32;
    if (qi < S) {
        uint16_t* orow = a.out + (((int64_t)b * S + qi) * Hq + h) * DV;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int d = db * 32 + 8 * ii + 4 * g;
                *(u32x2*)(orow + d) =
                    u32x2{pack_bf16x2(O[db][4 * ii] * inv, O[db][4 * ii + 1] * inv),
                          pack_bf16x2(O[db][4 * ii + 2] * inv, O[db][4 * ii + 3] * inv)};
            }
        }
    }
}

}  // namespace

int prefill_bf16_block_rows() { return BM; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, bool swa, bool sink, bool rot_k,
                               hipStream_t st) {
    const int nqblk = (a.S + BM - 1) / BM;
    const int64_t total = (int64_t)a.B * a.Hq * nqblk;
    if (total == 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)total), block(256);
    if (swa && !rot_k) return hipErrorInvalidValue;  // sliding layers always rotate K in-kernel
    if (swa) {
        if (sink) prefill_bf16_kernel<true, true, true><<<grid, block, 0, st>>>(a);
        else prefill_bf16_kernel<true, false, true><<<grid, block, 0, st>>>(a);
    } else if (rot_k) {
        if (sink) prefill_bf16_kernel<false, true, true><<<grid, block, 0, st>>>(a);
        else prefill_bf16_kernel<false, false, true><<<grid, block, 0, st>>>(a);
    } else {
        if (sink) prefill_bf16_kernel<false, true, false><<<grid, block, 0, st>>>(a);
        else prefill_bf16_kernel<false, false, false><<<grid, block, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace mimo
