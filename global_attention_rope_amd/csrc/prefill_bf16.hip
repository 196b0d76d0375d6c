// prefill_bf16.hip — flash-style prefill of the hybrid attention layer on gfx950 bf16 MFMA.
//
// Computes, for one layer (pages: "Add Xiaomi MiMo-V2", section "Additional useful info";
// "add Xiaomi MiMo v2 (mimo_v2_flash)", section "Architecture, verified against upstream"):
//   out[b,i,h,:] = v_scale * sum_j e^{z_ij} v_j / (e^{s_h} + sum_j e^{z_ij})
//   z_ij = tau * <rot(q_i, p_i), rot(k_j, p_j)>, keys j visible by the causal or window mask,
//   partial RoPE on the first r dims, GQA head h -> KV head h / (Hq / Hkv), optional sink s_h.
//
// Shape of the computation (qk head dim 192, v head dim 128):
//   * one workgroup = 4 waves = 128 query rows of one query head; each wave owns 32 rows; two
//     workgroups share a CU (<= 256 registers per lane);
//   * scores are formed transposed, S^T = K * Q^T, with v_mfma_f32_32x32x16_bf16: the MFMA
//     result column is the query, so every lane holds whole columns of S^T for "its" query and
//     the softmax row statistics need one exchange between lane l and l+32;
//   * rotated Q (bf16) lives in registers as the B operand for the whole kernel; the RoPE of Q is
//     applied while it is loaded;
//   * K tiles (64 keys x 192, 400-byte LDS rows: conflict-free 16-byte reads) and V tiles (64 keys
//     x 128, 320-byte rows) are staged row-major; the next tile is fetched into registers while
//     the current one is computed;
//   * for sliding-window layers the raw K rows are rotated in LDS right after staging (one thread
//     per pair of 8-dim chunks); global layers read keys rotated once by the cache-store pass;
//   * O^T = V^T * P^T takes P^T straight from the score registers; the V^T operand comes from
//     the row-major tile with ds_read_b64_tr_b16 (4 keys x 1 dv column per lane per read), in the
//     key order of the score layout;
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
constexpr int V_PITCH = DV + 32;     // bf16 per V row in LDS (320 bytes)
constexpr int KCH = DQK / 16;        // 16-wide k chunks of the QK contraction
constexpr int K_LOADS = BN * DQK / 8 / 256;   // 16-byte K chunks per thread per tile (6)
constexpr int V_LOADS = BN * DV / 8 / 256;    // 16-byte V chunks per thread per tile (4)

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Rotate the 8 dims held in lo (dims f0..f0+7 < r/2) against their partners hi (dims + r/2).
__device__ __forceinline__ void rotate_pair8(u32x4& lo, u32x4& hi, int32_t pos, const double* om) {
    float x[8], y[8];
    unpack8(lo, x);
    unpack8(hi, y);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        float c, s;
        rope_cos_sin_rev(pos, om[t], c, s);
        const float xl = x[t], xh = y[t];
        x[t] = xl * c - xh * s;
        y[t] = xh * c + xl * s;
    }
    lo = pack8(x);
    hi = pack8(y);
}

template <bool SWA, bool SINK, bool ROTK>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(const PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * K_PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[BN * V_PITCH];
    __shared__ __attribute__((aligned(16))) double om_s[kMaxRopeHalf];

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

    for (int f = tid; f < half; f += 256) om_s[f] = a.omega_rev[f];
    __syncthreads();

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
        u32x4 qw[KCH];
#pragma unroll
        for (int c = 0; c < KCH; ++c) qw[c] = *(const u32x4*)(qrow + 16 * c + 8 * g);
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int d0 = 16 * c + 8 * g;
            if (d0 < r) {
                const bool lower = d0 < half;
                u32x4 lo = lower ? qw[c] : *(const u32x4*)(qrow + d0 - half);
                u32x4 hi = lower ? *(const u32x4*)(qrow + d0 + half) : qw[c];
                rotate_pair8(lo, hi, p0 + qi, om_s + (lower ? d0 : d0 - half));
                qw[c] = lower ? lo : hi;
            }
            if (!qok) qw[c] = u32x4{0u, 0u, 0u, 0u};
            Qb[c] = as_bf16x8(qw[c]);
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
    const uint16_t* kbase = a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
    const int32_t koff = a.k_pos_off ? p0 : 0;
    const uint16_t* vbase = a.v + (int64_t)b * S * a.Hkv * DV + (int64_t)kvh * DV;
    const int64_t v_sj = (int64_t)a.Hkv * DV;

    u32x4 kreg[K_LOADS], vreg[V_LOADS];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int it = 0; it < K_LOADS; ++it) {
            const int cidx = tid + it * 256;
            const int row = cidx / (DQK / 8), col = cidx % (DQK / 8);
            const int j = j0 + row;
            kreg[it] = j < S ? *(const u32x4*)(kbase + (int64_t)(j + koff) * a.k_sj + col * 8)
                             : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < V_LOADS; ++it) {
            const int cidx = tid + it * 256;
            const int row = cidx / (DV / 8), col = cidx % (DV / 8);
            const int j = j0 + row;
            vreg[it] = j < S ? *(const u32x4*)(vbase + (int64_t)j * v_sj + col * 8)
                             : u32x4{0u, 0u, 0u, 0u};
        }
    };
    fetch(kt_lo * BN);

    const int q_l = q_first + l32;   // this lane's query row
    const int qsel = lane >> 4, jsel = lane & 15;   // ds_read_tr lane roles

    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
        const int j0 = kt * BN;
        // ---- registers -> LDS
#pragma unroll
        for (int it = 0; it < K_LOADS; ++it) {
            const int cidx = tid + it * 256;
            *(u32x4*)(Ks + (cidx / (DQK / 8)) * K_PITCH + (cidx % (DQK / 8)) * 8) = kreg[it];
        }
#pragma unroll
        for (int it = 0; it < V_LOADS; ++it) {
            const int cidx = tid + it * 256;
            *(u32x4*)(Vs + (cidx / (DV / 8)) * V_PITCH + (cidx % (DV / 8)) * 8) = vreg[it];
        }
        __syncthreads();
        if (ROTK && r > 0) {
            // rotate raw keys in place: one thread per (row, 8-dim chunk below r/2)
            const int per_row = half / 8;
            for (int e = tid; e < BN * per_row; e += 256) {
                const int row = e / per_row, c8 = (e % per_row) * 8;
                uint16_t* kr = Ks + row * K_PITCH;
                u32x4 lo = *(const u32x4*)(kr + c8);
                u32x4 hi = *(const u32x4*)(kr + c8 + half);
                rotate_pair8(lo, hi, p0 + j0 + row, om_s + c8);
                *(u32x4*)(kr + c8) = lo;
                *(u32x4*)(kr + c8 + half) = hi;
            }
            __syncthreads();
        }
        if (kt < kt_hi) fetch(j0 + BN);   // next tile in flight during the compute below

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
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float s = Sacc[kb][i] * a.score_scale_log2;
                    if (!full) {
                        const int j = j0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                        const bool ok = j <= q_l && j < S && (!SWA || q_l - j < a.window);
                        s = ok ? s : -INFINITY;
                    }
                    Sacc[kb][i] = s;
                    mx = fmaxf(mx, s);
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            m_run = m_new;
            float psum = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(Sacc[kb][i] - m_use);
                    Sacc[kb][i] = p;
                    psum += p;
                }
            }
            l_run = l_run * alpha + psum;
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int db = 0; db < DV / 32; ++db) O[db] *= alpha;
            }

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
            // 16c + 8 + 4g + (t - 4) (t >= 4), matching the score register order.  Each
            // ds_read_b64_tr_b16 hands lane i of a 16-lane group V[key0 + t][dv0 + i], t < 4,
            // when lane i points at V[key0 + i/4][dv0 + 4*(i%4)].
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int key0 = 16 * c + 4 * (qsel >> 1) + (jsel >> 2);
#pragma unroll
                for (int db = 0; db < DV / 32; ++db) {
                    const int col = db * 32 + 16 * (qsel & 1) + 4 * (jsel & 3);
                    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4*)(Vs + key0 * V_PITCH + col));
                    const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (lds_bf16x4*)(Vs + (key0 + 8) * V_PITCH + col));
                    const bf16x8 A = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                    O[db] = mfma32x32x16(A, Pb[c], O[db]);
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: out = v_scale * O / l, bf16.
    const float lt = l_run + __shfl_xor(l_run, 32);
    const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
    if (q_l < S) {
        uint16_t* orow = a.out + (((int64_t)b * S + q_l) * Hq + h) * DV;
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
