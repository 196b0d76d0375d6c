// verify_bf16.hip — a few new tokens per sequence (speculative or multi-token verification, short
// extends) against the key rows of their sequence, on gfx950 bf16 MFMA.
//
// Same layer as the prefill kernel (pages: "Add Xiaomi MiMo-V2", "Additional useful info";
// "add Xiaomi MiMo v2 (mimo_v2_flash)", "Architecture, verified against upstream" and
// "Implementation plan"), shaped for T <= 16 queries per sequence: the query columns of the
// S^T = K * Q^T products are (query head, token) pairs of one KV group — 16 heads x 4 tokens fill
// two 32-column waves — so every K/V tile is read from memory once per (sequence, KV head) and
// feeds all heads and tokens.  The key rows are split across workgroups (split-K); each split
// writes (O, max, sum) partials for the decode combine kernel, or the output when there is one.
// Tiles: 64 keys, staged through a 2-stage LDS ring by global_load_lds_dwordx4, XOR-swizzled as
// in the prefill kernel; per-column online softmax in the log2 domain with a lazily raised
// running maximum.
#include <type_traits>

#include "device_common.h"
#include "verify.h"

namespace mimo {
namespace {

constexpr int DQK = 192;
constexpr int DV = 128;
constexpr int BN = 64;                       // keys per tile
constexpr int K_TILE = BN * DQK * 2;         // bytes
constexpr int V_TILE = BN * DV * 2;
constexpr int KCH = DQK / 16;
constexpr int STAGES = 2;
constexpr int PSTRIDE = DV + 2;              // floats per partial record: O[128], m, l
constexpr float kRescaleLog2 = 8.0f;         // raise the running max only beyond 2^8

template <int NW, bool WINDOW, bool SINK, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void verify_tiles_kernel(const VerifyArgs a) {
    constexpr int K_DMA = K_TILE / 1024 / NW;      // 1-KiB DMA instructions per wave per tile
    constexpr int V_DMA = V_TILE / 1024 / NW;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * (K_TILE + V_TILE)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int Hq = a.Hq, T = a.T, TP = a.TP;
    const int G = Hq / a.Hkv;

    // this lane's column: query head kvh * G + hl, token t
    const int col = wave * 32 + l32;
    const int hl = col / TP, t = col - hl * TP;
    const bool col_ok = hl < G && t < T;
    const int h = kvh * G + min(hl, G - 1);
    const int tq = min(t, T - 1);

    // the column's query row and the rotation partners of its rotated dims go out first: they do
    // not depend on the start position, which then comes by a scalar load that leaves them in flight
    const uint16_t* qrow = a.q + (((int64_t)b * T + tq) * Hq + h) * DQK;
    const int r = a.rope_dims, half = r >> 1;
    u32x4 qw[KCH], pw[KCH];
#pragma unroll
    for (int c = 0; c < KCH; ++c) qw[c] = *(const u32x4*)(qrow + 16 * c + 8 * g);
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const int d0 = 16 * c + 8 * g;
        if (d0 < r) pw[c] = *(const u32x4*)(qrow + (d0 < half ? d0 + half : d0 - half));
    }

    // key rows: row j sits at position kpos0 + j, token t meets row t + shift at its own position
    const int32_t st = load_scalar_i32(a.start_pos + b);
    const bool seq_ok = (unsigned)st <= (unsigned)a.max_start;
    const int32_t kpos0 = (a.kpos_rel ? (seq_ok ? st : 0) : 0) + a.kpos_off;
    const int shift = (seq_ok ? st : 0) - kpos0;
    const int jmin = max(0, -kpos0);
    const int nk = T + shift;                        // rows the last token reaches
    const int W = a.window;

    if (!seq_ok) {   // defined result: zero output (a split combine writes the zeros itself)
        if (!SPLIT && col_ok) {
            uint16_t* orow = a.out + (((int64_t)b * T + t) * Hq + h) * DV;
            for (int d = 4 * g; d < DV; d += 8) *(u32x2*)(orow + d) = u32x2{0u, 0u};
        }
        return;
    }
    const int k_begin = s * a.chunk;
    if (k_begin >= nk) return;                       // no token reads this split's record
    // rows [r0, r1) of this split that some token sees (chunk is a multiple of the tile)
    const int lo = max(jmin, WINDOW ? shift - W + 1 : 0);
    const int r0 = max(k_begin, lo), r1 = min(k_begin + a.chunk, nk);
    const int kt_lo = r0 / BN;
    const int n_tiles = r1 > r0 ? (r1 - 1) / BN + 1 - kt_lo : 0;

    // ---- DMA source mapping (LDS 16-byte slot P of this wave's instruction i holds K row P / 24,
    //      chunk (P % 24) ^ swizzle; V row P / 16, chunk (P % 16) ^ swizzle)
    const uint16_t* kslice = a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
    const uint16_t* vslice = a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;
    // rows held by a ring cache (the earlier positions of a sliding layer), read in place
    const int ring_w = a.ring_k ? a.ring_w : 0;
    const int64_t ring_row0 = ((int64_t)b * a.Hkv + kvh) * (ring_w > 0 ? ring_w : 1);
    const uint16_t* ring_k = ring_w > 0 ? a.ring_k + ring_row0 * DQK : nullptr;
    const uint16_t* ring_v = ring_w > 0 ? a.ring_v + ring_row0 * DV : nullptr;
    int k_row[K_DMA], k_off[K_DMA], v_row[V_DMA], v_off[V_DMA];
#pragma unroll
    for (int i = 0; i < K_DMA; ++i) {
        const int P = (wave * K_DMA + i) * 64 + lane;
        const int row = P / (DQK / 8), phys = P % (DQK / 8);
        k_row[i] = row;
        k_off[i] = (phys ^ ((row >> 1) & 7)) * 8;
    }
#pragma unroll
    for (int i = 0; i < V_DMA; ++i) {
        const int P = (wave * V_DMA + i) * 64 + lane;
        const int row = P / (DV / 8), phys = P % (DV / 8);
        v_row[i] = row;
        v_off[i] = (phys ^ ((row & 3) << 2)) * 8;
    }
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8_t*)smem;
    // rows outside [jmin, nk) are clamped into it (masked anyway; unwritten rows stay unread)
    auto issue = [&](int tt, auto stage_c) {
        constexpr int ST = decltype(stage_c)::value;
        const int j0 = (kt_lo + tt) * BN;
        const uint32_t kst = lds0 + ST * K_TILE;
        const uint32_t vst = lds0 + STAGES * K_TILE + ST * V_TILE;
#pragma unroll
        for (int i = 0; i < K_DMA; ++i) {
            const int j = min(max(j0 + k_row[i], jmin), nk - 1);
            const uint16_t* src = j < ring_w ? ring_k + (int64_t)((kpos0 + j) % ring_w) * DQK
                                             : kslice + (int64_t)j * DQK;
            dma16(src + k_off[i], kst + (wave * K_DMA + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < V_DMA; ++i) {
            const int j = min(max(j0 + v_row[i], jmin), nk - 1);
            const uint16_t* src = j < ring_w ? ring_v + (int64_t)((kpos0 + j) % ring_w) * DV
                                             : vslice + (int64_t)j * DV;
            dma16(src + v_off[i], vst + (wave * V_DMA + i) * 1024);
        }
    };
    if (n_tiles > 0) issue(0, std::integral_constant<int, 0>{});

    // ---- Q^T operands of this column, rotated at the token's position, in registers
    bf16x8 Qb[KCH];
    {
        const int32_t pos = st + tq;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int d0 = 16 * c + 8 * g;
            if (d0 < r) {
                const bool lower = d0 < half;
                float x[8], y[8];
                unpack8(qw[c], x);
                unpack8(pw[c], y);
                const int f0 = lower ? d0 : d0 - half;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float cs, sn;
                    rope_cos_sin_rev(pos, a.omega_rev[f0 + e], cs, sn);
                    x[e] = lower ? x[e] * cs - y[e] * sn : x[e] * cs + y[e] * sn;
                }
                qw[c] = pack8(x);
            }
            if (!col_ok) qw[c] = u32x4{0u, 0u, 0u, 0u};
            Qb[c] = as_bf16x8(qw[c]);
        }
    }

    // ---- per-lane LDS read offsets (bytes, within a stage), as in the prefill kernel
    const int swz = (l32 >> 1) & 7;
    int k_rd[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) k_rd[x] = l32 * (DQK * 2) + 16 * ((2 * x + g) ^ swz);
    const int qsel = lane >> 4, jsel = lane & 15;
    const int vrow = 4 * (qsel >> 1) + (jsel >> 2);
    int v_rd[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        v_rd[db] = STAGES * K_TILE + vrow * (DV * 2) +
                   16 * (4 * (db ^ ((jsel >> 2) & 3)) + 2 * (qsel & 1) + ((jsel & 3) >> 1)) +
                   8 * (jsel & 1);
        asm volatile("" : "+v"(v_rd[db]));
    }

    const float sink_l2 = (SINK && !SPLIT) ? a.sinks[h] * kLog2e : -INFINITY;
    float m_run = sink_l2;
    float l_run = (SINK && !SPLIT && g == 0) ? 1.0f : 0.0f;
    f32x16 O[DV / 32];
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) O[db] = f32x16{};
    const float sc = a.score_scale_log2;
    // column (token tc = t + shift in row coordinates) sees row j iff tc - j lies in [0, lim)
    const int tc = t + shift;
    const unsigned lim = (unsigned)max(0, min(WINDOW ? W : 0x7fffffff, tc - jmin + 1));
    const int tc_first = shift, tc_last = T - 1 + shift;   // over the valid tokens

    for (int tt = 0; tt < n_tiles; ++tt) {
        const int ST = tt & 1;
        wait_vmcnt<0>();
        block_sync_lds();   // tile tt in LDS for every wave; the other stage is free
        if (tt + 1 < n_tiles) {
            if (ST == 0) issue(tt + 1, std::integral_constant<int, 1>{});
            else issue(tt + 1, std::integral_constant<int, 0>{});
        }
        const int j0 = (kt_lo + tt) * BN;
        if (j0 > tc_last || (WINDOW && j0 + BN - 1 <= tc_first - W)) continue;
        const bool full = j0 >= jmin && j0 + BN - 1 <= tc_first && (!WINDOW || tc_last - j0 < W);
        const uint8_t* kst = smem + ST * K_TILE;
        const uint8_t* vst = smem + ST * V_TILE;   // + v_rd, which holds the V area's base

        f32x16 S0 = f32x16{}, S1 = f32x16{};
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const uint8_t* kp = kst + k_rd[c & 3] + (c >> 2) * 128;
            const bf16x8 A0 = *(const bf16x8*)(kp);
            const bf16x8 A1 = *(const bf16x8*)(kp + 32 * DQK * 2);
            S0 = mfma32x32x16(A0, Qb[c], S0);
            S1 = mfma32x32x16(A1, Qb[c], S1);
        }
        if (!full) {
            asm volatile("");
            const int d = tc - j0 - 4 * g;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = 8 * (i >> 2) + (i & 3);
                S0[i] = (unsigned)(d - off) < lim ? S0[i] : -INFINITY;
                S1[i] = (unsigned)(d - off - 32) < lim ? S1[i] : -INFINITY;
            }
        }
        float ma = fmaxf(S0[0], S1[0]), mb = fmaxf(S0[8], S1[8]);
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            ma = fmaxf(fmaxf(ma, S0[i]), S1[i]);
            mb = fmaxf(fmaxf(mb, S0[i + 8]), S1[i + 8]);
        }
        const float mx = max_lane_pair32(fmaxf(ma, mb)) * sc;
        const bool raise = mx > m_run + kRescaleLog2 || m_run == -INFINITY;
        const float m_new = raise ? fmaxf(m_run, mx) : m_run;
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        if (__any(raise)) {
            asm volatile("");
            const float alpha = fast_exp2(m_run - m_use);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DV / 32; ++db) O[db] *= alpha;
        }
        m_run = m_new;
        float ps0 = 0.0f, ps1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            S0[i] = fast_exp2(__builtin_fmaf(S0[i], sc, -m_use));
            S1[i] = fast_exp2(__builtin_fmaf(S1[i], sc, -m_use));
            ps0 += S0[i];
            ps1 += S1[i];
        }
        l_run += ps0 + ps1;
        bf16x8 Pb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x16& Sx = (c >> 1) ? S1 : S0;
            const int o = 8 * (c & 1);
            Pb[c] = as_bf16x8(u32x4{pack_bf16x2(Sx[o], Sx[o + 1]), pack_bf16x2(Sx[o + 2], Sx[o + 3]),
                                    pack_bf16x2(Sx[o + 4], Sx[o + 5]), pack_bf16x2(Sx[o + 6], Sx[o + 7])});
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int db = 0; db < DV / 32; ++db) {
                const uint8_t* vp = vst + v_rd[db] + 16 * c * (DV * 2);
                const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp));
                const bf16x4 v1 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * DV * 2));
                O[db] = mfma32x32x16(__builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7), Pb[c],
                                     O[db]);
            }
        }
    }

    // ---- epilogue: partial record (split) or out = v_scale * O / l (bf16)
    const float lt = sum_lane_pair32(l_run);
    if (!col_ok) return;
    if (SPLIT) {
        float* rec = a.partial + ((((int64_t)b * T + t) * Hq + h) * a.nsplit + s) * PSTRIDE;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int d = db * 32 + 8 * ii + 4 * g;
                *(f32x4*)(rec + d) = f32x4{O[db][4 * ii], O[db][4 * ii + 1], O[db][4 * ii + 2],
                                           O[db][4 * ii + 3]};
            }
        }
        if (g == 0) *(float2*)(rec + DV) = make_float2(m_run, lt);
    } else {
        const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
        uint16_t* orow = a.out + (((int64_t)b * T + t) * Hq + h) * DV;
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

template <int NW, bool WINDOW, bool SINK>
hipError_t launch_nw(const VerifyArgs& a, hipStream_t st) {
    const dim3 grid(a.nsplit, a.Hkv, a.B), block(NW * 64);
    if (a.nsplit > 1) verify_tiles_kernel<NW, WINDOW, SINK, true><<<grid, block, 0, st>>>(a);
    else verify_tiles_kernel<NW, WINDOW, SINK, false><<<grid, block, 0, st>>>(a);
    return hipGetLastError();
}

template <bool WINDOW, bool SINK>
hipError_t launch_ws(const VerifyArgs& a, int nw, hipStream_t st) {
    switch (nw) {
        case 1: return launch_nw<1, WINDOW, SINK>(a, st);
        case 2: return launch_nw<2, WINDOW, SINK>(a, st);
        case 4: return launch_nw<4, WINDOW, SINK>(a, st);
        default: return launch_nw<8, WINDOW, SINK>(a, st);
    }
}

}  // namespace

int verify_tile_waves(int G, int TP) {
    const int cols = G * TP;
    return cols <= 32 ? 1 : cols <= 64 ? 2 : cols <= 128 ? 4 : cols <= 256 ? 8 : 0;
}

hipError_t launch_verify_tiles_bf16(const VerifyArgs& a, bool window, bool sink, hipStream_t st) {
    if (a.B == 0 || a.T == 0) return hipSuccess;
    const int nw = verify_tile_waves(a.Hq / a.Hkv, a.TP);
    if (nw == 0 || a.TP < a.T || (a.TP & (a.TP - 1)) || a.chunk % BN || a.nsplit < 1 ||
        a.nsplit > decode_max_splits())
        return hipErrorInvalidConfiguration;
    if (window) return sink ? launch_ws<true, true>(a, nw, st) : launch_ws<true, false>(a, nw, st);
    return sink ? launch_ws<false, true>(a, nw, st) : launch_ws<false, false>(a, nw, st);
}

}  // namespace mimo
