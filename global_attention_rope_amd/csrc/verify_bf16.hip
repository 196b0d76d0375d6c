// verify_bf16.hip — a few new tokens per sequence (speculative or multi-token verification, short
// extends) against the key rows of their sequence, on gfx950 bf16 MFMA.
//
// Same layer as the prefill kernel (pages: "Add Xiaomi MiMo-V2", "Additional useful info";
// "add Xiaomi MiMo v2 (mimo_v2_flash)", "Architecture, verified against upstream" and
// "Implementation plan"), shaped for T <= 16 queries per sequence: the query columns of the
// S^T = K * Q^T products are (query head, token) pairs of one KV group — 16 heads x 4 tokens fill
// two 32-column waves — so every K/V tile is read from memory once per (sequence, KV head) and
// feeds all heads and tokens.  Up to 128 columns, each column wave is doubled: one wave takes the
// first 32 keys of every tile, its twin the last 32, each with a softmax state of its own, merged
// through LDS at the end — half the score registers per wave, so that two waves share a SIMD and
// cover each other's operand-read and product latencies.  The key rows are split across
// workgroups (split-K, at most 4096 rows each, the grid split-major); each split writes
// (O, max, sum) partials for the decode combine kernel, or the output when there is one.
// Tiles: 64 keys, staged through a 2-stage LDS ring by global_load_lds_dwordx4, XOR-swizzled as
// in the prefill kernel; per-column online softmax in the log2 domain with a lazily raised
// running maximum.  Global layers read a bf16 cache non-temporally: every row is streamed once,
// by one split, in whole 1-KiB spans per instruction.
// fp8 caches (global layers): the cached rows' e4m3 codes go memory -> registers (half the bytes
// of a bf16 tile, two tiles ahead), and each tile is widened into the bf16 LDS tile before its
// products as the codes' exact values; the two cache scales ride on the score scale and the output
// scale, and the new tokens' rows (at most 16, full precision, staged once per workgroup and copied
// into the tiles that hold them) have their scores and softmax weights divided by them instead.
// No pass over the whole cache.
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
// fp8: one bf16 tile and the new rows
constexpr int NEW_ROWS = 16;
constexpr int NEW_BYTES = NEW_ROWS * (DQK + DV) * 2;
constexpr int kFp8Depth = 2;                 // fp8: tiles of codes in flight (register sets)

// CW column waves of CWD query columns each, times KS key halves: with KS = 2 the waves of half
// kh take keys 32 kh .. 32 kh + 31 of every tile with a softmax state of their own, merged at the
// end.  CWD = 32: 32x32x16 products (a wave's scores are one 32-key x 32-column block per half);
// CWD = 16: 16x16x32 products on the operand layout of the 16-row sliding prefill kernel (two
// 16-key blocks x 16 columns per half), about half the registers and twice the waves.
template <int CWD, int CW, int KS, bool WINDOW, bool SINK, bool SPLIT, bool FP8>
__global__ __launch_bounds__(CW * KS * 64)
__attribute__((amdgpu_waves_per_eu(CWD == 16 ? 2 : KS))) void verify_tiles_kernel(const VerifyArgs a) {
    constexpr bool M16 = CWD == 16;
    constexpr int QC = M16 ? DQK / 32 : KCH;       // Q^T operand chunks of QSTEP dims
    constexpr int QSTEP = M16 ? 32 : 16;
    constexpr int NW = CW * KS;
    constexpr int KH_ROWS = BN / KS;               // keys of a tile per wave
    constexpr int NB = KH_ROWS / 32;               // 32-key score blocks per wave
    constexpr int K_DMA = K_TILE / 1024 / NW;      // 1-KiB DMA instructions per wave per tile
    constexpr int V_DMA = V_TILE / 1024 / NW;
    constexpr int NST = FP8 ? 1 : STAGES;          // bf16 tile stages
    constexpr int SMEM = FP8 ? K_TILE + V_TILE + NEW_BYTES : STAGES * (K_TILE + V_TILE);
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cw = wave % CW, kh = wave / CW;      // column wave, key half (scalar)
    const int l32 = lane & 31, g = lane >> 5;
    const int l16 = lane & 15, gq = lane >> 4;
    const int lc = M16 ? l16 : l32;                // this lane's column within its wave
    const int lsub = M16 ? gq : g;                 // its 8-dim slot of a Q^T chunk
    // (split-major grid: the dispatcher hands out every sequence's first split before any second
    //  one, so the last workgroups to start are the longest sequences' last splits)
    const int kvh = blockIdx.x, b = blockIdx.y, s = blockIdx.z;
    const int Hq = a.Hq, T = a.T, TP = a.TP;
    const int G = Hq / a.Hkv;

    // this lane's column: query head kvh * G + hl, token t
    const int col = cw * CWD + lc;
    const int hl = col / TP, t = col - hl * TP;
    const bool col_ok = hl < G && t < T;
    const int h = kvh * G + min(hl, G - 1);
    const int tq = min(t, T - 1);

    // the column's query row and the rotation partners of its rotated dims go out first: they do
    // not depend on the start position, which then comes by a scalar load that leaves them in flight
    const uint16_t* qrow = a.q + (((int64_t)b * T + tq) * Hq + h) * DQK;
    const int r = a.rope_dims, half = r >> 1;
    u32x4 qw[QC], pw[QC];
#pragma unroll
    for (int c = 0; c < QC; ++c) qw[c] = *(const u32x4*)(qrow + QSTEP * c + 8 * lsub);
#pragma unroll
    for (int c = 0; c < QC; ++c) {
        const int d0 = QSTEP * c + 8 * lsub;
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
        if (!SPLIT && col_ok && kh == 0) {
            uint16_t* orow = a.out + (((int64_t)b * T + t) * Hq + h) * DV;
            for (int d = 4 * lsub; d < DV; d += 4 * (64 / CWD))
                *(u32x2*)(orow + d) = u32x2{0u, 0u};
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
            if constexpr (WINDOW) dma16(src + k_off[i], kst + (wave * K_DMA + i) * 1024);
            else dma16_nt(src + k_off[i], kst + (wave * K_DMA + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < V_DMA; ++i) {
            const int j = min(max(j0 + v_row[i], jmin), nk - 1);
            const uint16_t* src = j < ring_w ? ring_v + (int64_t)((kpos0 + j) % ring_w) * DV
                                             : vslice + (int64_t)j * DV;
            if constexpr (WINDOW) dma16(src + v_off[i], vst + (wave * V_DMA + i) * 1024);
            else dma16_nt(src + v_off[i], vst + (wave * V_DMA + i) * 1024);
        }
    };
    if (!FP8 && n_tiles > 0) issue(0, std::integral_constant<int, 0>{});

    // fp8: the new tokens' rows (bf16, [T, 192] and [T, 128] of this sequence and KV head) into
    // LDS once; rows past T as zeros
    uint8_t* const newk = smem + K_TILE + V_TILE;
    uint8_t* const newv = newk + NEW_ROWS * DQK * 2;
    if constexpr (FP8) {
        constexpr int UNITS = NEW_ROWS * (DQK + DV) / 8;
        for (int u = tid; u < UNITS; u += NW * 64) {
            const bool key = u < NEW_ROWS * DQK / 8;
            const int uu = key ? u : u - NEW_ROWS * DQK / 8, cpr = key ? DQK / 8 : DV / 8;
            const int row = uu / cpr, c8 = uu - row * cpr;
            u32x4 w = u32x4{0u, 0u, 0u, 0u};
            if (row < T)
                w = key ? *(const u32x4*)(kslice + (int64_t)row * DQK + 8 * c8)
                        : *(const u32x4*)(vslice + (int64_t)row * DV + 8 * c8);
            *(u32x4*)((key ? newk + row * DQK * 2 : newv + row * DV * 2) + 16 * c8) = w;
        }
    }
    // fp8: the cached rows' codes of a tile go memory -> registers (units of 16 codes: K rows of
    // 12 units, then V rows of 8), DEPTH tiles ahead of the products; widening writes the bf16
    // tile: the codes' exact values for positions before the start, the staged new rows after it,
    // zeros past the last token.  Every load is issued unconditionally, with its code row clamped
    // in bounds (rows at or past the start, tiles past the last are loaded and not used): the
    // compiler then counts exactly which loads a widening has to wait for, instead of waiting for
    // all of them on the paths where a later load might have been skipped.
    constexpr int NT = NW * 64;
    constexpr int K_UNITS = BN * (DQK / 16), V_UNITS = BN * (DV / 16);
    constexpr int KU = (K_UNITS + NT - 1) / NT, VU = (V_UNITS + NT - 1) / NT;   // per thread
    // (a unit past the tile's occurs only where NT does not divide the units, 8 waves: it loads
    //  the last unit again and widens nothing)
    auto unit_ok = [&](int k) {
        if (k < KU) return K_UNITS % NT == 0 || tid + k * NT < K_UNITS;
        return V_UNITS % NT == 0 || tid + (k - KU) * NT < V_UNITS;
    };
    const int64_t code_row0 = ((int64_t)b * a.Hkv + kvh) * (FP8 ? a.code_cap : 1);
    auto load_codes = [&](u32x4 (&c)[KU + VU], int tt) {
        const int j0 = (kt_lo + tt) * BN, jlast = max(st - 1, 0);
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int u = min(tid + k * NT, K_UNITS - 1), row = u / (DQK / 16), c16 = u % (DQK / 16);
            c[k] = *(const u32x4*)(a.code_k + (code_row0 + min(j0 + row, jlast)) * DQK + 16 * c16);
        }
#pragma unroll
        for (int k = 0; k < VU; ++k) {
            const int u = min(tid + k * NT, V_UNITS - 1), row = u / (DV / 16), c16 = u % (DV / 16);
            c[KU + k] = *(const u32x4*)(a.code_v + (code_row0 + min(j0 + row, jlast)) * DV + 16 * c16);
        }
    };
    auto widen = [&](const u32x4 (&c)[KU + VU], int tt) {
        const int j0 = (kt_lo + tt) * BN;
#pragma unroll
        for (int k = 0; k < KU + VU; ++k) {
            if (!unit_ok(k)) continue;
            const bool key = k < KU;
            const int u = tid + (key ? k : k - KU) * NT;
            const int cpr = key ? DQK / 16 : DV / 16;
            const int row = u / cpr, c16 = u % cpr;
            const int j = j0 + row;
            u32x4 w[2];
            if (j < st) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    w[hh] = bf16x8_from_e4m3x8(u32x2{c[k][2 * hh], c[k][2 * hh + 1]});
            } else if (j < st + T) {
                const uint8_t* nr = key ? newk + (j - st) * DQK * 2 : newv + (j - st) * DV * 2;
                w[0] = *(const u32x4*)(nr + 32 * c16);
                w[1] = *(const u32x4*)(nr + 32 * c16 + 16);
            } else {
                w[0] = w[1] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c8 = 2 * c16 + hh;
                uint8_t* dst = key ? smem + row * (DQK * 2) + 16 * (c8 ^ ((row >> 1) & 7))
                                   : smem + K_TILE + row * (DV * 2) + 16 * (c8 ^ ((row & 3) << 2));
                *(u32x4*)dst = w[hh];
            }
        }
    };

    // ---- Q^T operands of this column, rotated at the token's position, in registers
    bf16x8 Qb[QC];
    {
        const int32_t pos = st + tq;
#pragma unroll
        for (int c = 0; c < QC; ++c) {
            const int d0 = QSTEP * c + 8 * lsub;
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

    // ---- per-lane LDS read offsets (bytes, within a stage), as in the prefill kernels
    int k_rd[M16 ? QC : 4], v_rd[M16 ? DV / 16 : 4];
    if constexpr (M16) {
        // K: key l16 of a 16-key block, chunk 4c + gq; V^T: rows 4gq + l16 / 4 (and + 16), dims
        // 16db + 4(l16 % 4)
#pragma unroll
        for (int c = 0; c < QC; ++c)
            k_rd[c] = l16 * (DQK * 2) + 16 * ((4 * c + gq) ^ ((l16 >> 1) & 7));
        const int vrow = 4 * gq + (l16 >> 2);
#pragma unroll
        for (int db = 0; db < DV / 16; ++db) {
            const int byte = (db * 16 + 4 * (l16 & 3)) * 2;
            v_rd[db] = NST * K_TILE + vrow * (DV * 2) + 16 * ((byte >> 4) ^ ((vrow & 3) << 2)) +
                       (byte & 15);
            asm volatile("" : "+v"(v_rd[db]));
        }
    } else {
        const int swz = (l32 >> 1) & 7;
#pragma unroll
        for (int x = 0; x < 4; ++x) k_rd[x] = l32 * (DQK * 2) + 16 * ((2 * x + g) ^ swz);
        const int qsel = lane >> 4, jsel = lane & 15;
        const int vrow = 4 * (qsel >> 1) + (jsel >> 2);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            v_rd[db] = NST * K_TILE + vrow * (DV * 2) +
                       16 * (4 * (db ^ ((jsel >> 2) & 3)) + 2 * (qsel & 1) + ((jsel & 3) >> 1)) +
                       8 * (jsel & 1);
            asm volatile("" : "+v"(v_rd[db]));
        }
    }

    // (the sink joins the first key half's state)
    const float sink_l2 = (SINK && !SPLIT && kh == 0) ? a.sinks[h] * kLog2e : -INFINITY;
    float m_run = sink_l2;
    float l_run = (SINK && !SPLIT && kh == 0 && lsub == 0) ? 1.0f : 0.0f;
    f32x16 O[DV / 32];     // CWD = 32: lane (column l32, half g) holds dims 32db + 8(i / 4) + 4g + i % 4
    f32x4 O16[DV / 16];    // CWD = 16: lane (column l16, group gq) holds dims 16db + 4gq + i
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) O[db] = f32x16{};
#pragma unroll
    for (int db = 0; db < DV / 16; ++db) O16[db] = f32x4{};
    const float sc = a.score_scale_log2;
    // column (token tc = t + shift in row coordinates) sees row j iff tc - j lies in [0, lim)
    const int tc = t + shift;
    const unsigned lim = (unsigned)max(0, min(WINDOW ? W : 0x7fffffff, tc - jmin + 1));
    const int tc_first = shift, tc_last = T - 1 + shift;   // over the valid tokens

    // products of this wave's keys of tile tt, in bf16 stage ST of the LDS ring (the swizzles
    // repeat every 16 rows, so a key half starts on the same pattern)
    auto tile_products = [&](int tt, int ST) {
        const int j0 = (kt_lo + tt) * BN + kh * KH_ROWS;   // this wave's first key row
        if (j0 > tc_last || (WINDOW && j0 + KH_ROWS - 1 <= tc_first - W)) return;
        const bool full =
            j0 >= jmin && j0 + KH_ROWS - 1 <= tc_first && (!WINDOW || tc_last - j0 < W);
        const uint8_t* kst = smem + ST * K_TILE + kh * KH_ROWS * DQK * 2;
        // (+ v_rd, which holds the V area's base)
        const uint8_t* vst = smem + ST * V_TILE + kh * KH_ROWS * DV * 2;

        if constexpr (M16) {
            // S^T blocks kb (keys j0 + 16kb + 4gq + i against column l16)
            f32x4 Sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4 acc = f32x4{};
#pragma unroll
                for (int c = 0; c < QC; ++c)
                    acc = mfma16x16x32(*(const bf16x8*)(kst + k_rd[c] + kb * 16 * (DQK * 2)), Qb[c], acc);
                Sacc[kb] = acc;
            }
            const int rr = j0 + 4 * gq - st;   // (fp8: key offsets at or past the start are new rows)
            if constexpr (FP8) {
                if (j0 + KH_ROWS > st) {
                    asm volatile("");
                    const float ik = 1.0f / a.code_k_scale;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) Sacc[kb][i] *= rr + 16 * kb + i >= 0 ? ik : 1.0f;
                }
            }
            if (!full) {
                asm volatile("");
                const int d = tc - j0 - 4 * gq;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Sacc[kb][i] = (unsigned)(d - 16 * kb - i) < lim ? Sacc[kb][i] : -INFINITY;
            }
            float mx = fmaxf(fmaxf(fmaxf(Sacc[0][0], Sacc[0][1]), fmaxf(Sacc[0][2], Sacc[0][3])),
                             fmaxf(fmaxf(Sacc[1][0], Sacc[1][1]), fmaxf(Sacc[1][2], Sacc[1][3])));
            mx = max_lane_pair32(max_lane_pair16(mx)) * sc;
            const bool raise = mx > m_run + kRescaleLog2 || m_run == -INFINITY;
            const float m_new = raise ? fmaxf(m_run, mx) : m_run;
            const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
            if (__any(raise)) {
                asm volatile("");
                const float alpha = fast_exp2(m_run - m_use);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DV / 16; ++db) O16[db] *= alpha;
            }
            m_run = m_new;
            float ps = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Sacc[kb][i] = fast_exp2(__builtin_fmaf(Sacc[kb][i], sc, -m_use));
                    ps += Sacc[kb][i];
                }
            l_run += ps;
            if constexpr (FP8) {
                if (j0 + KH_ROWS > st) {
                    asm volatile("");
                    const float iv = 1.0f / a.code_v_scale;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) Sacc[kb][i] *= rr + 16 * kb + i >= 0 ? iv : 1.0f;
                }
            }
            // P^T: k-slot i of group gq is key 4gq + i (i < 4) or 16 + 4gq + (i - 4), as the
            // transposed V reads below hand out V's rows
            const bf16x8 Pb = as_bf16x8(u32x4{pack_bf16x2(Sacc[0][0], Sacc[0][1]),
                                              pack_bf16x2(Sacc[0][2], Sacc[0][3]),
                                              pack_bf16x2(Sacc[1][0], Sacc[1][1]),
                                              pack_bf16x2(Sacc[1][2], Sacc[1][3])});
#pragma unroll
            for (int db = 0; db < DV / 16; ++db) {
                const uint8_t* vp = vst + v_rd[db];
                const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp));
                const bf16x4 v1 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 16 * DV * 2));
                O16[db] = mfma16x16x32(__builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7), Pb,
                                       O16[db]);
            }
            return;
        }

        f32x16 Sb[NB];
#pragma unroll
        for (int x = 0; x < NB; ++x) Sb[x] = f32x16{};
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const uint8_t* kp = kst + k_rd[c & 3] + (c >> 2) * 128;
#pragma unroll
            for (int x = 0; x < NB; ++x)
                Sb[x] = mfma32x32x16(*(const bf16x8*)(kp + x * 32 * DQK * 2), Qb[c], Sb[x]);
        }
        if constexpr (FP8) {
            // the score scale carries the key cache's scale: the new tokens' rows (positions at
            // or past the start, full-precision keys) are divided by it
            if (j0 + KH_ROWS > st) {
                asm volatile("");
                const float ik = 1.0f / a.code_k_scale;
                const int rr = j0 + 4 * g - st;
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int off = 8 * (i >> 2) + (i & 3) + 32 * x;
                        Sb[x][i] *= rr + off >= 0 ? ik : 1.0f;
                    }
            }
        }
        if (!full) {
            asm volatile("");
            const int d = tc - j0 - 4 * g;
#pragma unroll
            for (int x = 0; x < NB; ++x)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int off = 8 * (i >> 2) + (i & 3) + 32 * x;
                    Sb[x][i] = (unsigned)(d - off) < lim ? Sb[x][i] : -INFINITY;
                }
        }
        float ma = Sb[0][0], mb = Sb[0][8];
#pragma unroll
        for (int x = 0; x < NB; ++x)
#pragma unroll
            for (int i = x == 0 ? 1 : 0; i < 8; ++i) {
                ma = fmaxf(ma, Sb[x][i]);
                mb = fmaxf(mb, Sb[x][i + 8]);
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
        float ps[NB];
#pragma unroll
        for (int x = 0; x < NB; ++x) {
            ps[x] = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                Sb[x][i] = fast_exp2(__builtin_fmaf(Sb[x][i], sc, -m_use));
                ps[x] += Sb[x][i];
            }
        }
#pragma unroll
        for (int x = 0; x < NB; ++x) l_run += ps[x];
        if constexpr (FP8) {
            // the output scale carries the value cache's scale: the new tokens' weights are
            // divided by it (after the sum, which takes them as they are)
            if (j0 + KH_ROWS > st) {
                asm volatile("");
                const float iv = 1.0f / a.code_v_scale;
                const int rr = j0 + 4 * g - st;
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int off = 8 * (i >> 2) + (i & 3) + 32 * x;
                        Sb[x][i] *= rr + off >= 0 ? iv : 1.0f;
                    }
            }
        }
        bf16x8 Pb[2 * NB];
#pragma unroll
        for (int c = 0; c < 2 * NB; ++c) {
            const f32x16& Sx = Sb[c >> 1];
            const int o = 8 * (c & 1);
            Pb[c] = as_bf16x8(u32x4{pack_bf16x2(Sx[o], Sx[o + 1]), pack_bf16x2(Sx[o + 2], Sx[o + 3]),
                                    pack_bf16x2(Sx[o + 4], Sx[o + 5]), pack_bf16x2(Sx[o + 6], Sx[o + 7])});
        }
#pragma unroll
        for (int c = 0; c < 2 * NB; ++c) {
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
    };

    if constexpr (FP8) {
        // DEPTH tiles of codes in flight (one where the registers would not hold more: a single
        // wave, or 8 waves two to a SIMD); register set d holds tiles d, d + DEPTH, ...
        constexpr int DEPTH = (NW <= 2 || (NW == 8 && KS == 1)) ? 1 : kFp8Depth;
        u32x4 cs[DEPTH][KU + VU];
        // Round r runs DEPTH steps: step d widens tile DEPTH * r + d from register set d (a
        // uniform branch skips it in round -1, which only loads) and loads the tile DEPTH later
        // into the same set.  Every round runs all DEPTH steps, past the last tile too, and the
        // first loads come from the same instructions as the later ones, so that every path into
        // the loop head has issued the sets' loads in the same order.
        auto step = [&](u32x4 (&c)[KU + VU], int tt) {
            if (tt >= 0) {
                block_sync_lds();   // the previous tile's products are done with the bf16 tile
                widen(c, tt);       // (waits for this tile's codes; later tiles' stay in flight)
                block_sync_lds();
            }
            load_codes(c, min(tt + DEPTH, n_tiles - 1));   // (past the last: that tile again)
            if (tt >= 0 && tt < n_tiles) tile_products(tt, 0);
        };
        if (n_tiles > 0) {
            for (int tt = -DEPTH; tt < n_tiles; tt += DEPTH) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) step(cs[d], tt + d);
            }
        }
    } else {
        for (int tt = 0; tt < n_tiles; ++tt) {
            const int ST = tt & 1;
            wait_vmcnt<0>();
            block_sync_lds();   // tile tt in LDS for every wave; the other stage is free
            if (tt + 1 < n_tiles) {
                if (ST == 0) issue(tt + 1, std::integral_constant<int, 1>{});
                else issue(tt + 1, std::integral_constant<int, 0>{});
            }
            tile_products(tt, ST);
        }
    }

    // ---- the key halves' states merged into the first half's waves, through LDS in two rounds
    //      of two O blocks (lane-for-lane: the partner lane holds the same column and dims)
    if constexpr (KS == 2) {
        constexpr int XS = 36;   // floats per lane and round: 32 of O, then m and l
        constexpr int ROUNDS = M16 ? 1 : 2;
        float* const xch = (float*)smem + (cw * 64 + lane) * XS;
        float a0 = 1.0f, a1 = 0.0f;
        // the 32 floats of O that round rd moves: f32x4 number q4 (0..7)
        auto get4 = [&](int rd, int q4) -> f32x4 {
            if constexpr (M16) {
                return O16[q4];
            } else {
                const f32x16& o = O[2 * rd + (q4 >> 2)];
                const int e = 4 * (q4 & 3);
                return f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
            }
        };
        auto set4 = [&](int rd, int q4, const f32x4& v) {
            if constexpr (M16) {
                O16[q4] = v;
            } else {
                f32x16& o = O[2 * rd + (q4 >> 2)];
                const int e = 4 * (q4 & 3);
                o[e] = v[0];
                o[e + 1] = v[1];
                o[e + 2] = v[2];
                o[e + 3] = v[3];
            }
        };
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            block_sync_lds();   // every wave done with the tiles (round 1: with round 0's data)
            if (kh == 1) {
#pragma unroll
                for (int q4 = 0; q4 < 8; ++q4) *(f32x4*)(xch + 4 * q4) = get4(rd, q4);
                if (rd == 0) *(float2*)(xch + 32) = make_float2(m_run, l_run);
            }
            block_sync_lds();
            if (kh == 0) {
                if (rd == 0) {
                    const float2 ml = *(const float2*)(xch + 32);
                    const float m = fmaxf(m_run, ml.x);
                    const float ref = m == -INFINITY ? 0.0f : m;
                    a0 = fast_exp2(m_run - ref);
                    a1 = fast_exp2(ml.x - ref);
                    l_run = l_run * a0 + ml.y * a1;
                    m_run = m;
                }
#pragma unroll
                for (int q4 = 0; q4 < 8; ++q4) {
                    const f32x4 o1 = *(const f32x4*)(xch + 4 * q4);
                    const f32x4 o0 = get4(rd, q4);
                    set4(rd, q4, f32x4{o0[0] * a0 + o1[0] * a1, o0[1] * a0 + o1[1] * a1,
                                       o0[2] * a0 + o1[2] * a1, o0[3] * a0 + o1[3] * a1});
                }
            }
        }
    }

    // ---- epilogue (first key half): partial record (split) or out = v_scale * O / l (bf16)
    const float lt = M16 ? sum_lane_pair32(sum_lane_pair16(l_run)) : sum_lane_pair32(l_run);
    if (!col_ok || kh != 0) return;
    if constexpr (M16) {
        if (SPLIT) {
            float* rec = a.partial + ((((int64_t)b * T + t) * Hq + h) * a.nsplit + s) * PSTRIDE;
#pragma unroll
            for (int db = 0; db < DV / 16; ++db) *(f32x4*)(rec + 16 * db + 4 * gq) = O16[db];
            if (gq == 0) *(float2*)(rec + DV) = make_float2(m_run, lt);
        } else {
            const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
            uint16_t* orow = a.out + (((int64_t)b * T + t) * Hq + h) * DV;
#pragma unroll
            for (int db = 0; db < DV / 16; ++db)
                *(u32x2*)(orow + 16 * db + 4 * gq) =
                    u32x2{pack_bf16x2(O16[db][0] * inv, O16[db][1] * inv),
                          pack_bf16x2(O16[db][2] * inv, O16[db][3] * inv)};
        }
        return;
    }
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

template <int CWD, int CW, bool WINDOW, bool SINK>
hipError_t launch_cw(const VerifyArgs& a, hipStream_t st) {
    // (32-column waves: 8 column waves take whole tiles, 1024 threads at most)
    constexpr int KS = (CWD == 16 || CW <= 4) ? 2 : 1;
    const dim3 grid(a.Hkv, a.B, a.nsplit), block(CW * KS * 64);
    if constexpr (!WINDOW) {
        if (a.code_k) {
            if (a.nsplit > 1)
                verify_tiles_kernel<CWD, CW, KS, false, SINK, true, true><<<grid, block, 0, st>>>(a);
            else
                verify_tiles_kernel<CWD, CW, KS, false, SINK, false, true><<<grid, block, 0, st>>>(a);
            return hipGetLastError();
        }
    }
    if (a.nsplit > 1)
        verify_tiles_kernel<CWD, CW, KS, WINDOW, SINK, true, false><<<grid, block, 0, st>>>(a);
    else
        verify_tiles_kernel<CWD, CW, KS, WINDOW, SINK, false, false><<<grid, block, 0, st>>>(a);
    return hipGetLastError();
}

template <bool WINDOW, bool SINK>
hipError_t launch_ws(const VerifyArgs& a, int nw, hipStream_t st) {
    switch (nw) {
        // up to 16 columns one twinned 16-column wave pair (B64, one token per sequence after
        // 1024-32768 fp8 positions: 0.50 ms against 0.73 on 32-column waves; at 64 columns the
        // 16-column layout was slower over fp8 caches, its 160 registers leaving one workgroup
        // per CU, and no faster over bf16 ones)
        case 1: return (a.Hq / a.Hkv) * a.TP <= 16 ? launch_cw<16, 1, WINDOW, SINK>(a, st)
                                                   : launch_cw<32, 1, WINDOW, SINK>(a, st);
        case 2: return launch_cw<32, 2, WINDOW, SINK>(a, st);
        case 4: return launch_cw<32, 4, WINDOW, SINK>(a, st);
        default: return launch_cw<32, 8, WINDOW, SINK>(a, st);
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
    // codes read in place: global layers, key row = position, at most NEW_ROWS new tokens
    if (a.code_k && (window || a.ring_k || a.kpos_rel || a.kpos_off || a.T > NEW_ROWS || !a.code_v))
        return hipErrorInvalidConfiguration;
    if (window) return sink ? launch_ws<true, true>(a, nw, st) : launch_ws<true, false>(a, nw, st);
    return sink ? launch_ws<false, true>(a, nw, st) : launch_ws<false, false>(a, nw, st);
}

}  // namespace mimo
