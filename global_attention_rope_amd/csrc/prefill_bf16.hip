// prefill_bf16.hip — prefill of the hybrid attention layer (global and sliding-window kinds) on
// gfx950 bf16 MFMA.
//
// Computes (pages: "Add Xiaomi MiMo-V2", section "Additional useful info"; "add Xiaomi MiMo v2
// (mimo_v2_flash)", section "Architecture, verified against upstream"):
//   out[b,i,h,:] = v_scale * sum_{j visible} e^{z_ij} v_j / (e^{s_h} + sum e^{z_ij}),
//   z_ij = tau * <rot(q_i), k'_j>, k'_j the keys already rotated by the key-rotation pass,
//   visible: p_j <= p_i (global) and additionally p_i - p_j < window (sliding), GQA head
//   h -> KV head h / (Hq / Hkv), optional sink s_h (sliding layers in the model).
//
// Shape of the computation (qk head dim 192, v head dim 128):
//   * prefill_kernel: each wave owns 32 query rows of one query head and keeps their rotated Q^T
//     (bf16) in registers; global layers: 8 waves on 8 consecutive row blocks of one head, one
//     workgroup per CU; sliding layers whose GQA group is not a multiple of 4: 4 waves, two
//     workgroups per CU;
//   * prefill_sw16_kernel (sliding layers, GQA group a multiple of 4): 4 waves take 4 heads of one
//     KV group over the same 16 rows on 16x16x32 products and 32-key tiles, so each K/V tile feeds
//     4 heads and four workgroups share a CU (details at the kernel);
//   * K (64 x 192) and V (64 x 128) tiles stream through a 3-stage (global) or 2-stage (sliding)
//     LDS ring filled by global_load_lds_dwordx4 (memory -> LDS without registers) one or two
//     tiles ahead of the one being computed; one barrier per tile;
//   * LDS layouts are unpadded and XOR-swizzled at 16-byte granularity so that the MFMA operand
//     reads are conflict-free: K chunk c of row r sits at c ^ ((r >> 1) & 7); V chunk c of row r at
//     c ^ ((r & 3) << 2);
//   * S^T = K * Q^T with v_mfma_f32_32x32x16_bf16 (each lane owns one query column); Q carries the
//     score scale tau * log2(e) and the accumulators start at minus the running maximum, so the
//     products hand the softmax its exponents directly (one v_exp_f32 per score, no scale or
//     subtraction); online softmax in the log2 domain with a lazily raised running maximum (moved
//     only when a tile exceeds it by more than 2^8, so the O rescale is rare; the result is exact
//     because numerator and denominator share the reference); O^T += V^T * P^T with V^T read by
//     ds_read_b64_tr_b16;
//   * the wave index is made scalar so tile skipping and the band-edge masking are uniform
//     branches; sliding-window workgroups only stream the tiles of their band, and each wave only
//     computes the tiles its own rows can see;
//   * global layers: workgroups are ordered heavy-first; the dispatcher's round-robin over the 8
//     XCDs is undone so that each XCD takes whole (sequence, KV head) pairs where their count is a
//     multiple of 8 (else 8 heads of a KV head per row block), and that K/V stays in its L2;
//     sliding layers: each XCD walks consecutive row blocks of a few (sequence, head unit) pairs,
//     so the sliding K/V band is fetched from memory about once.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mimo {
namespace {

constexpr int DQK = 192;
constexpr int DV = 128;
constexpr int BN = 64;                       // keys per tile
constexpr int QPW = 32;                      // query rows per wave
constexpr int K_TILE = BN * DQK * 2;         // bytes
constexpr int V_TILE = BN * DV * 2;
constexpr int KCH = DQK / 16;

// Launch shapes.  Global layers: 8 waves (256 rows) and a 3-stage ring, one workgroup per CU.
// Sliding layers see only ~3 tiles per wave, so pipeline fill and the Q prologue dominate a
// workgroup's life: 4 waves (128 rows) and a 2-stage ring let two workgroups share a CU and hide
// each other's latency.
constexpr int GA_WAVES = 8, GA_STAGES = 3;
constexpr int SW_WAVES = 4, SW_STAGES = 2;
constexpr float kRescaleLog2 = 8.0f;         // raise the running max only beyond 2^8
// a lane's 32 weights of a tile summing past this (or overflowing) move its row's reference; below
// it every weight is at most 2^16, so O (f32) holds any row length a tile count reaches
constexpr float kSumLimit = 65536.0f;


// Rotate the pairs (lo[t], hi[t]) at pos and return the chunk this lane keeps (lo when `lower`),
// times `scale`, rounded once to bf16.
__device__ __forceinline__ u32x4 rotate_pair8_kernarg(const u32x4& lo, const u32x4& hi, bool lower,
                                                      int32_t pos, const double* om, float scale) {
    float x[8], y[8];
    unpack8(lo, x);
    unpack8(hi, y);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        float c, s;
        rope_cos_sin_rev(pos, om[t], c, s);
        const float xl = x[t], xh = y[t];
        x[t] = (lower ? xl * c - xh * s : xh * c + xl * s) * scale;
    }
    return pack8(x);
}

// 8 bf16 times `scale`, rounded once to bf16.
__device__ __forceinline__ u32x4 scale8(const u32x4& w, float scale) {
    float x[8];
    unpack8(w, x);
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] *= scale;
    return pack8(x);
}

// A workgroup covers NW consecutive 32-row blocks of one query head.
template <int NW, int STAGES, bool WINDOW, bool SINK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    const PrefillArgs a) {
    constexpr int BM = NW * QPW;                   // query rows per workgroup
    constexpr int K_DMA = K_TILE / 1024 / NW;      // 1-KiB DMA instructions per wave per tile
    constexpr int V_DMA = V_TILE / 1024 / NW;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * (K_TILE + V_TILE)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int S = a.S, Hq = a.Hq;
    const int nqblk = (S + BM - 1) / BM;
    const int hunits = Hq;                         // heads per (row block, sequence)
    const int total = a.B * hunits * nqblk;

    // ---- work item (XCD-aware order; heavy-first on global layers)
    const int id = blockIdx.x;
    int w = id;
    const int pairs = a.B * hunits;                // (sequence, head unit) pairs
    if (WINDOW && pairs % 8 == 0) {
        // sliding layers: workgroup ids go round-robin to the 8 XCDs; each XCD walks the row
        // blocks of its own pairs in order (its pairs interleaved), so the K/V band, which
        // consecutive row blocks share, stays in that XCD's L2 as it slides
        const int P = pairs / 8, xcd = id & 7, k = id >> 3;
        w = (k / P) * pairs + xcd * P + k % P;
    } else if (!WINDOW) {
        const int xcd = id & 7, slot = id >> 3;
        const int P = a.B * a.Hkv, G = Hq / a.Hkv;
        if (P % 8 == 0) {
            // each XCD takes whole (sequence, KV head) pairs (x, x + 8, ...), all their heads'
            // row blocks heaviest first: its L2 holds the K/V of those pairs only (B2 S16384,
            // 4 KV heads: 39% fewer bytes fetched from beyond the L2 than with a pair per 2 XCDs)
            const int per = Hq * a.B / 8;               // items per row block on this XCD
            const int qr = slot / per, rem = slot - qr * per;
            const int pair = xcd + 8 * (rem / G), hl = rem % G;
            w = qr * (Hq * a.B) + (pair / a.Hkv) * Hq + (pair % a.Hkv) * G + hl;
        } else {
            // XCD x takes heads 8x..8x+7 of each group of 64 work items (heads of one row block)
            const int grp = slot >> 3;
            if ((grp + 1) * 64 <= total) w = grp * 64 + xcd * 8 + (slot & 7);
        }
    }
    const int hu = w % hunits;
    const int b = (w / hunits) % a.B;
    const int qrank = w / (hunits * a.B);
    const int qblk = WINDOW ? qrank : nqblk - 1 - qrank;   // global: heaviest blocks first
    const int h = hu;
    const int kvh = hu / (Hq / a.Hkv);
    const int r = a.rope_dims, half = r >> 1;
    // (the start position comes by a scalar load that waits for nothing but itself, so the vector
    //  loads issued before it stay in flight)
    int32_t p0 = 0;

    // Key rows: row j sits at position kpos0 + j.  Query row i (position p0 + i) thus meets key
    // row i + shift at its own position; rows below jmin (negative positions) hold no token, and
    // the last query row reaches key row nk - 1.  A sequence outside the accepted start range
    // streams no tiles and gets a zero output.  When the keys are the sequence's own rows and
    // every start is accepted, none of this depends on the start position (start_pos >= 0), so
    // the tile loads below go out before it arrives.
    bool seq_ok;
    int shift, jmin;
    const bool own_rows = a.max_start < 0 && a.kpos_rel && a.kpos_off >= 0;
    if (own_rows) {
        seq_ok = true;
        shift = -a.kpos_off;
        jmin = 0;
    } else {
        p0 = load_scalar_i32(a.start_pos + b);
        seq_ok = a.max_start < 0 || (unsigned)p0 <= (unsigned)a.max_start;
        const int32_t kpos0 = (a.kpos_rel ? (seq_ok ? p0 : 0) : 0) + a.kpos_off;
        shift = (seq_ok ? p0 : 0) - kpos0;
        jmin = max(0, -kpos0);
    }
    const int nk = S + shift;

    const int W = a.window;
    const int q_first = qblk * BM + wave * QPW;   // this wave's first row (scalar)
    const int q_last = min(q_first + QPW, S) - 1;                 // its last valid row
    const int blk_first = qblk * BM;
    const int blk_last = min(blk_first + BM, S) - 1;
    const int kt_lo = max(jmin, WINDOW ? blk_first + shift - W + 1 : 0) / BN;
    const int n_tiles = seq_ok ? (blk_last + shift) / BN + 1 - kt_lo : 0;

    // ---- DMA source mapping: LDS 16-byte slot P of this wave's instruction i holds
    //      K row P / 24, logical chunk (P % 24) ^ swizzle; V row P / 16, chunk (P % 16) ^ swizzle.
    //      A tile whose rows all lie in [jmin, nk) is read from a scalar base (its first row) plus
    //      per-lane byte offsets that are the same for every tile; a tile that reaches past those
    //      rows has them clamped into the range (they are masked anyway, and clamping keeps
    //      unwritten rows out of the products), its addresses formed on the spot.
    const uint16_t* kslice = a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
    const uint16_t* vslice = a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;
    const int64_t v_sj = a.v_sj;
    auto k_slot = [&](int i, int ln, int& row, int& col) __attribute__((always_inline)) {
        const int P = (wave * K_DMA + i) * 64 + ln;
        row = P / (DQK / 8);
        col = ((P % (DQK / 8)) ^ ((row >> 1) & 7)) * 8;
    };
    auto v_slot = [&](int i, int ln, int& row, int& col) __attribute__((always_inline)) {
        const int P = (wave * V_DMA + i) * 64 + ln;
        row = P / (DV / 8);
        col = ((P % (DV / 8)) ^ ((row & 3) << 2)) * 8;
    };
    uint32_t k_lo[K_DMA], v_lo[V_DMA];   // byte offsets within a tile
#pragma unroll
    for (int i = 0; i < K_DMA; ++i) {
        int row, col;
        k_slot(i, lane, row, col);
        k_lo[i] = (uint32_t)(row * DQK + col) * 2u;
    }
#pragma unroll
    for (int i = 0; i < V_DMA; ++i) {
        int row, col;
        v_slot(i, lane, row, col);
        v_lo[i] = (uint32_t)((int64_t)row * v_sj + col) * 2u;
    }
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8_t*)smem;
    auto issue = [&](int t, auto stage_c) {
        constexpr int ST = decltype(stage_c)::value;
        const int j0 = (kt_lo + t) * BN;
        const uint32_t kst = lds0 + ST * K_TILE;
        const uint32_t vst = lds0 + STAGES * K_TILE + ST * V_TILE;
        if (j0 >= jmin && j0 + BN <= nk) {
            const uint16_t* kb = kslice + (int64_t)j0 * DQK;
            const uint16_t* vb = vslice + (int64_t)j0 * v_sj;
#pragma unroll
            for (int i = 0; i < K_DMA; ++i) dma16_sbase(kb, k_lo[i], kst + (wave * K_DMA + i) * 1024);
#pragma unroll
            for (int i = 0; i < V_DMA; ++i) dma16_sbase(vb, v_lo[i], vst + (wave * V_DMA + i) * 1024);
        } else {
            int ln = lane;
            asm volatile("" : "+v"(ln));   // (kept here, not hoisted out of the tile loop)
#pragma unroll
            for (int i = 0; i < K_DMA; ++i) {
                int row, col;
                k_slot(i, ln, row, col);
                const int j = min(max(j0 + row, jmin), nk - 1);
                dma16(kslice + (int64_t)j * DQK + col, kst + (wave * K_DMA + i) * 1024);
            }
#pragma unroll
            for (int i = 0; i < V_DMA; ++i) {
                int row, col;
                v_slot(i, ln, row, col);
                const int j = min(max(j0 + row, jmin), nk - 1);
                dma16(vslice + (int64_t)j * v_sj + col, vst + (wave * V_DMA + i) * 1024);
            }
        }
    };
    if (n_tiles > 0) issue(0, std::integral_constant<int, 0>{});
    if (STAGES == 3 && n_tiles > 1) issue(1, std::integral_constant<int, 1 % STAGES>{});

    // ---- Q^T operands, rotated and scaled by tau * log2(e) (so that the products give the scores
    //      in the log2 domain), rounded once to bf16, in registers
    const float sc = a.score_scale_log2;
    bf16x8 Qb[KCH];
    {
        const int qi = q_first + l32;
        const bool qok = qi < S;
        const uint16_t* qrow = a.q + (((int64_t)b * S + (qok ? qi : S - 1)) * Hq + h) * DQK;
        u32x4 qw[KCH];
#pragma unroll
        for (int c = 0; c < KCH; ++c) qw[c] = *(const u32x4*)(qrow + 16 * c + 8 * g);
        if (own_rows) p0 = load_scalar_i32(a.start_pos + b);
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int d0 = 16 * c + 8 * g;
            if (d0 < r) {
                const bool lower = d0 < half;
                const u32x4 lo = lower ? qw[c] : *(const u32x4*)(qrow + d0 - half);
                const u32x4 hi = lower ? *(const u32x4*)(qrow + d0 + half) : qw[c];
                qw[c] = rotate_pair8_kernarg(lo, hi, lower, p0 + qi,
                                             a.omega_rev + (lower ? d0 : d0 - half), sc);
            } else {
                qw[c] = scale8(qw[c], sc);
            }
            if (!qok) qw[c] = u32x4{0u, 0u, 0u, 0u};
            Qb[c] = as_bf16x8(qw[c]);
        }
    }

    // ---- per-lane LDS read offsets (bytes, within a stage)
    const int swz = (l32 >> 1) & 7;
    int k_rd[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) k_rd[x] = l32 * (DQK * 2) + 16 * ((2 * x + g) ^ swz);
    const int qsel = lane >> 4, jsel = lane & 15;
    const int vrow = 4 * (qsel >> 1) + (jsel >> 2);
    // (V stages start past 64 KiB on global layers, beyond the 16-bit immediate offset of LDS
    //  reads: the V stage base is folded into these registers, hidden from the compiler so that
    //  it does not split it back out into a per-read address add)
    int v_rd[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        v_rd[db] = STAGES * K_TILE + vrow * (DV * 2) +
                   16 * (4 * (db ^ ((jsel >> 2) & 3)) + 2 * (qsel & 1) + ((jsel & 3) >> 1)) +
                   8 * (jsel & 1);
        asm volatile("" : "+v"(v_rd[db]));
    }

    const float sink_l2 = SINK ? a.sinks[h] * kLog2e : -INFINITY;
    float m_run = SINK ? sink_l2 : -INFINITY;
    float l_run = (SINK && g == 0) ? 1.0f : 0.0f;
    f32x16 O[DV / 32];
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) O[db] = f32x16{};
    // The products return sc * z - m_ref: the score accumulators start from -m_ref, kept as a
    // 16-register copy (negm), where m_ref is the running maximum once one is known (the sink when
    // there is one, else 0 until the first visible key).
    f32x16 negm;
    {
        const float m0 = SINK ? sink_l2 : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = -m0;
    }
    const int q_l = q_first + l32;
    // row q_l sees key row j iff q_l + shift - j lies in [0, lim): the window (sliding) and the
    // first key row holding a token both bound it
    const unsigned lim = (unsigned)max(0, min(WINDOW ? W : 0x7fffffff, q_l + shift - jmin + 1));

    auto compute = [&](int t, auto stage_c) {
        constexpr int ST = decltype(stage_c)::value;
        const int j0 = (kt_lo + t) * BN;
        // nothing visible for this wave (uniform branch)
        if (q_first > q_last || j0 > q_last + shift || (WINDOW && j0 + BN - 1 <= q_first + shift - W))
            return;
        // every key visible to every row of the wave
        const bool full = j0 >= jmin && j0 + BN - 1 <= q_first + shift &&
                          (!WINDOW || q_last + shift - j0 < W);
        const uint8_t* kst = smem + ST * K_TILE;
        const uint8_t* vst = smem + ST * V_TILE;   // + v_rd, which holds the V area's base

        f32x16 S0, S1;
        // the tile's scores minus the rows' references, masked outside each row's visible keys
        auto scores = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
                const uint8_t* kp = kst + k_rd[c & 3] + (c >> 2) * 128;
                const bf16x8 A0 = *(const bf16x8*)(kp);
                const bf16x8 A1 = *(const bf16x8*)(kp + 32 * DQK * 2);
                S0 = mfma32x32x16(A0, Qb[c], c == 0 ? negm : S0);
                S1 = mfma32x32x16(A1, Qb[c], c == 0 ? negm : S1);
            }
            if (!full) {
                // (the empty asm keeps the compiler from if-converting this uniform branch, which
                //  would run the masking on every tile)
                asm volatile("");
                // key j0 + 8(i/4) + 4g + i%4 (+32 in block 1) against row q_l: visible iff the
                // unsigned difference d - off is below the row's limit
                const int d = q_l + shift - j0 - 4 * g;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int off = 8 * (i >> 2) + (i & 3);
                    S0[i] = (unsigned)(d - off) < lim ? S0[i] : -INFINITY;
                    S1[i] = (unsigned)(d - off - 32) < lim ? S1[i] : -INFINITY;
                }
            }
        };
        // the reference moves to the row's maximum on its first visible key, later when a tile
        // exceeds it by more than 2^kRescaleLog2; the tile's scores, the sum and O follow the move
        auto rebase = [&]() __attribute__((always_inline)) {
            float ma = fmaxf(S0[0], S1[0]), mb = fmaxf(S0[8], S1[8]);
#pragma unroll
            for (int i = 1; i < 8; ++i) {
                ma = fmaxf(fmaxf(ma, S0[i]), S1[i]);
                mb = fmaxf(fmaxf(mb, S0[i + 8]), S1[i + 8]);
            }
            const float mx = max_lane_pair32(fmaxf(ma, mb));   // relative to the reference
            const bool first = m_run == -INFINITY;
            const bool raise = mx > kRescaleLog2 || (first && mx != -INFINITY);
            const float ref = -negm[0];
            const float shift = raise ? mx : 0.0f;
            const float alpha = first ? 1.0f : fast_exp2(-shift);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DV / 32; ++db) O[db] *= alpha;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                S0[i] -= shift;
                S1[i] -= shift;
                negm[i] = -(ref + shift);
            }
            if (raise) m_run = ref + shift;
        };
        float ps0, ps1;
        auto weights = [&]() __attribute__((always_inline)) {
            ps0 = ps1 = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                S0[i] = fast_exp2(S0[i]);
                S1[i] = fast_exp2(S1[i]);
                ps0 += S0[i];
                ps1 += S1[i];
            }
        };
        // No row maximum on the common path: the weights come straight from the scores, and a
        // row whose scores outgrew its reference shows in its lanes' sums of weights (above
        // 2^kSumLog2, or infinite).  Only then (and on a row's first visible keys) are the tile's
        // scores computed again, still in LDS, and the reference moved to the maximum.
        scores();
        if (__any(m_run == -INFINITY)) {
            asm volatile("");   // a row's first keys (uniform branch)
            rebase();
        }
        weights();
        if (__any(ps0 + ps1 > kSumLimit)) {
            asm volatile("");   // rare (uniform branch)
            scores();
            rebase();
            weights();
        }
        l_run += ps0 + ps1;

        // P^T operands: 16-key chunk c = registers 8*(c%2) .. +8 of block c/2
        bf16x8 Pb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x16& Sx = (c >> 1) ? S1 : S0;
            const int o = 8 * (c & 1);
            Pb[c] = as_bf16x8(u32x4{pack_bf16x2(Sx[o], Sx[o + 1]), pack_bf16x2(Sx[o + 2], Sx[o + 3]),
                                    pack_bf16x2(Sx[o + 4], Sx[o + 5]), pack_bf16x2(Sx[o + 6], Sx[o + 7])});
        }
        // O^T += V^T * P^T: k-slot t of lane group g is key 16c + 4g + t (t < 4) or
        // 16c + 8 + 4g + (t - 4); ds_read_b64_tr_b16 hands lane i of a 16-lane group
        // V[key0 + t][dv0 + i] when it points at V[key0 + i/4][dv0 + 4(i%4)].
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
    };

    // ---- main loop: tile t lives in stage t % STAGES; up to STAGES - 2 later tiles may still be
    //      in flight while tile t is awaited
    auto step = [&](int t, auto stage_c) {
        constexpr int ST = decltype(stage_c)::value;
        if (STAGES == 3 && t + 1 < n_tiles) wait_vmcnt<K_DMA + V_DMA>();
        else wait_vmcnt<0>();
        block_sync_lds();   // tile t is in LDS for every wave; stage (t - 1) % STAGES is free
        if (t + STAGES - 1 < n_tiles)
            issue(t + STAGES - 1, std::integral_constant<int, (ST + STAGES - 1) % STAGES>{});
        compute(t, stage_c);
    };
    for (int t = 0; t < n_tiles; t += STAGES) {
        step(t, std::integral_constant<int, 0>{});
        if (t + 1 < n_tiles) step(t + 1, std::integral_constant<int, 1 % STAGES>{});
        if (STAGES == 3 && t + 2 < n_tiles) step(t + 2, std::integral_constant<int, 2 % STAGES>{});
    }

    // ---- epilogue: out = v_scale * O / l, bf16.  Lane (l32, g) holds row q_l, dims
    //      32 db + 8 ii + 4 g..; on global layers the wave's 32 rows (8 KiB) pass through LDS so
    //      that the stores write whole 256-byte rows (16 lanes x 16 bytes, non-temporally).  The
    //      staging areas are the two ring stages the last tile does not use (free since that
    //      tile's barrier: no copy is issued after it): waves 0-5 in their K parts, 6-7 in the V
    //      part of the first; 32-byte blocks of row r sit at block ^ (r % 8).
    const float lt = sum_lane_pair32(l_run);
    const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
    if constexpr (!WINDOW && STAGES == 3 && NW == 8) {
        const int s_last = (n_tiles + STAGES - 1) % STAGES;   // stage of the last tile (if any)
        const int f0 = s_last == 0 ? 1 : 0, f1 = s_last == 2 ? 1 : 2;   // the other two
        uint8_t* const stg = wave < 6 ? smem + (wave < 3 ? f0 : f1) * K_TILE + (wave % 3) * 8192
                                      : smem + STAGES * K_TILE + f0 * V_TILE + (wave - 6) * 8192;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                // row l32, bytes 64 db + 16 ii + 8 g: 32-byte block 2 db + ii / 2
                const int blk = 2 * db + (ii >> 1);
                *(u32x2*)(stg + l32 * 256 + 32 * (blk ^ (l32 & 7)) + 16 * (ii & 1) + 8 * g) =
                    u32x2{pack_bf16x2(O[db][4 * ii] * inv, O[db][4 * ii + 1] * inv),
                          pack_bf16x2(O[db][4 * ii + 2] * inv, O[db][4 * ii + 3] * inv)};
            }
        }
        __builtin_amdgcn_wave_barrier();
        const int c16 = lane & 15;   // 16-byte column of the row
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int row = (lane >> 4) + 4 * k, q = q_first + row;
            const u32x4 ov =
                *(const u32x4*)(stg + row * 256 + 32 * ((c16 >> 1) ^ (row & 7)) + 16 * (c16 & 1));
            if (q < S)   // (written once: non-temporal)
                __builtin_nontemporal_store(
                    ov, (u32x4*)(a.out + (((int64_t)b * S + q) * Hq + h) * DV + 8 * c16));
        }
    } else if (q_l < S) {
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


// Sliding layers, GQA group a multiple of 4: a workgroup of 4 waves takes 4 query heads of one KV
// group over 16 rows (wave w: head 4 * unit + w), on v_mfma_f32_16x16x32_bf16, with 32-key tiles
// through a 2-stage LDS ring (40 KiB): about 100 registers and 40 KiB per workgroup, so that four
// workgroups share a CU and their memory phases (query rows in, outputs out) overlap the others'
// products.  Layouts in LDS as in prefill_kernel (K chunk c of row r at c ^ ((r >> 1) & 7), V
// chunk c at c ^ ((r & 3) << 2)); the scores and the weighted sum follow the decode kernel's
// operand layout:
//   S^T (16 keys x 16 rows) = K * Q^T: A = K, lane l holds key l % 16, dims 32c + 8(l / 16) + [0, 8);
//     B = Q^T, lane l holds row l % 16, the same dims; C: lane l holds row l % 16, keys 4(l / 16) + i;
//   O^T (16 dims x 16 rows) += V^T * P^T: k-slot t of lane group gq is key 4gq + t (t < 4) or
//     16 + 4gq + (t - 4) of the 32-key tile, on both operands.
constexpr int SW16_ROWS = 16;
constexpr int SW16_BN = 32;
constexpr int SW16_K_TILE = SW16_BN * DQK * 2;   // 12 KiB
constexpr int SW16_V_TILE = SW16_BN * DV * 2;    // 8 KiB
constexpr int SW16_WAVES = 4;

template <bool SINK>
__global__ __launch_bounds__(SW16_WAVES * 64) __attribute__((amdgpu_waves_per_eu(4))) void
prefill_sw16_kernel(const PrefillArgs a) {
    constexpr int NW = SW16_WAVES, BN = SW16_BN, QR = SW16_ROWS;
    constexpr int K_DMA = SW16_K_TILE / 1024 / NW;   // 3
    constexpr int V_DMA = SW16_V_TILE / 1024 / NW;   // 2
    constexpr int KC = DQK / 32;                     // 32-dim k-chunks of the scores
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * (SW16_K_TILE + SW16_V_TILE)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, gq = lane >> 4;
    const int S = a.S, Hq = a.Hq;
    const int nqblk = (S + QR - 1) / QR;
    const int hunits = Hq / NW;

    // work item: workgroup ids go round-robin to the 8 XCDs; each XCD walks the row blocks of its
    // own (sequence, head unit) pairs in order, so the K/V band stays in that XCD's L2
    const int id = blockIdx.x;
    int w = id;
    const int pairs = a.B * hunits;
    if (pairs % 8 == 0) {
        const int P = pairs / 8, xcd = id & 7, k = id >> 3;
        w = (k / P) * pairs + xcd * P + k % P;
    }
    const int hu = w % hunits;
    const int b = (w / hunits) % a.B;
    const int qblk = w / (hunits * a.B);
    const int h = hu * NW + wave;
    const int kvh = hu * NW / (Hq / a.Hkv);
    const int r = a.rope_dims, half = r >> 1;

    // the frequencies of this thread's entries of the rows' cos/sin table (entry e = row * r/2 + f,
    // thread tid taking e = tid, tid + 256, ...), from the argument segment through a pointer the
    // compiler cannot trace back to it, so that the loads stay ahead of the table's barrier
    constexpr int TAB = (QR * kMaxRopeHalfArgs + NW * 64 - 1) / (NW * 64);
    double om_tab[TAB];
    {
        const char* kargs = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(kargs));
        const __attribute__((address_space(1))) double* om_args =
            (const __attribute__((address_space(1))) double*)(kargs + offsetof(PrefillArgs, omega_rev));
#pragma unroll
        for (int k = 0; k < TAB; ++k) {
            const int e = tid + k * NW * 64;
            om_tab[k] = e < QR * half ? om_args[e % half] : 0.0;
        }
    }

    // key rows (as in prefill_kernel): row j at position kpos0 + j; query row i meets key row
    // i + shift at its own position; rows below jmin hold no token
    int32_t p0 = 0;
    bool seq_ok;
    int shift, jmin;
    const bool own_rows = a.max_start < 0 && a.kpos_rel && a.kpos_off >= 0;
    if (own_rows) {
        seq_ok = true;
        shift = -a.kpos_off;
        jmin = 0;
    } else {
        p0 = load_scalar_i32(a.start_pos + b);
        seq_ok = a.max_start < 0 || (unsigned)p0 <= (unsigned)a.max_start;
        const int32_t kpos0 = (a.kpos_rel ? (seq_ok ? p0 : 0) : 0) + a.kpos_off;
        shift = (seq_ok ? p0 : 0) - kpos0;
        jmin = max(0, -kpos0);
    }
    const int nk = S + shift;
    const int W = a.window;
    const int q_first = qblk * QR;
    const int q_last = min(q_first + QR, S) - 1;
    const int kt_lo = max(jmin, q_first + shift - W + 1) / BN;
    const int n_tiles = seq_ok ? (q_last + shift) / BN + 1 - kt_lo : 0;

    // DMA: LDS 16-byte slot P of this wave's instruction i holds K row P / 24, chunk
    // (P % 24) ^ ((row >> 1) & 7); V row P / 16, chunk (P % 16) ^ ((row & 3) << 2)
    const uint16_t* kslice = a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
    const uint16_t* vslice = a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;
    const int64_t v_sj = a.v_sj;
    auto k_slot = [&](int i, int ln, int& row, int& col) __attribute__((always_inline)) {
        const int P = (wave * K_DMA + i) * 64 + ln;
        row = P / (DQK / 8);
        col = ((P % (DQK / 8)) ^ ((row >> 1) & 7)) * 8;
    };
    auto v_slot = [&](int i, int ln, int& row, int& col) __attribute__((always_inline)) {
        const int P = (wave * V_DMA + i) * 64 + ln;
        row = P / (DV / 8);
        col = ((P % (DV / 8)) ^ ((row & 3) << 2)) * 8;
    };
    uint32_t k_lo[K_DMA], v_lo[V_DMA];
#pragma unroll
    for (int i = 0; i < K_DMA; ++i) {
        int row, col;
        k_slot(i, lane, row, col);
        k_lo[i] = (uint32_t)(row * DQK + col) * 2u;
    }
#pragma unroll
    for (int i = 0; i < V_DMA; ++i) {
        int row, col;
        v_slot(i, lane, row, col);
        v_lo[i] = (uint32_t)((int64_t)row * v_sj + col) * 2u;
    }
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8_t*)smem;
    auto issue = [&](int t, int st) __attribute__((always_inline)) {
        const int j0 = (kt_lo + t) * BN;
        const uint32_t kst = lds0 + st * SW16_K_TILE;
        const uint32_t vst = lds0 + 2 * SW16_K_TILE + st * SW16_V_TILE;
        if (j0 >= jmin && j0 + BN <= nk) {
            const uint16_t* kb = kslice + (int64_t)j0 * DQK;
            const uint16_t* vb = vslice + (int64_t)j0 * v_sj;
#pragma unroll
            for (int i = 0; i < K_DMA; ++i) dma16_sbase(kb, k_lo[i], kst + (wave * K_DMA + i) * 1024);
#pragma unroll
            for (int i = 0; i < V_DMA; ++i) dma16_sbase(vb, v_lo[i], vst + (wave * V_DMA + i) * 1024);
        } else {
            int ln = lane;
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int i = 0; i < K_DMA; ++i) {
                int row, col;
                k_slot(i, ln, row, col);
                const int j = min(max(j0 + row, jmin), nk - 1);
                dma16(kslice + (int64_t)j * DQK + col, kst + (wave * K_DMA + i) * 1024);
            }
#pragma unroll
            for (int i = 0; i < V_DMA; ++i) {
                int row, col;
                v_slot(i, ln, row, col);
                const int j = min(max(j0 + row, jmin), nk - 1);
                dma16(vslice + (int64_t)j * v_sj + col, vst + (wave * V_DMA + i) * 1024);
            }
        }
    };
    if (n_tiles > 0) issue(0, 0);

    // ---- Q^T operands (rows q_first + l16, dims 32c + 8gq..), rotated and scaled by
    //      tau * log2(e), rounded once to bf16; the rows' cos/sin table lives in K stage 1 until
    //      the first tile step
    const float sc = a.score_scale_log2;
    bf16x8 Qb[KC];
    {
        const int qi = q_first + l16;
        const bool qok = qi < S;
        const uint16_t* qrow = a.q + (((int64_t)b * S + (qok ? qi : S - 1)) * Hq + h) * DQK;
        u32x4 qw[KC], pw[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) qw[c] = *(const u32x4*)(qrow + 32 * c + 8 * gq);
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const int d0 = 32 * c + 8 * gq;
            if (d0 < r) pw[c] = *(const u32x4*)(qrow + (d0 < half ? d0 + half : d0 - half));
        }
        if (own_rows) p0 = load_scalar_i32(a.start_pos + b);
        float2* cs = (float2*)(smem + SW16_K_TILE);
        const int pitch = QR * (half + 1) * 8 <= SW16_K_TILE ? half + 1 : half;
#pragma unroll
        for (int k = 0; k < TAB; ++k) {
            const int e = tid + k * NW * 64;
            if (e < QR * half) {
                const int row = e / half, f = e - row * half;
                float c, sn;
                rope_cos_sin_rev(p0 + min(q_first + row, S - 1), om_tab[k], c, sn);
                cs[row * pitch + f] = make_float2(c, sn);
            }
        }
        block_sync_lds();
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const int d0 = 32 * c + 8 * gq;
            if (d0 < r) {
                const bool lower = d0 < half;
                const float2* e = cs + l16 * pitch + (lower ? d0 : d0 - half);
                float x[8], y[8];
                unpack8(qw[c], x);
                unpack8(pw[c], y);
                const float sgn = lower ? -1.0f : 1.0f;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float2 cst = e[t];
                    x[t] = __builtin_fmaf(sgn * y[t], cst.y, x[t] * cst.x) * sc;
                }
                qw[c] = pack8(x);
            } else {
                qw[c] = scale8(qw[c], sc);
            }
            if (!qok) qw[c] = u32x4{0u, 0u, 0u, 0u};
            Qb[c] = as_bf16x8(qw[c]);
        }
    }

    // ---- per-lane LDS read offsets within a stage: K (key l16 of block kb, chunk 4c + gq),
    //      V^T (rows 4gq + l16 / 4 and + 16, dims 16db + 4(l16 % 4))
    int k_rd[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) k_rd[c] = l16 * (DQK * 2) + 16 * ((4 * c + gq) ^ ((l16 >> 1) & 7));
    int v_rd[DV / 16];
    {
        const int vrow = 4 * gq + (l16 >> 2);
#pragma unroll
        for (int db = 0; db < DV / 16; ++db) {
            const int byte = (db * 16 + 4 * (l16 & 3)) * 2;
            v_rd[db] = 2 * SW16_K_TILE + vrow * (DV * 2) + 16 * ((byte >> 4) ^ ((vrow & 3) << 2)) +
                       (byte & 15);
            asm volatile("" : "+v"(v_rd[db]));
        }
    }

    const float sink_l2 = SINK ? a.sinks[h] * kLog2e : -INFINITY;
    float m_run = SINK ? sink_l2 : -INFINITY;      // reference maximum (lazily raised)
    float l_run = (SINK && gq == 0) ? 1.0f : 0.0f;
    float m_ref = SINK ? sink_l2 : 0.0f;
    f32x4 O[DV / 16];
#pragma unroll
    for (int db = 0; db < DV / 16; ++db) O[db] = f32x4{};
    const int q_l = q_first + l16;
    const unsigned lim = (unsigned)max(0, min(W, q_l + shift - jmin + 1));

    auto compute = [&](int t, int st) __attribute__((always_inline)) {
        const int j0 = (kt_lo + t) * BN;
        if (j0 > q_last + shift || j0 + BN - 1 <= q_first + shift - W) return;   // uniform
        const bool full = j0 >= jmin && j0 + BN - 1 <= q_first + shift && q_last + shift - j0 < W;
        const uint8_t* kst = smem + st * SW16_K_TILE;
        const uint8_t* vst = smem + st * SW16_V_TILE;   // + v_rd, which holds the V area's base
        f32x4 Sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x4 acc = f32x4{};
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const bf16x8 A = *(const bf16x8*)(kst + k_rd[c] + kb * 16 * (DQK * 2));
                acc = mfma16x16x32(A, Qb[c], acc);
            }
            Sacc[kb] = acc;
        }
        if (!full) {
            asm volatile("");
            // key j0 + 16kb + 4gq + i against row q_l
            const int d = q_l + shift - j0 - 4 * gq;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sacc[kb][i] = (unsigned)(d - 16 * kb - i) < lim ? Sacc[kb][i] : -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(Sacc[0][0], Sacc[0][1]), fmaxf(Sacc[0][2], Sacc[0][3])),
                         fmaxf(fmaxf(Sacc[1][0], Sacc[1][1]), fmaxf(Sacc[1][2], Sacc[1][3])));
        mx = max_lane_pair32(max_lane_pair16(mx));
        const bool first = m_run == -INFINITY;
        const bool raise = first ? mx != -INFINITY : mx > m_ref + kRescaleLog2;
        if (__any(raise)) {
            asm volatile("");
            const float m_new = raise ? mx : m_ref;
            const float alpha = (raise && !first) ? fast_exp2(m_ref - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DV / 16; ++db) O[db] *= alpha;
            m_ref = m_new;
            if (raise) m_run = m_new;
        }
        float ps = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Sacc[kb][i] = fast_exp2(Sacc[kb][i] - m_ref);
                ps += Sacc[kb][i];
            }
        l_run += ps;
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
            O[db] = mfma16x16x32(__builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7), Pb, O[db]);
        }
    };

    for (int t = 0; t < n_tiles; ++t) {
        const int st = t & 1;
        wait_vmcnt<0>();
        block_sync_lds();   // tile t in LDS for every wave; the other stage (and the table) free
        if (t + 1 < n_tiles) issue(t + 1, st ^ 1);
        compute(t, st);
    }

    // ---- epilogue: out = v_scale * O / l (bf16).  Lane l holds row q_l, dims 16db + 4gq..; the
    //      wave's 16 rows (4 KiB) pass through LDS so that the stores write whole 256-byte rows
    //      (16 lanes x 16 bytes, non-temporally) instead of 32 bytes of a row per instruction.  The
    //      staging area is the ring stage the last tile does not use (free since that tile's
    //      barrier): waves 0-2 in its K part, wave 3 in its V part; 32-byte blocks of row r sit at
    //      block ^ (r % 8).
    const float lt = sum_lane_pair32(sum_lane_pair16(l_run));
    const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
    const int st_free = n_tiles & 1;
    uint8_t* const stg = wave < 3 ? smem + st_free * SW16_K_TILE + wave * 4096
                                  : smem + 2 * SW16_K_TILE + st_free * SW16_V_TILE;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int db = 0; db < DV / 16; ++db)
        *(u32x2*)(stg + l16 * 256 + 32 * (db ^ (l16 & 7)) + 8 * gq) =
            u32x2{pack_bf16x2(O[db][0] * inv, O[db][1] * inv),
                  pack_bf16x2(O[db][2] * inv, O[db][3] * inv)};
    __builtin_amdgcn_wave_barrier();
    const int c16 = lane & 15;   // 16-byte column of the row
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int row = (lane >> 4) + 4 * k, q = q_first + row;
        const u32x4 ov = *(const u32x4*)(stg + row * 256 + 32 * ((c16 >> 1) ^ (row & 7)) + 16 * (c16 & 1));
        if (q < S)   // (written once: non-temporal)
            __builtin_nontemporal_store(ov, (u32x4*)(a.out + (((int64_t)b * S + q) * Hq + h) * DV + 8 * c16));
    }
}

}  // namespace

int prefill_bf16_block_rows(bool window) { return (window ? SW_WAVES : GA_WAVES) * QPW; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, bool window, bool sink, hipStream_t st) {
    if (a.k_sj != DQK) return hipErrorInvalidValue;   // keys must be contiguous rotated rows
    if (window && (a.Hq / a.Hkv) % SW16_WAVES == 0 && a.v_sj < (1 << 24)) {
        // sliding layers with whole groups of 4 query heads per KV head: 16-row workgroups of 4
        // heads, four per CU
        const int64_t nwg = (int64_t)a.B * (a.Hq / SW16_WAVES) * ((a.S + SW16_ROWS - 1) / SW16_ROWS);
        if (nwg == 0) return hipSuccess;
        if (nwg > 0x7fffffff) return hipErrorInvalidConfiguration;
        if (sink) prefill_sw16_kernel<true><<<dim3((unsigned)nwg), dim3(SW16_WAVES * 64), 0, st>>>(a);
        else prefill_sw16_kernel<false><<<dim3((unsigned)nwg), dim3(SW16_WAVES * 64), 0, st>>>(a);
        return hipGetLastError();
    }
    const int bm = prefill_bf16_block_rows(window);
    const int nqblk = (a.S + bm - 1) / bm;
    const int64_t total = (int64_t)a.B * a.Hq * nqblk;
    if (total == 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)total);
    if (window) {
        const dim3 block(SW_WAVES * 64);
        if (sink) prefill_kernel<SW_WAVES, SW_STAGES, true, true><<<grid, block, 0, st>>>(a);
        else prefill_kernel<SW_WAVES, SW_STAGES, true, false><<<grid, block, 0, st>>>(a);
    } else {
        const dim3 block(GA_WAVES * 64);
        if (sink) prefill_kernel<GA_WAVES, GA_STAGES, false, true><<<grid, block, 0, st>>>(a);
        else prefill_kernel<GA_WAVES, GA_STAGES, false, false><<<grid, block, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace mimo
