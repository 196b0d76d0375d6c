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
//   * each wave owns 32 query rows of one query head and keeps their rotated Q^T (bf16) in
//     registers; global layers: 8 waves on 8 consecutive row blocks of one head, one workgroup per
//     CU; sliding layers: 4 waves, two workgroups per CU, and when the GQA group is a multiple of 4
//     the 4 waves take 4 heads of one KV group over the same 32 rows, so every wave computes every
//     tile of the ~3-tile band and each K/V tile feeds 4 heads;
//   * K (64 x 192) and V (64 x 128) tiles stream through a 3-stage (global) or 2-stage (sliding)
//     LDS ring filled by global_load_lds_dwordx4 (memory -> LDS without registers) one or two
//     tiles ahead of the one being computed; one barrier per tile;
//   * LDS layouts are unpadded and XOR-swizzled at 16-byte granularity so that the MFMA operand
//     reads are conflict-free: K chunk c of row r sits at c ^ ((r >> 1) & 7); V chunk c of row r at
//     c ^ ((r & 3) << 2);
//   * S^T = K * Q^T with v_mfma_f32_32x32x16_bf16 (each lane owns one query column), online
//     softmax in the log2 domain with a lazily raised running maximum (the maximum is only moved
//     when a tile exceeds it by more than 2^8, so the O rescale is rare; the result is exact because
//     numerator and denominator share the reference), O^T += V^T * P^T with V^T read by
//     ds_read_b64_tr_b16;
//   * the wave index is made scalar so tile skipping and the band-edge masking are uniform
//     branches; sliding-window workgroups only stream the tiles of their band, and each wave only
//     computes the tiles its own rows can see;
//   * global layers: workgroups are ordered heavy-first and grouped so that the workgroups the
//     dispatcher sends to one XCD in a row share a KV head (its K/V stay hot in that XCD's L2);
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


__device__ __forceinline__ void rotate_pair8_kernarg(u32x4& lo, u32x4& hi, int32_t pos,
                                                     const double* om) {
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

// GROUPED: a workgroup covers NW query heads of one KV group over the same 32 rows (wave w takes
// head base + w); otherwise it covers NW consecutive 32-row blocks of one query head.
template <int NW, int STAGES, bool WINDOW, bool SINK, bool GROUPED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    const PrefillArgs a) {
    constexpr int BM = GROUPED ? QPW : NW * QPW;   // query rows per workgroup
    constexpr int K_DMA = K_TILE / 1024 / NW;      // 1-KiB DMA instructions per wave per tile
    constexpr int V_DMA = V_TILE / 1024 / NW;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * (K_TILE + V_TILE)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int S = a.S, Hq = a.Hq;
    const int nqblk = (S + BM - 1) / BM;
    const int hunits = GROUPED ? Hq / NW : Hq;     // head units per (row block, sequence)
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
        const int xcd = id & 7, slot = id >> 3, grp = slot >> 3;
        if ((grp + 1) * 64 <= total) w = grp * 64 + xcd * 8 + (slot & 7);
    }
    const int hu = w % hunits;
    const int b = (w / hunits) % a.B;
    const int qrank = w / (hunits * a.B);
    const int qblk = WINDOW ? qrank : nqblk - 1 - qrank;   // global: heaviest blocks first
    const int h = GROUPED ? hu * NW + wave : hu;
    const int kvh = (GROUPED ? hu * NW : hu) / (Hq / a.Hkv);
    const int r = a.rope_dims, half = r >> 1;
    // GROUPED: the frequencies of this thread's entries of the rows' cos/sin table (entry
    // e = row * r/2 + frequency, thread tid taking e = tid, tid + 256, ...), requested first, from
    // the argument segment through a pointer the compiler cannot trace back to it, so that the
    // loads stay ahead of the barrier that follows the table
    constexpr int TAB = GROUPED ? (QPW * kMaxRopeHalfArgs + NW * 64 - 1) / (NW * 64) : 1;
    double om_tab[TAB];
    if constexpr (GROUPED) {
        const char* kargs = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(kargs));
        const __attribute__((address_space(1))) double* om_args =
            (const __attribute__((address_space(1))) double*)(kargs + offsetof(PrefillArgs, omega_rev));
#pragma unroll
        for (int k = 0; k < TAB; ++k) {
            const int e = tid + k * NW * 64;
            om_tab[k] = e < QPW * half ? om_args[e % half] : 0.0;
        }
    }
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
    const int q_first = qblk * BM + (GROUPED ? 0 : wave * QPW);   // this wave's first row (scalar)
    const int q_last = min(q_first + QPW, S) - 1;                 // its last valid row
    const int blk_first = qblk * BM;
    const int blk_last = min(blk_first + BM, S) - 1;
    const int kt_lo = max(jmin, WINDOW ? blk_first + shift - W + 1 : 0) / BN;
    const int n_tiles = seq_ok ? (blk_last + shift) / BN + 1 - kt_lo : 0;

    // ---- DMA source mapping: LDS 16-byte slot P of this wave's instruction i holds
    //      K row P / 24, logical chunk (P % 24) ^ swizzle; V row P / 16, chunk (P % 16) ^ swizzle.
    const uint16_t* kslice = a.k + (int64_t)b * a.k_sb + (int64_t)kvh * a.k_sh;
    const uint16_t* vslice = a.v + (int64_t)b * a.v_sb + (int64_t)kvh * a.v_sh;
    const int64_t v_sj = a.v_sj;
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
    // per-lane source pointers of tile 0; tile t adds t * BN rows (a scalar offset) except on a
    // tile that reaches past the key rows [jmin, nk): its rows are clamped into that range (they
    // are masked anyway, and clamping keeps unwritten rows out of the products)
    const uint16_t* kp[K_DMA];
    const uint16_t* vp[V_DMA];
#pragma unroll
    for (int i = 0; i < K_DMA; ++i) kp[i] = kslice + (int64_t)(kt_lo * BN + k_row[i]) * DQK + k_off[i];
#pragma unroll
    for (int i = 0; i < V_DMA; ++i) vp[i] = vslice + (int64_t)(kt_lo * BN + v_row[i]) * v_sj + v_off[i];
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8_t*)smem;
    auto issue = [&](int t, auto stage_c) {
        constexpr int ST = decltype(stage_c)::value;
        const int j0 = (kt_lo + t) * BN;
        const uint32_t kst = lds0 + ST * K_TILE;
        const uint32_t vst = lds0 + STAGES * K_TILE + ST * V_TILE;
        if (j0 >= jmin && j0 + BN <= nk) {
            const int64_t dk = (int64_t)t * BN * DQK, dv = (int64_t)t * BN * v_sj;
#pragma unroll
            for (int i = 0; i < K_DMA; ++i) dma16(kp[i] + dk, kst + (wave * K_DMA + i) * 1024);
#pragma unroll
            for (int i = 0; i < V_DMA; ++i) dma16(vp[i] + dv, vst + (wave * V_DMA + i) * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < K_DMA; ++i) {
                const int j = min(max(j0 + k_row[i], jmin), nk - 1);
                dma16(kslice + (int64_t)j * DQK + k_off[i], kst + (wave * K_DMA + i) * 1024);
            }
#pragma unroll
            for (int i = 0; i < V_DMA; ++i) {
                const int j = min(max(j0 + v_row[i], jmin), nk - 1);
                dma16(vslice + (int64_t)j * v_sj + v_off[i], vst + (wave * V_DMA + i) * 1024);
            }
        }
    };
    if (n_tiles > 0) issue(0, std::integral_constant<int, 0>{});
    if (STAGES == 3 && n_tiles > 1) issue(1, std::integral_constant<int, 1 % STAGES>{});

    // ---- Q^T operands, rotated, in registers
    bf16x8 Qb[KCH];
    {
        const int qi = q_first + l32;
        const bool qok = qi < S;
        const uint16_t* qrow = a.q + (((int64_t)b * S + (qok ? qi : S - 1)) * Hq + h) * DQK;
        u32x4 qw[KCH];
#pragma unroll
        for (int c = 0; c < KCH; ++c) qw[c] = *(const u32x4*)(qrow + 16 * c + 8 * g);
        if constexpr (GROUPED) {
            // rotation partners, requested with the rows themselves
            u32x4 pw[KCH];
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
                const int d0 = 16 * c + 8 * g;
                if (d0 < r) pw[c] = *(const u32x4*)(qrow + (d0 < half ? d0 + half : d0 - half));
            }
            if (own_rows) p0 = load_scalar_i32(a.start_pos + b);
            // The NW waves share the 32 rows (one head each): the cos/sin of the rows' positions
            // per frequency are evaluated once for the workgroup into a table in K stage 1, which
            // no tile uses before the first tile step.  Rows are padded by one entry (so that the
            // 32 rows' reads of one frequency hit distinct banks) while 32 x (r/2 + 1) entries of
            // 8 bytes fit the stage, i.e. up to r = 190; at r = 192 they are packed.
            static_assert(STAGES == 2, "table lives in stage 1");
            float2* cs = (float2*)(smem + K_TILE);
            const int pitch = QPW * (half + 1) * 8 <= K_TILE ? half + 1 : half;
#pragma unroll
            for (int k = 0; k < TAB; ++k) {
                const int e = tid + k * NW * 64;
                if (e < QPW * half) {
                    const int row = e / half, f = e - row * half;
                    float c, sn;
                    rope_cos_sin_rev(p0 + min(q_first + row, S - 1), om_tab[k], c, sn);
                    cs[row * pitch + f] = make_float2(c, sn);
                }
            }
            block_sync_lds();
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
                const int d0 = 16 * c + 8 * g;
                if (d0 < r) {
                    const bool lower = d0 < half;
                    const float2* e = cs + l32 * pitch + (lower ? d0 : d0 - half);
                    float x[8], y[8];
                    unpack8(qw[c], x);
                    unpack8(pw[c], y);
                    const float sgn = lower ? -1.0f : 1.0f;
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float2 cst = e[t];
                        x[t] = __builtin_fmaf(sgn * y[t], cst.y, x[t] * cst.x);
                    }
                    qw[c] = pack8(x);
                }
                if (!qok) qw[c] = u32x4{0u, 0u, 0u, 0u};
                Qb[c] = as_bf16x8(qw[c]);
            }
        } else {
            if (own_rows) p0 = load_scalar_i32(a.start_pos + b);
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
                const int d0 = 16 * c + 8 * g;
                if (d0 < r) {
                    const bool lower = d0 < half;
                    u32x4 lo = lower ? qw[c] : *(const u32x4*)(qrow + d0 - half);
                    u32x4 hi = lower ? *(const u32x4*)(qrow + d0 + half) : qw[c];
                    rotate_pair8_kernarg(lo, hi, p0 + qi, a.omega_rev + (lower ? d0 : d0 - half));
                    qw[c] = lower ? lo : hi;
                }
                if (!qok) qw[c] = u32x4{0u, 0u, 0u, 0u};
                Qb[c] = as_bf16x8(qw[c]);
            }
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
    const float sc = a.score_scale_log2;
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
        // row maximum: two chains of 3-input maxima
        float ma = fmaxf(S0[0], S1[0]), mb = fmaxf(S0[8], S1[8]);
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            ma = fmaxf(fmaxf(ma, S0[i]), S1[i]);
            mb = fmaxf(fmaxf(mb, S0[i + 8]), S1[i + 8]);
        }
        const float mx = max_lane_pair32(fmaxf(ma, mb)) * sc;
        // lazily raised reference maximum
        const bool raise = mx > m_run + kRescaleLog2 || m_run == -INFINITY;
        const float m_new = raise ? fmaxf(m_run, mx) : m_run;
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        if (__any(raise)) {
            asm volatile("");   // rare: keep it a branch (see above)
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

    // ---- epilogue: out = v_scale * O / l, bf16
    const float lt = sum_lane_pair32(l_run);
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

int prefill_bf16_block_rows(bool window) { return (window ? SW_WAVES : GA_WAVES) * QPW; }

hipError_t launch_prefill_bf16(const PrefillArgs& a, bool window, bool sink, hipStream_t st) {
    if (a.k_sj != DQK) return hipErrorInvalidValue;   // keys must be contiguous rotated rows
    const int group = a.Hq / a.Hkv;
    const bool grouped = window && group % SW_WAVES == 0;
    const int bm = grouped ? QPW : prefill_bf16_block_rows(window);
    const int nqblk = (a.S + bm - 1) / bm;
    const int64_t total = (int64_t)a.B * (grouped ? a.Hq / SW_WAVES : a.Hq) * nqblk;
    if (total == 0) return hipSuccess;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)total);
    if (window) {
        const dim3 block(SW_WAVES * 64);
        if (grouped) {
            if (sink) prefill_kernel<SW_WAVES, SW_STAGES, true, true, true><<<grid, block, 0, st>>>(a);
            else prefill_kernel<SW_WAVES, SW_STAGES, true, false, true><<<grid, block, 0, st>>>(a);
        } else {
            if (sink) prefill_kernel<SW_WAVES, SW_STAGES, true, true, false><<<grid, block, 0, st>>>(a);
            else prefill_kernel<SW_WAVES, SW_STAGES, true, false, false><<<grid, block, 0, st>>>(a);
        }
    } else {
        const dim3 block(GA_WAVES * 64);
        if (sink) prefill_kernel<GA_WAVES, GA_STAGES, false, true, false><<<grid, block, 0, st>>>(a);
        else prefill_kernel<GA_WAVES, GA_STAGES, false, false, false><<<grid, block, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace mimo
