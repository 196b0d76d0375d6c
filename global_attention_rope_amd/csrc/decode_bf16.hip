// decode_bf16.hip — single-token decode of the hybrid attention layer against its KV cache.
//
// Pages: "Add Xiaomi MiMo-V2", section "Additional useful info" (per-kind theta and KV groups,
// decoupled V dim, value rescale, SWA-only sink); "add Xiaomi MiMo v2 (mimo_v2_flash)", section
// "Implementation plan" (sliding layers keep a rotating cache of the window).
//
// Per (sequence b, KV head g, split s) one workgroup of 4 waves:
//   * each wave issues the loads of its first 32-slot tile early — before the position is even
//     read on sliding layers and on small global-layer grids — so their latency overlaps the
//     query rotation.  Sliding layers load K straight into MFMA operand layout; global layers
//     load it as whole 1-KiB spans, non-temporally (each slot is read once), and pass it through
//     the wave's LDS tile area into operand layout; V comes as coalesced 16-byte rows
//     (non-temporal on global layers);
//   * the query heads of group g (<= 16) are rotated at the new token's position and kept as the
//     B operand of v_mfma_f32_16x16x32_bf16 (heads are the 16-wide N dimension);
//   * the split that owns the new token's slot rotates k_new, stores it and v_new into the cache
//     (linear: slot = position; ring: slot = position % window) and substitutes them for that
//     slot, so no workgroup reads a slot another one is writing;
//   * nothing before the slot loop waits for the other waves: each wave evaluates the cos/sin of
//     the position into its own LDS table, and only the wave whose tiles hold the new token's slot
//     prepares the new token, in its own LDS area (wave-level ordering only);
//   * per tile: S^T = K * Q^T, online softmax per head in the log2 domain, V staged in a per-wave
//     LDS tile and read transposed with ds_read_b64_tr_b16, O^T += V^T * P^T; the next tile's
//     loads are in flight meanwhile (two waves per SIMD keep ~160 KB per CU in flight);
//   * the waves are merged through LDS; with one split the sink is folded in and the bf16 output
//     written, otherwise (max, sum, O) partials go to the workspace and the combine kernel merges
//     the splits in one pass (running maximum) and adds the sink exactly once.
// The combine kernel also merges the split partials of the multi-token tile kernel (a few new
// tokens per sequence: one record per (sequence, token, query head, split)).
// fp8 caches (e4m3 codes, one scale per cache tensor): the slot loads are half as wide, codes are
// turned into their exact bf16 values in registers (K) or on their way into the LDS tile (V), the
// two scales are folded into the score scale and the output scale, and the new token is coded
// before it is stored and used.
#include <cstddef>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "verify.h"

namespace mimo {
namespace {

constexpr int DQK = 192;
constexpr int DV = 128;
constexpr int NW = 4;
constexpr int TILE = 32;                 // slots per wave iteration
constexpr int PSTRIDE = DV + 2;          // floats per partial record: O[128], m, l
constexpr int kDecodeSplitShift = 2;     // 2^shift consecutive splits of one pair in the dispatch order
constexpr int kDecodeSplitBlock = 1 << kDecodeSplitShift;
constexpr int VT_PITCH = DV + 16;        // bf16 per V row in the per-wave LDS tile (288 bytes)

constexpr int RO_PITCH = DV + 4;         // floats per head row of the wave-merge buffer
constexpr float kRescaleLog2 = 8.0f;     // raise a head's reference maximum only beyond 2^8

// Rotate 8 consecutive dims d0.. of a row (w) against their partners (pw) with the cos/sin of the
// row's position per frequency (cs, in LDS).  Dims at or past r read the identity entries
// (cos 1, sin 0) stored after the table, so every chunk runs the same straight-line code and the
// table reads of several chunks overlap.
constexpr int kIdentity = kMaxRopeHalf;   // first of 8 identity entries in the table
__device__ __forceinline__ void rotate8_cs_f32(const u32x4& w, const u32x4& pw, int d0, int half,
                                               int r, const float2* cs, float* x) {
    const bool lower = d0 < half;
    const int f0 = d0 < r ? (lower ? d0 : d0 - half) : kIdentity;
    float4 e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = *(const float4*)(cs + f0 + 2 * i);
    float y[8];
    unpack8(w, x);
    unpack8(pw, y);
    const float sgn = lower ? -1.0f : 1.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float c = (t & 1) ? e[t >> 1].z : e[t >> 1].x;
        const float sn = (t & 1) ? e[t >> 1].w : e[t >> 1].y;
        x[t] = __builtin_fmaf(sgn * y[t], sn, x[t] * c);
    }
}

__device__ __forceinline__ u32x4 rotate8_cs(const u32x4& w, const u32x4& pw, int d0, int half,
                                            int r, const float2* cs) {
    float x[8];
    rotate8_cs_f32(w, pw, d0, half, r, cs, x);
    return pack8(x);
}

// The per-wave tile areas and the wave-merge buffer: overlapping (the merge waits for every wave
// to leave its tile) or apart (SEP: the merge writes at once).
template <int KVE, bool SEP>
struct TileAreas {
    union {
        uint16_t kv[NW][KVE];
        float red_o[NW][16][RO_PITCH];
    };
};
template <int KVE>
struct TileAreas<KVE, true> {
    uint16_t kv[NW][KVE];
    float red_o[NW][16][RO_PITCH];
};

// KVE: bf16 elements of a wave's tile area (the V tile, or on bf16 global layers the larger K
// tile that passes through it first).
template <int KVE, bool SEP>
struct LdsDecode {
    float2 cs[NW][kMaxRopeHalf + 8];          // per wave: cos/sin of the position per frequency,
                                              // then the identity entries
    uint16_t Kn[NW][DQK];                     // per wave: the new token (bf16, or e4m3 codes in
    uint16_t Vn[NW][DV];                      // the first half), in the wave that owns its slot
    float red_m[NW][16], red_l[NW][16];
    float sink[16];
    TileAreas<KVE, SEP> u;                    // per-wave tile areas (the V tile in rows of
                                              // VT_PITCH, before it the K tile on global
                                              // layers) and the wave merge after the slot loop
};

// ROT: how many of a lane's 32-dim query chunk rows can hold rotated dims (2 when r <= 64).
// FP8: the caches hold e4m3 codes.
// EARLY: the first slot tile is requested before the position is known (always on sliding layers,
// whose ring slots are all in bounds; on global layers when the grid fits one round of resident
// workgroups, where every call is latency-bound: a split past a short sequence's position then
// fetches one tile it does not use, which a larger grid would pay for in bandwidth).
// ONE: a split holds at most one tile per wave (a sliding ring of up to 128 slots), so there is no
// slot loop and no refill: the kernel, fetched cold on every launch, is that much shorter.
template <bool SWA, bool SINK, bool SPLIT, int ROT, bool FP8, bool EARLY, bool ONE>
__global__ __launch_bounds__(256) void decode_bf16_kernel(const DecodeArgs a) {
    constexpr bool KLDS = !SWA;   // (global layers: keys through LDS, below)
    constexpr int KVE = (KLDS && !FP8) ? TILE * DQK : TILE * VT_PITCH;
    // sliding layers (latency-bound, few workgroups): the merge buffer apart from the tiles
    constexpr bool SEP = SWA;
    __shared__ __attribute__((aligned(16))) LdsDecode<KVE, SEP> sm;
    // Every argument the kernel reads is requested here, in one batch of scalar loads waited for
    // once: the compiler would otherwise fetch them in several dependent rounds as they come up.
    asm volatile("" ::"s"(a.q), "s"(a.k_new), "s"(a.v_new), "s"(a.positions), "s"(a.k_cache),
                 "s"(a.v_cache), "s"(a.sinks), "s"(a.out), "s"(a.partial));
    asm volatile("" ::"s"(a.Hq), "s"(a.Hkv), "s"(a.rope_dims), "s"(a.window), "s"(a.cap),
                 "s"(a.max_position), "s"(a.chunk), "s"(a.nsplit), "s"(a.k_inv), "s"(a.v_inv),
                 "s"(a.split_blocked), "s"(a.score_scale_log2), "s"(a.v_scale));
    using elem_t = std::conditional_t<FP8, uint8_t, uint16_t>;
    constexpr int EB = sizeof(elem_t);
    // K: 16-byte loads per lane per tile (two 16-slot blocks x 6 bf16 chunks of 8 dims, or
    // x 3 fp8 chunks of 16 dims; either way a load instruction reads 64 contiguous bytes of each
    // of 16 slots)
    constexpr int KREG = FP8 ? 2 * (DQK / 64) : 2 * (DQK / 32);
    constexpr int VPL = 16 / EB;                             // V elements per 16-byte load
    constexpr int VREG = TILE * DV / VPL / 64;               // V loads per lane per tile (8 or 4)
    constexpr int VCH = DV / VPL;                            // 16-byte chunks per V row

    // Work item.  A grid of more than one round of resident workgroups is laid out in blocks of
    // kDecodeSplitBlock consecutive splits of one (sequence, KV head) pair, the pairs in turn,
    // then the pairs' next block of splits (x = split within the block + block size * KV head,
    // y = sequence, z = block): the splits that hold keys for every sequence go out first and
    // the empty splits of short sequences last.  Interleaved among the long-running ones,
    // early-exiting workgroups leave the dispatcher's round-robin over the XCDs waiting on a full
    // XCD while others have free slots.  The blocks round the splits up; a split past the last
    // one starts at or past every sequence's key range and leaves at the empty-split check
    // below, having written nothing.  A grid that fits in one round keeps (split, KV head,
    // sequence).  (Selects and shifts only, no branch: this sits in front of every load.)
    const bool blk = a.split_blocked != 0;
    const int s = blk ? ((int)blockIdx.z << kDecodeSplitShift) + ((int)blockIdx.x & (kDecodeSplitBlock - 1))
                      : (int)blockIdx.x;
    const int g = blk ? (int)blockIdx.x >> kDecodeSplitShift : (int)blockIdx.y;
    const int b = blk ? (int)blockIdx.y : (int)blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, gq = lane >> 4;
    const int G = a.Hq / a.Hkv;
    const int k_begin = s * a.chunk;
    const int64_t cache_row0 = ((int64_t)b * a.Hkv + g) * a.cap;
    elem_t* const kc = (elem_t*)a.k_cache + cache_row0 * DQK;
    elem_t* const vc = (elem_t*)a.v_cache + cache_row0 * DV;

    // ---- slot loads into registers, one tile ahead of the one being computed, as buffer loads:
    //      one resource per cache slice, a per-lane byte offset computed once, the tile's slot in
    //      the scalar offset and the chunk in the immediate (no per-load address arithmetic).
    //      Slots at or past the capacity read zeros (the resource's bound); slots past the
    //      visible range and the new token's slot are fixed up when used.
    //      (byte sizes and offsets are unsigned 32-bit: the host keeps a cache slice below 4 GiB)
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)kc, (short)0, (int)((uint32_t)a.cap * (uint32_t)(DQK * EB)), kBufferFormat);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)vc, (short)0, (int)((uint32_t)a.cap * (uint32_t)(DV * EB)), kBufferFormat);
    const int k_lane = (l16 * DQK + (FP8 ? 16 : 8) * gq) * EB;
    // (V: lane holds row (lane + 64 it) / VCH of the tile, chunk (lane + 64 it) % VCH)
    const int v_lane = ((lane / VCH) * DV + (lane % VCH) * VPL) * EB;
    u32x4 kA[KREG], vA[VREG];
    // Global layers read each key tile as whole 1-KiB spans, non-temporally (every slot is read
    // once): load i of lane l holds 16-byte chunk 64 i + l of the tile (row (64 i + l) / KCPR,
    // chunk (64 i + l) % KCPR), and the tile passes through the wave's LDS tile area into operand
    // layout (KLDS).  Sliding layers load the operand layout straight from the ring (16 rows x
    // 64 bytes per instruction, ordinary loads: the ring is read again at the next step).
    constexpr int KPOL = SWA ? 0 : 2;
    constexpr int KCPR = DQK * EB / 16;                      // 16-byte chunks per key row
    // LDS position of chunk c of key row r: c ^ kswz(r), which keeps it within its row (bf16: 24
    // chunks, any 3-bit mask; fp8: 12 chunks, 2-bit masks) and spreads the operand reads of the
    // 16 rows over the banks
    auto kswz = [](int r) { return FP8 ? ((r >> 1) ^ (r >> 3)) & 3 : r & 7; };
    auto fetch = [&](u32x4 (&kr)[KREG], u32x4 (&vr)[VREG], int t0) {
        if constexpr (KLDS) {
#pragma unroll
            for (int i = 0; i < KREG; ++i)
                kr[i] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               krs, lane * 16, (int)((uint32_t)t0 * (DQK * EB) + i * 1024), KPOL));
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int c = 0; c < KREG / 2; ++c)
                    kr[kb * (KREG / 2) + c] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   krs, k_lane + 64 * c,
                                   (int)((uint32_t)(t0 + kb * 16) * (uint32_t)(DQK * EB)), KPOL));
            }
        }
        // (64 / VCH rows per instruction: it % 4 picks the row group within 16 rows on bf16;
        //  global layers read V non-temporally: whole rows per instruction, streamed once)
        constexpr int VPOL = SWA ? 0 : 2;
#pragma unroll
        for (int it = 0; it < VREG; ++it) {
            if constexpr (FP8)
                vr[it] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               vrs, v_lane, (int)((uint32_t)t0 * DV + it * (64 / VCH) * DV), VPOL));
            else
                vr[it] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               vrs, v_lane + (it & 3) * 4 * (DV * 2),
                               (int)((uint32_t)t0 * (DV * 2) + (it >> 2) * 16 * (DV * 2)), VPOL));
        }
    };
    // ---- every load that does not depend on the position goes out first, unconditionally (a
    //      load under a branch would be waited for at the branch's end): this lane's query chunks
    //      in B-operand layout (head l16 of the group, dims 32c + 8gq..; lanes past the group's
    //      heads read its last head, and those copies are never written out) with their rotation
    //      partners, the new token, the sinks, one frequency per thread and, on sliding layers, the
    //      first slot tile.
    const int r = a.rope_dims, half = r >> 1;
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + g * G + min(l16, G - 1)) * DQK;
    // Dims of MFMA k-chunk c held by lane group gq: 32c + 8gq.. for bf16 caches; for fp8 caches
    // 64(c/2) + 16gq + 8(c%2).., the order in which one 16-byte load of 16 key codes splits into
    // two chunks (the dot product does not depend on how its dims are ordered, as long as keys
    // and queries agree; chunks 0 and 1 still hold dims 0..63)
    auto qdim = [&](int c) { return FP8 ? 64 * (c >> 1) + 16 * gq + 8 * (c & 1) : 32 * c + 8 * gq; };
    u32x4 qraw[DQK / 32], qpar[ROT];
#pragma unroll
    for (int c = 0; c < DQK / 32; ++c) qraw[c] = *(const u32x4*)(qrow + qdim(c));
#pragma unroll
    for (int c = 0; c < ROT; ++c) {
        const int d0 = qdim(c);
        qpar[c] = *(const u32x4*)(qrow + (d0 < half ? d0 + half : (d0 < r ? d0 - half : d0)));
    }
    const int64_t kv_row = (int64_t)b * a.Hkv + g;
    const int nd0 = lane < DQK / 8 ? lane * 8 : 0;   // k_new dims of this lane (lane < 24)
    const uint16_t* nsrc = lane >= DQK / 8 && lane < DQK / 8 + DV / 8
                               ? a.v_new + kv_row * DV + (lane - DQK / 8) * 8
                               : a.k_new + kv_row * DQK + nd0;
    const u32x4 nraw = *(const u32x4*)nsrc;
    const u32x4 npar = *(const u32x4*)(a.k_new + kv_row * DQK +
                                       (nd0 < half ? nd0 + half : (nd0 < r ? nd0 - half : nd0)));
    const float sink_pre = (SINK && !SPLIT) ? a.sinks[g * G + min(tid & 15, G - 1)] : 0.0f;
    // (kernel arguments count as invariant memory, which the barrier below does not hold in place:
    //  read the frequencies, which sit in the argument segment, through a pointer the compiler
    //  cannot trace back to it)
    const char* kargs = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(kargs));
    const __attribute__((address_space(1))) double* om_args =
        (const __attribute__((address_space(1))) double*)(kargs + offsetof(DecodeArgs, omega_rev));
    const double om0 = om_args[lane], om1 = om_args[lane + 64];   // frequencies lane, lane + 64
    const int stride = NW * TILE;
    int t0 = k_begin + wave * TILE;
    if (EARLY) fetch(kA, vA, t0);
    // The position comes by a scalar load, counted apart from the vector loads (lgkmcnt, not
    // vmcnt): the work that needs only the position and the query (cos/sin table, query and
    // new-token rotation) runs while the slot tile is still in flight.  The load waits for its
    // own result in the same statement; the memory clobber keeps the loads above in place (the
    // compiler would otherwise sink each one next to its use, behind the position check).
    const int32_t pos = load_scalar_i32(a.positions + b);

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
    if (!EARLY) fetch(kA, vA, t0);

    // ---- cos/sin of the position per frequency, in this wave's table (read by this wave only)
    float2* const cs = sm.cs[wave];
    if (lane < half) {
        float c, sn;
        rope_cos_sin_rev(pos, om0, c, sn);
        cs[lane] = make_float2(c, sn);
    }
    if (lane + 64 < half) {
        float c, sn;
        rope_cos_sin_rev(pos, om1, c, sn);
        cs[lane + 64] = make_float2(c, sn);
    }
    if (lane < 8) cs[kIdentity + lane] = make_float2(1.0f, 0.0f);
    if (SINK && !SPLIT && tid < 16) sm.sink[tid] = sink_pre * kLog2e;   // (read after the merge barriers)
    __builtin_amdgcn_wave_barrier();

    // ---- this lane's rotated query chunks: the B operand of v_mfma_f32_16x16x32_bf16
    bf16x8 Qb[DQK / 32];
#pragma unroll
    for (int c = 0; c < DQK / 32; ++c)
        Qb[c] = as_bf16x8(c < ROT ? rotate8_cs(qraw[c], qpar[c], qdim(c), half, r, cs) : qraw[c]);
    // ---- the new token: rotate, keep in LDS, append to the cache, in the wave whose tiles hold
    //      its slot (wave w computes the tiles at k_begin + 32 w + 128 i).  An fp8 cache stores
    //      (and the tile loop reads) its codes.
    const bool own_new_w = own_new && wave == (((slot_new - k_begin) >> 5) & (NW - 1));
    elem_t* const Kn = (elem_t*)sm.Kn[wave];
    elem_t* const Vn = (elem_t*)sm.Vn[wave];
    if (own_new_w) {
        if (lane < DQK / 8) {
            if constexpr (FP8) {
                float x[8];
                rotate8_cs_f32(nraw, npar, nd0, half, r, cs, x);
                const u32x2 code = e4m3x8_from_f32(x, a.k_inv);
                *(u32x2*)(Kn + nd0) = code;
                *(u32x2*)(kc + (int64_t)slot_new * DQK + nd0) = code;
            } else {
                const u32x4 wv = rotate8_cs(nraw, npar, nd0, half, r, cs);
                *(u32x4*)(Kn + nd0) = wv;
                *(u32x4*)(kc + (int64_t)slot_new * DQK + nd0) = wv;
            }
        } else if (lane < DQK / 8 + DV / 8) {
            const int d0 = (lane - DQK / 8) * 8;
            if constexpr (FP8) {
                float x[8];
                unpack8(nraw, x);
                const u32x2 code = e4m3x8_from_f32(x, a.v_inv);
                *(u32x2*)(Vn + d0) = code;
                *(u32x2*)(vc + (int64_t)slot_new * DV + d0) = code;
            } else {
                *(u32x4*)(Vn + d0) = nraw;
                *(u32x4*)(vc + (int64_t)slot_new * DV + d0) = nraw;
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 O[DV / 16];
#pragma unroll
    for (int db = 0; db < DV / 16; ++db) O[db] = f32x4{};
    uint16_t* vt = sm.u.kv[wave];
    const float sc = a.score_scale_log2;

    // consume the tile held in (kr, vr) at slot t, refilling the registers with the next tile as
    // soon as the scores are formed
    auto consume = [&](u32x4 (&kr)[KREG], u32x4 (&vr)[VREG], int t) {
        if (own_new_w && slot_new >= t && slot_new < t + TILE) {
            if constexpr (KLDS) {
#pragma unroll
                for (int i = 0; i < KREG; ++i) {
                    const int P = 64 * i + lane;
                    if (t + P / KCPR == slot_new)
                        kr[i] = *(const u32x4*)((const uint8_t*)Kn + (P % KCPR) * 16);
                }
            } else {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    if (t + kb * 16 + l16 == slot_new) {
#pragma unroll
                        for (int c = 0; c < KREG / 2; ++c)
                            kr[kb * (KREG / 2) + c] =
                                *(const u32x4*)(Kn + (FP8 ? 16 : 8) * gq + (64 / EB) * c);
                    }
            }
#pragma unroll
            for (int it = 0; it < VREG; ++it) {
                const int e = lane + 64 * it;
                if (t + e / VCH == slot_new) vr[it] = *(const u32x4*)(Vn + (e % VCH) * VPL);
            }
        }
        // V rows -> this wave's LDS tile as bf16 (rows past the visible range as zeros)
        auto stage_v = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int it = 0; it < VREG; ++it) {
                const int e = lane + 64 * it;
                const int row = e / VCH;
                const bool live = t + row < k_end;
                uint16_t* dst = vt + row * VT_PITCH + (e % VCH) * VPL;
                if constexpr (FP8) {
                    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
                    *(u32x4*)dst = live ? bf16x8_from_e4m3x8(u32x2{vr[it][0], vr[it][1]}) : z;
                    *(u32x4*)(dst + 8) = live ? bf16x8_from_e4m3x8(u32x2{vr[it][2], vr[it][3]}) : z;
                } else {
                    *(u32x4*)dst = live ? vr[it] : u32x4{0u, 0u, 0u, 0u};
                }
            }
        };
        // S^T (16 slots x 16 heads) for the two 16-slot blocks of the tile
        f32x4 Sacc[2];
        __builtin_amdgcn_wave_barrier();
        if constexpr (KLDS) {
            // K chunks -> the wave's tile area (rows of DQK * EB bytes, chunk c of row r at
            // c ^ kswz(r)), then read back in operand layout (the chunks of every row cross
            // lanes); the area then takes the V tile (LDS operations of a wave run in order)
            uint8_t* const kt = (uint8_t*)vt;
#pragma unroll
            for (int i = 0; i < KREG; ++i) {
                const int P = 64 * i + lane, row = P / KCPR, ch = P % KCPR;
                *(u32x4*)(kt + row * (DQK * EB) + (ch ^ kswz(row)) * 16) = kr[i];
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4 acc = f32x4{};
                const int row = kb * 16 + l16;
                const uint8_t* krow = kt + row * (DQK * EB);
                if constexpr (FP8) {
                    // chunk 4 c2 + gq of the codes holds dims 64 c2 + 16 gq.. (two k-chunks)
#pragma unroll
                    for (int c2 = 0; c2 < DQK / 64; ++c2) {
                        const u32x4 w = *(const u32x4*)(krow + ((4 * c2 + gq) ^ kswz(row)) * 16);
                        acc = mfma16x16x32(as_bf16x8(bf16x8_from_e4m3x8(u32x2{w[0], w[1]})),
                                           Qb[2 * c2], acc);
                        acc = mfma16x16x32(as_bf16x8(bf16x8_from_e4m3x8(u32x2{w[2], w[3]})),
                                           Qb[2 * c2 + 1], acc);
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < DQK / 32; ++c)
                        acc = mfma16x16x32(*(const bf16x8*)(krow + ((4 * c + gq) ^ kswz(row)) * 16),
                                           Qb[c], acc);
                }
                Sacc[kb] = acc;
            }
            __builtin_amdgcn_wave_barrier();
            stage_v();
        } else {
            stage_v();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x4 acc = f32x4{};
#pragma unroll
                for (int c = 0; c < DQK / 32; ++c) {
                    u32x4 kw;
                    if constexpr (FP8) {
                        const u32x4& w = kr[kb * (KREG / 2) + (c >> 1)];
                        kw = bf16x8_from_e4m3x8((c & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]});
                    } else {
                        kw = kr[kb * (KREG / 2) + c];
                    }
                    acc = mfma16x16x32(as_bf16x8(kw), Qb[c], acc);
                }
                Sacc[kb] = acc;
            }
        }
        if (!ONE && t + stride < k_end) fetch(kr, vr, t + stride);

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
        mx = max_lane_pair32(max_lane_pair16(mx));
        // lazily raised reference maximum (per head): set by the head's first visible key, later
        // moved only when a tile exceeds it by more than 2^kRescaleLog2, so O is rarely rescaled
        // (the weights stay below 2^kRescaleLog2; numerator and denominator share the reference)
        const bool first = m_run == -INFINITY;
        const bool raise = first ? mx != -INFINITY : mx > m_run + kRescaleLog2;
        if (__any(raise)) {
            asm volatile("");   // (keep it a branch: rare after a wave's first tile)
            const float m_new = raise ? mx : m_run;
            if (__any(raise && !first)) {
                const float alpha = (raise && !first) ? fast_exp2(m_run - m_new) : 1.0f;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DV / 16; ++db) O[db] *= alpha;
            }
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
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
        l_run += psum;
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
    if constexpr (ONE) {
        if (t0 < k_end) consume(kA, vA, t0);
    } else {
        for (; t0 < k_end; t0 += stride) consume(kA, vA, t0);
    }

    // ---- merge the waves of the workgroup (red_o overlays the dead V tiles, or sits apart).
    l_run = sum_lane_pair32(sum_lane_pair16(l_run));
    if constexpr (!SEP) block_sync_lds();   // (every wave out of its tile before red_o overlays it)
    if (gq == 0) {
        sm.red_m[wave][l16] = m_run;
        sm.red_l[wave][l16] = l_run;
    }
#pragma unroll
    for (int db = 0; db < DV / 16; ++db)
        *(f32x4*)&sm.u.red_o[wave][l16][db * 16 + 4 * gq] = O[db];
    block_sync_lds();

    // one thread per (head, 4 dims): the head's wave weights once, then 4 outputs
    for (int e4 = tid; e4 < G * (DV / 4); e4 += 256) {
        const int hh = e4 / (DV / 4), d0 = (e4 % (DV / 4)) * 4;
        const int h = g * G + hh;
        float M = SINK && !SPLIT ? sm.sink[hh] : -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.red_m[w][hh]);
        const float Mu = (M == -INFINITY) ? 0.0f : M;
        float L = SINK && !SPLIT ? fast_exp2(sm.sink[hh] - Mu) : 0.0f;
        f32x4 acc = f32x4{};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = fast_exp2(sm.red_m[w][hh] - Mu);
            L += sm.red_l[w][hh] * f;
            acc += *(const f32x4*)&sm.u.red_o[w][hh][d0] * f;
        }
        if (SPLIT) {
            float* rec = a.partial + (((int64_t)b * a.Hq + h) * a.nsplit + s) * PSTRIDE;
            *(float2*)(rec + d0) = make_float2(acc[0], acc[1]);
            *(float2*)(rec + d0 + 2) = make_float2(acc[2], acc[3]);
            if (d0 == 0) *(float2*)(rec + DV) = make_float2(M, L);
        } else {
            const float sc_o = L > 0.0f ? a.v_scale / L : 0.0f;
            const u32x2 o2 = u32x2{pack_bf16x2(acc[0] * sc_o, acc[1] * sc_o),
                                   pack_bf16x2(acc[2] * sc_o, acc[3] * sc_o)};
            *(u32x2*)(a.out + ((int64_t)b * a.Hq + h) * DV + d0) = o2;
        }
    }
}

// Merge the splits of one (sequence, query head); the sink joins the denominator once, here.  One
// wave per (sequence, head), two output dims per lane (d and d + 64).  The position, the first
// 64 splits' (max, sum) and the first PRE records' values are requested together, before
// anything waits (records past the last split are read as the last one again): splits the
// position leaves empty never wrote their records, so those values are masked, never used.  The
// common maximum and the denominator are wave reductions; the weights go through LDS within the
// wave (no workgroup barrier) and each lane sums its dims in split order (PRE, the prefetch depth,
// is picked at launch from the split count; the sum is the same for any PRE).
template <bool SWA, bool SINK, bool VERIFY, int PRE>
__global__ __launch_bounds__(64) void decode_combine_kernel(const DecodeArgs a) {
    constexpr int CH = 16;
    __shared__ float w_s[1024];
    // (every argument read, requested in one batch of scalar loads)
    asm volatile("" ::"s"(a.partial), "s"(a.sinks), "s"(a.positions), "s"(a.out), "s"(a.Hq),
                 "s"(a.nsplit), "s"(a.q_per_seq), "s"(a.max_position), "s"(a.cap), "s"(a.window),
                 "s"(a.kpos_rel), "s"(a.kpos_off), "s"(a.chunk), "s"(a.v_scale));
    const int h = blockIdx.x, bq = blockIdx.y, lane = threadIdx.x;
    const int b = VERIFY ? bq / a.q_per_seq : bq;
    const int nsp = a.nsplit;
    const float* rec = a.partial + ((int64_t)bq * a.Hq + h) * nsp * PSTRIDE;
    float x0[PRE], x1[PRE];
#pragma unroll
    for (int i = 0; i < PRE; ++i) {
        const float* r = rec + (int64_t)min(i, nsp - 1) * PSTRIDE;
        x0[i] = r[lane];
        x1[i] = r[lane + 64];
    }
    const float* r0 = rec + (int64_t)min(lane, nsp - 1) * PSTRIDE;
    const float m0 = r0[DV], l0 = r0[DV + 1];
    const float sk = SINK ? a.sinks[h] * kLog2e : -INFINITY;
    const int32_t p_in = load_scalar_i32(a.positions + b);   // (also keeps the loads above first)
    uint16_t* o = a.out + ((int64_t)bq * a.Hq + h) * DV;
    const int32_t pos = VERIFY ? p_in + (bq - b * a.q_per_seq) : p_in;
    const bool pos_ok = VERIFY ? (p_in >= 0 && p_in <= a.max_position)
                               : (pos >= 0 && pos <= a.max_position && (SWA || pos < a.cap));
    if (!pos_ok) {
        o[lane] = 0;
        o[lane + 64] = 0;
        return;
    }
    // key rows the decode kernel's splits covered (the same count it used)
    const int n_valid = VERIFY ? pos - ((a.kpos_rel ? p_in : 0) + a.kpos_off) + 1
                               : (SWA ? min(a.window, pos + 1) : pos + 1);
    const int ns = min(nsp, (n_valid + a.chunk - 1) / a.chunk);   // splits that wrote a record
    float mx = lane < ns ? m0 : -INFINITY;
    for (int i = lane + 64; i < ns; i += 64) mx = fmaxf(mx, rec[(int64_t)i * PSTRIDE + DV]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float M = fmaxf(mx, sk);
    const float Mu = (M == -INFINITY) ? 0.0f : M;
    float ls = 0.0f;
    if (lane < ns) {
        const float w = fast_exp2(m0 - Mu);
        w_s[lane] = w;
        ls = w * l0;
    }
    for (int i = lane + 64; i < ns; i += 64) {
        const float w = fast_exp2(rec[(int64_t)i * PSTRIDE + DV] - Mu);
        w_s[i] = w;
        ls += w * rec[(int64_t)i * PSTRIDE + DV + 1];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ls += __shfl_xor(ls, off);
    const float L = ls + (SINK ? fast_exp2(sk - Mu) : 0.0f);
    __builtin_amdgcn_wave_barrier();   // (the weights in LDS: written and read by this wave only)
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int i = 0; i < PRE; ++i) {
        const float w = i < ns ? w_s[i] : 0.0f;
        acc0 += w * x0[i];
        acc1 += w * x1[i];
    }
    for (int s0 = PRE; s0 < ns; s0 += CH) {
        float y0[CH], y1[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const float* r = rec + (int64_t)min(s0 + i, ns - 1) * PSTRIDE;
            y0[i] = r[lane];
            y1[i] = r[lane + 64];
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const float w = s0 + i < ns ? w_s[s0 + i] : 0.0f;
            acc0 += w * y0[i];
            acc1 += w * y1[i];
        }
    }
    const float f = L > 0.0f ? a.v_scale / L : 0.0f;
    o[lane] = f32_to_bf16_bits(acc0 * f);
    o[lane + 64] = f32_to_bf16_bits(acc1 * f);
}

// The combine with the smallest prefetch depth that holds every split (at most 64; more splits
// are read in further chunks of 16).
template <bool SWA, bool SINK, bool VERIFY>
void launch_combine(const DecodeArgs& a, dim3 grid, hipStream_t st) {
    if (a.nsplit <= 16) decode_combine_kernel<SWA, SINK, VERIFY, 16><<<grid, 64, 0, st>>>(a);
    else if (a.nsplit <= 32) decode_combine_kernel<SWA, SINK, VERIFY, 32><<<grid, 64, 0, st>>>(a);
    else decode_combine_kernel<SWA, SINK, VERIFY, 64><<<grid, 64, 0, st>>>(a);
}

template <bool SWA, bool SINK, int ROT, bool FP8>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t st) {
    DecodeArgs k = a;
    k.split_blocked = a.nsplit >= kDecodeSplitBlock &&
                      (int64_t)a.B * a.Hkv * a.nsplit > kResidentDecodeGroups;
    const dim3 grid = k.split_blocked
                          ? dim3(a.Hkv * kDecodeSplitBlock, a.B,
                                 (a.nsplit + kDecodeSplitBlock - 1) / kDecodeSplitBlock)
                          : dim3(a.nsplit, a.Hkv, a.B);
    const bool early = SWA || (int64_t)a.B * a.Hkv * a.nsplit <= kResidentDecodeGroups;
    if (a.nsplit == 1) {
        if constexpr (SWA) {   // (rings of at most one tile per wave)
            if (a.chunk <= NW * TILE) {
                decode_bf16_kernel<SWA, SINK, false, ROT, FP8, true, true><<<grid, 256, 0, st>>>(k);
                return hipGetLastError();
            }
        }
        if (early) decode_bf16_kernel<SWA, SINK, false, ROT, FP8, true, false><<<grid, 256, 0, st>>>(k);
        else decode_bf16_kernel<SWA, SINK, false, ROT, FP8, false, false><<<grid, 256, 0, st>>>(k);
        return hipGetLastError();
    }
    if (early) decode_bf16_kernel<SWA, SINK, true, ROT, FP8, true, false><<<grid, 256, 0, st>>>(k);
    else decode_bf16_kernel<SWA, SINK, true, ROT, FP8, false, false><<<grid, 256, 0, st>>>(k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_combine<SWA, SINK, false>(a, dim3(a.Hq, a.B), st);
    return hipGetLastError();
}

}  // namespace

int decode_max_splits() { return 1024; }

template <bool FP8>
hipError_t launch_kind(const DecodeArgs& a, bool swa, bool sink, hipStream_t st) {
    if (a.rope_dims <= 64) {
        if (swa) return sink ? launch_typed<true, true, 2, FP8>(a, st) : launch_typed<true, false, 2, FP8>(a, st);
        return sink ? launch_typed<false, true, 2, FP8>(a, st) : launch_typed<false, false, 2, FP8>(a, st);
    }
    if (swa) return sink ? launch_typed<true, true, 6, FP8>(a, st) : launch_typed<true, false, 6, FP8>(a, st);
    return sink ? launch_typed<false, true, 6, FP8>(a, st) : launch_typed<false, false, 6, FP8>(a, st);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, bool swa, bool sink, hipStream_t st) {
    if (a.B == 0) return hipSuccess;
    if (a.nsplit > decode_max_splits()) return hipErrorInvalidConfiguration;
    return a.cache_fp8 ? launch_kind<true>(a, swa, sink, st) : launch_kind<false>(a, swa, sink, st);
}

hipError_t launch_verify_combine(const DecodeArgs& a, bool swa, bool sink, hipStream_t st) {
    const int64_t nq = (int64_t)a.B * a.q_per_seq;
    if (nq == 0 || a.nsplit <= 1) return hipSuccess;
    if (nq > 65535 || a.nsplit > decode_max_splits()) return hipErrorInvalidConfiguration;
    const dim3 grid(a.Hq, (unsigned)nq);
    if (swa) {
        if (sink) launch_combine<true, true, true>(a, grid, st);
        else launch_combine<true, false, true>(a, grid, st);
    } else {
        if (sink) launch_combine<false, true, true>(a, grid, st);
        else launch_combine<false, false, true>(a, grid, st);
    }
    return hipGetLastError();
}

}  // namespace mimo
