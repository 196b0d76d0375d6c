// kernels.h — argument blocks and launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mimo {

constexpr int kMaxRopeHalfArgs = 128;  // r/2 frequencies passed by value, in revolutions
// Decode workgroups resident on the chip at once: 256 CUs x two 4-wave workgroups (their registers
// allow two per CU).
constexpr int64_t kResidentDecodeGroups = 512;

// Rotate K (first rope_dims dims) once per token i in [i0, S) of each sequence b (position
// start_pos[b] + i) and store it
//   * into k_ws [B,Hkv,ws_rows,dqk] at row ws_row0 + i (ws_rel: start_pos[b] + ws_row0 + i), when
//     k_ws is set (rotated-K scratch of a prefill), and V likewise into v_ws [B,Hkv,ws_rows,dv]
//     when v_ws is set;
//   * with V into the cache k_dst [B,Hkv,cap,dqk] / v_dst [B,Hkv,cap,dv], when k_dst is set and
//     i >= cache_i0, at slot position % ring_window (ring_window > 0) or slot position (linear; a
//     token whose slot falls outside [0, cap) is not stored).
// With max_start >= 0, sequences whose start_pos lies outside [0, max_start] are skipped.
struct RopeKVArgs {
    const void* k;       // [B,S,Hkv,dqk]
    const void* v;       // [B,S,Hkv,dv]
    const int32_t* start_pos;
    void* k_ws;          // [B,Hkv,ws_rows,dqk] or null
    void* v_ws;          // [B,Hkv,ws_rows,dv] or null
    void* k_dst;         // [B,Hkv,cap,dqk] or null
    void* v_dst;         // [B,Hkv,cap,dv], set iff k_dst is
    int32_t B, S, Hkv, dqk, dv, rope_dims, cap, i0, cache_i0, ring_window;
    int32_t ws_rows, ws_row0, ws_rel, max_start;
    int32_t cache_fp8;   // caches hold e4m3 codes of x * k_inv / v_inv (bf16 kernel only)
    float k_inv, v_inv;
    double omega_rev[kMaxRopeHalfArgs];  // theta^(-2d/r) / (2 pi)
};

// Copy the cached positions before start_pos[b] that an extend reads into bf16 workspace rows in
// position order, row r of [B,Hkv,ws_rows,d]:
//   * ring (W > 0; cap == W): the W most recent positions, row r holding position
//     start_pos[b] - W + r (slot position % W); rows of negative positions are left as they are;
//   * linear (W == 0): row j holding position j (slot j) for j < min(start_pos[b], rows).
// fp8 caches (cache_fp8) are widened on the way: row element = bf16(e4m3(code) * scale).  With
// max_start >= 0, sequences whose start_pos lies outside [0, max_start] are skipped.
struct CacheRowsArgs {
    const void* k_cache;       // [B,Hkv,cap,dqk] bf16, or e4m3 codes
    const void* v_cache;       // [B,Hkv,cap,dv]
    const int32_t* start_pos;
    uint16_t* k_ws;            // [B,Hkv,ws_rows,dqk]
    uint16_t* v_ws;            // [B,Hkv,ws_rows,dv]
    int32_t B, Hkv, dqk, dv, W, cap, rows, ws_rows, max_start;
    int32_t cache_fp8;
    float k_scale, v_scale;
};

// bf16 prefill.  Query row i of sequence b sits at position start_pos[b] + i.  Key row j (rotated
// K at k + b*k_sb + g*k_sh + j*k_sj, V at v + b*v_sb + g*v_sh + j*v_sj; element strides, rows
// contiguous: k_sj == 192) sits at position kpos0 = (kpos_rel ? start_pos[b] : 0) + kpos_off,
// plus j; key rows run up to the last query's position, and rows of negative positions hold no
// token.  With max_start >= 0, a sequence whose start_pos lies outside [0, max_start] gets a
// zero output.
struct PrefillArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* start_pos;
    const float* sinks;
    uint16_t* out;
    int64_t k_sb, k_sh, k_sj;
    int64_t v_sb, v_sh, v_sj;
    int32_t kpos_rel, kpos_off, max_start;
    int32_t B, S, Hq, Hkv, rope_dims, window;
    float score_scale_log2;
    float v_scale;
    double omega_rev[kMaxRopeHalfArgs];  // theta^(-2d/r) / (2 pi)
};

// bf16 decode (split-K over cache slots).
struct DecodeArgs {
    const uint16_t* q;       // [B,Hq,192]
    const uint16_t* k_new;   // [B,Hkv,192]
    const uint16_t* v_new;   // [B,Hkv,128]
    const int32_t* positions;
    void* k_cache;           // [B,Hkv,cap,192] bf16, or e4m3 codes (cache_fp8)
    void* v_cache;           // [B,Hkv,cap,128] bf16, or e4m3 codes (cache_fp8)
    const float* sinks;
    uint16_t* out;           // [B,Hq,128]
    float* partial;          // [B,Hq,nsplit,130] (split mode)
    int32_t B, Hq, Hkv, rope_dims, window, cap, max_position, chunk, nsplit;
    int32_t cache_fp8;       // caches hold e4m3 codes: the new token is coded with k_inv/v_inv;
    float k_inv, v_inv;      // the code scales are folded into score_scale_log2 and v_scale
    // Combine of multi-token partials: out/partials hold q_per_seq tokens per sequence
    // ([B * T, Hq, d]); positions holds each sequence's first token position st; token t sits at
    // st + t and saw key rows up to its own, row j sitting at position
    // (kpos_rel ? st : 0) + kpos_off + j; sequences with st outside [0, max_position] get zeros.
    int32_t q_per_seq, kpos_rel, kpos_off;
    // decode grid layout (set by the launch): 0 = (split, KV head, sequence); 1 = blocks of
    // consecutive splits of a pair, the pairs in turn, then the next block
    int32_t split_blocked;
    float score_scale_log2;
    float v_scale;
    double omega_rev[kMaxRopeHalfArgs];  // theta^(-2d/r) / (2 pi)
};

// fp32 vector-ALU kernels for small head dims (dqk, dv <= 256).
struct F32PrefillArgs {
    const float* q;
    const float* k;
    const float* v;
    const int32_t* start_pos;
    const float* sinks;
    float* out;
    int32_t B, S, Hq, Hkv, dqk, dv, rope_dims, window, layer_kind;
    float score_scale;
    float v_scale;
    double omega_rev[kMaxRopeHalfArgs];  // theta^(-2d/r) / (2 pi)
};

struct F32DecodeArgs {
    const float* q;
    const float* k_new;
    const float* v_new;
    const int32_t* positions;
    float* k_cache;
    float* v_cache;
    const float* sinks;
    float* out;
    int32_t B, Hq, Hkv, dqk, dv, rope_dims, window, layer_kind, cap, max_position;
    float score_scale;
    float v_scale;
    double omega_rev[kMaxRopeHalfArgs];  // theta^(-2d/r) / (2 pi)
};

// bf16 dense products C_p = alpha * A[M, K] B_p[K, N_p] (row-major, fp32 accumulation,
// K % 64 == 0, N_p % 8 == 0) for up to three parts p sharing A, in one launch, each with one of
// three epilogues:
//   kGemmPlain: C_p [M, ldc] row-major;
//   kGemmKey:   rows are tokens (row m = b * S + s, position start_pos[b] + s), columns
//               heads * dqk; the leading rope_dims (0 or 64) dims of each head are rotated
//               (pairs (d, d + 32), frequencies omega_rev[d] in revolutions) and the result is
//               stored in the attention's [B, heads, S, dqk] layout at C_p, and into the part's
//               cache ([B, heads, cap, dqk]) when set, for tokens s >= cache_i0, at slot
//               position % ring_window (ring_window > 0) or position (slot < cap);
//   kGemmValue: C_p [M, ldc] row-major, columns heads * dv, plus the cache store as for keys.
// cache_fp8: caches hold e4m3 codes of value * code_inv (keys: the fp32 rotated value; values:
// their bf16 rounding), saturated at +-448.
enum { kGemmPlain = 0, kGemmKey = 1, kGemmValue = 2 };
struct GemmPart {
    const uint16_t* B;
    uint16_t* C;
    void* cache;
    int64_t ldb, ldc;
    int32_t N, epilogue;
    int32_t tiles;       // set by the launch
    float code_inv;
};
struct GemmArgs {
    const uint16_t* A;
    int64_t lda;
    int32_t M, K;
    float alpha;
    int32_t nparts;
    GemmPart part[3];
    // key / value epilogues
    int32_t S, heads, dqk, dv;
    const int32_t* start_pos;
    int32_t cap, ring_window, cache_i0, cache_fp8;
    int32_t rope_dims;
    double omega_rev[32];   // theta^(-2d/r) / (2 pi), d < 32 (rope_dims == 64)
};
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st);

hipError_t launch_rope_kv_bf16(const RopeKVArgs& a, hipStream_t st);
hipError_t launch_cache_rows_bf16(const CacheRowsArgs& a, hipStream_t st);
hipError_t launch_rope_kv_f32(const RopeKVArgs& a, hipStream_t st);
hipError_t launch_prefill_bf16(const PrefillArgs& a, bool window, bool sink, hipStream_t st);
hipError_t launch_decode_bf16(const DecodeArgs& a, bool swa, bool sink, hipStream_t st);
hipError_t launch_prefill_f32(const F32PrefillArgs& a, hipStream_t st);
hipError_t launch_decode_f32(const F32DecodeArgs& a, hipStream_t st);

// Query rows per prefill workgroup (bf16 kernel) for a sliding-window or global layer.
int prefill_bf16_block_rows(bool window);

// Largest number of decode splits per sequence the combine kernel merges.
int decode_max_splits();

// Frequencies of the rotated slice in revolutions per position, theta^(-2d/r) / (2 pi) for
// d < r/2 and 0 up to n.
void rope_omega_rev(double theta, int rope_dims, double* out, int n);

// The library's thread-local error message (mimo_attn_last_error): set it and return code.
int set_error(int code, const char* msg);
void clear_error();

}  // namespace mimo
