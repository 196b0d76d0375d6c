// verify.h — multi-token extend kernels (a few new tokens per sequence against its key rows):
// argument block and launchers (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace mimo {

// Every query head of a KV group times every new token of a sequence forms one column block
// of the tile kernel: column c = head * TP + token (TP: T rounded up to a power of two).
// q [B,T,Hq,192]; key rows of (b, g): K at k + b*k_sb + g*k_sh + j*192, V at v + b*v_sb + g*v_sh +
// j*128; row j sits at position (kpos_rel ? st : 0) + kpos_off + j with st = start_pos[b]; token
// t at st + t; rows of negative positions hold no token.  Splits of `chunk` rows (a multiple of
// 64) write (O, m, l) partials [B*T, Hq, nsplit, 130] merged by the combine kernel; one split
// writes out [B,T,Hq,128] directly.  Sequences with st outside [0, max_start] get a zero output.
struct VerifyArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* start_pos;
    const float* sinks;
    uint16_t* out;
    float* partial;
    // optional ring cache [B,Hkv,ring_w,d]: key rows j < ring_w are read from it at slot
    // (position of row j) % ring_w instead of from k/v
    const uint16_t* ring_k;
    const uint16_t* ring_v;
    int32_t ring_w;
    int64_t k_sb, k_sh, v_sb, v_sh;
    // fp8 caches read in place (global layers, key rows = positions): rows j < start_pos[b] are
    // e4m3 codes at slot j of code_k [B,Hkv,code_cap,192] / code_v [B,Hkv,code_cap,128], taken
    // as bf16(e4m3(code) * scale); rows start_pos[b] + t are the new tokens, row t of k / v
    const uint8_t* code_k;
    const uint8_t* code_v;
    int32_t code_cap;
    float code_k_scale, code_v_scale;
    int32_t B, T, TP, Hq, Hkv, rope_dims, window, kpos_rel, kpos_off, max_start, chunk, nsplit;
    float score_scale_log2;
    float v_scale;
    double omega_rev[kMaxRopeHalfArgs];  // theta^(-2d/r) / (2 pi)
};

// Column waves (32 query columns each) of the tile kernel for G query heads per KV head and TP
// token columns; 0 beyond 256 columns.
int verify_tile_waves(int G, int TP);

hipError_t launch_verify_tiles_bf16(const VerifyArgs& a, bool window, bool sink, hipStream_t st);

// The decode combine kernel in its multi-token mode over the partials of the tile kernel.
hipError_t launch_verify_combine(const DecodeArgs& a, bool swa, bool sink, hipStream_t st);

}  // namespace mimo
