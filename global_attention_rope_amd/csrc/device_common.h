// device_common.h — types and small device helpers shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mimo {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Largest rotated width the kernels accept (frequencies are passed by value in kernel args).
constexpr int kMaxRopeHalf = 128;

// cos/sin of the RoPE angle pos * omega, with the frequency given in revolutions
// (w_rev = omega / 2pi).  The product is formed and reduced to [0, 1) revolutions exactly enough
// in fp64 (positions reach tens of thousands of radians), then evaluated by the hardware sine and
// cosine, which take revolutions (max abs error 1.3e-7 over [0, 1) measured on gfx950).
__device__ __forceinline__ void rope_cos_sin_rev(int32_t pos, double w_rev, float& c, float& s) {
    const double x = (double)pos * w_rev;
    const float xf = (float)(x - floor(x));
    s = __builtin_amdgcn_sinf(xf);
    c = __builtin_amdgcn_cosf(xf);
}

// Workgroup barrier for LDS traffic only: every wave's LDS accesses have completed, nothing else
// is waited for.  (__syncthreads also releases global memory, which on gfx950 waits for every
// outstanding global load and store of the wave.)
__device__ __forceinline__ void block_sync_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane.  Issued as
// inline asm so that the compiler does not track these LDS writes: it would otherwise wait for
// every outstanding load before each transposed LDS read.  Completion is ordered explicitly with
// wait_vmcnt + block_sync_lds; the instruction has no register results.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_base)
                 : "memory", "m0");
}

// The same with a non-temporal load, for rows streamed once (a whole 1-KiB span per instruction).
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds_base)
                 : "memory", "m0");
}

// The same from a workgroup-uniform base plus a per-lane 32-bit byte offset (the base in scalar
// registers, so that per-tile address arithmetic stays scalar).
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t offset, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(offset), "s"(base),
                 "s"(lds_base)
                 : "memory", "m0");
}

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format, no swizzle).
constexpr int kBufferFormat = 0x00020000;

// 32-bit load of a workgroup-uniform address through the scalar cache, waited for in the same
// statement (its counter is the scalar one, so vector loads issued before it stay in flight).
// The memory clobber also keeps every earlier load ahead of it.
// (The address goes through readfirstlane, which is free for a value already in scalar registers
//  and keeps the operand a scalar register pair wherever the compiler is unsure of uniformity.)
__device__ __forceinline__ int32_t load_scalar_i32(const int32_t* p) {
    const uint64_t u = (uint64_t)(uintptr_t)p;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    const int32_t* ps = (const int32_t*)(uintptr_t)(lo | (hi << 32));
    int32_t v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ps) : "memory");
    return v;
}

// Maximum of x over the lane pair (l, l ^ 32), in registers (no LDS round trip).
__device__ __forceinline__ float max_lane_pair32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum of x over the lane pair (l, l ^ 16), in registers.
__device__ __forceinline__ float max_lane_pair16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum of x over the lane pair (l, l ^ 16).
__device__ __forceinline__ float sum_lane_pair16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum of x over the lane pair (l, l ^ 32).
__device__ __forceinline__ float sum_lane_pair32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x by the hardware exponential (softmax weights; x <= 0 here).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// Unpack 8 bf16 held in a 16-byte word into fp32.
__device__ __forceinline__ void unpack8(const u32x4& w, float* f) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f[2 * t] = __uint_as_float(w[t] << 16);
        f[2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
    }
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
    u32x4 w;
#pragma unroll
    for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(f[2 * t], f[2 * t + 1]);
    return w;
}

// fp8 KV cache elements: OCP e4m3 codes (the format of gfx950's fp8 conversions).
// Eight fp32 values times inv, clamped to +-448 (saturation instead of NaN), to their nearest
// codes (ties to even), packed low byte first.
__device__ __forceinline__ u32x2 e4m3x8_from_f32(const float* x, float inv) {
    u32x2 w;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) y[t] = fminf(fmaxf(x[4 * h + t] * inv, -448.0f), 448.0f);
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], v, true);
        w[h] = (uint32_t)v;
    }
    return w;
}

// Eight e4m3 codes (low byte first) to their exact bf16 values.
__device__ __forceinline__ u32x4 bf16x8_from_e4m3x8(const u32x2& w) {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        r[2 * h] = __builtin_bit_cast(uint32_t,
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, false));
        r[2 * h + 1] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.0f, true));
    }
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) {
    return __builtin_bit_cast(bf16x8, w);
}

// D = A(32x16) * B(16x32) + C, bf16 operands, fp32 accumulate.
//   A: lane l holds row (l % 32), k = 8 * (l / 32) + [0, 8).
//   B: lane l holds column (l % 32), k = 8 * (l / 32) + [0, 8).
//   C/D: lane l holds column (l % 32), rows 8 * (i / 4) + 4 * (l / 32) + (i % 4), i in [0, 16).
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A(16x32) * B(32x16) + C, bf16 operands, fp32 accumulate.
//   A: lane l holds row (l % 16), k = 8 * (l / 16) + [0, 8).
//   B: lane l holds column (l % 16), k = 8 * (l / 16) + [0, 8).
//   C/D: lane l holds column (l % 16), rows 4 * (l / 16) + i, i in [0, 4).
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace mimo
