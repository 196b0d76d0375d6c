// probe.hip — latency references for the decode path and attainable ceilings of the chip
// (measurement aid, `libmimo_probe.so`).
//
// A decode call on a small batch is a chain that no bandwidth hides: the launch, one dependent
// read of each workgroup's key/value tile, a little arithmetic and the output store.  These two
// kernels time the floor of that chain with nothing of the layer in it, so the decode kernels can
// be stated against it (both graph-replayed the way a decode step runs):
//   * empty: every workgroup stores one word per thread (launch + completion);
//   * tile read: every workgroup reads its own contiguous slice of 4 KiB x NL with all of a
//     thread's 16-byte loads in flight at once, folds them and stores one word per thread.
// Two more kernels measure what the memory system and the matrix cores deliver to code of this
// kind, the attainable ceilings next to the nominal peaks (8 TB/s, 2.5 PFLOP/s dense bf16):
//   * stream read: a read of a buffer, consecutive lanes on consecutive 16 bytes, 8 loads in
//     flight per thread, the grid sweeping it together or each workgroup over a slice of its own,
//     with ordinary or non-temporal loads (nothing but one word per thread is written);
//   * MFMA loop: every wave runs 4 independent chains of v_mfma_f32_32x32x16_bf16 (the prefill
//     kernel's product) on register operands, no memory traffic in the loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mimo_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_empty_kernel(uint32_t* dst) {
    dst[blockIdx.x * 256 + threadIdx.x] = blockIdx.x;
}

template <int NL>
__global__ __launch_bounds__(256) void probe_tile_read_kernel(const u32x4* src, uint32_t* dst) {
    const u32x4* p = src + (int64_t)blockIdx.x * (NL * 256) + threadIdx.x;
    u32x4 w[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) w[i] = p[i * 256];
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < NL; ++i) acc ^= w[i][0] ^ w[i][1] ^ w[i][2] ^ w[i][3];
    dst[blockIdx.x * 256 + threadIdx.x] = acc;
}

// SLICE: each workgroup reads a contiguous slice of its own (n16 / gridDim.x units, 4 KiB per
// round of 256 threads); otherwise the whole grid sweeps the buffer together.
template <bool NT, bool SLICE>
__global__ __launch_bounds__(256) void probe_stream_read_kernel(const u32x4* src, int64_t n16,
                                                                uint32_t* dst) {
    const int64_t per = SLICE ? n16 / gridDim.x : n16;
    const int64_t stride = SLICE ? 256 : (int64_t)gridDim.x * 256;
    const u32x4* base = SLICE ? src + (int64_t)blockIdx.x * per : src;
    int64_t i = SLICE ? (int64_t)threadIdx.x : (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * stride < per; i += 8 * stride) {
        u32x4 w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            w[k] = NT ? __builtin_nontemporal_load(base + i + k * stride) : base[i + k * stride];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc ^= w[k][0] ^ w[k][1] ^ w[k][2] ^ w[k][3];
    }
    for (; i < per; i += stride) {
        const u32x4 w = base[i];
        acc ^= w[0] ^ w[1] ^ w[2] ^ w[3];
    }
    dst[blockIdx.x * 256 + threadIdx.x] = acc;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void probe_mfma_kernel(float* dst, int iters) {
    // operands from the thread index, so that nothing folds at compile time
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
        b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 7);
    }
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += c0[i] + c1[i] + c2[i] + c3[i];
    dst[blockIdx.x * 512 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

int mimo_probe_empty(void* dst, int32_t groups, void* stream) {
    if (!dst || groups < 1) return -1;
    probe_empty_kernel<<<groups, 256, 0, (hipStream_t)stream>>>((uint32_t*)dst);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mimo_probe_tile_read(const void* src, void* dst, int32_t groups, int32_t kib_per_group,
                         void* stream) {
    if (!src || !dst || groups < 1) return -1;
    const dim3 g(groups);
    hipStream_t st = (hipStream_t)stream;
    switch (kib_per_group) {
        case 20: probe_tile_read_kernel<5><<<g, 256, 0, st>>>((const u32x4*)src, (uint32_t*)dst); break;
        case 40: probe_tile_read_kernel<10><<<g, 256, 0, st>>>((const u32x4*)src, (uint32_t*)dst); break;
        case 80: probe_tile_read_kernel<20><<<g, 256, 0, st>>>((const u32x4*)src, (uint32_t*)dst); break;
        default: return -2;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mimo_probe_stream_read(const void* src, int64_t bytes, int32_t flags, void* dst,
                           int32_t groups, void* stream) {
    if (!src || !dst || groups < 1) return -1;
    if (bytes < 16 || bytes % 16) return -2;
    const bool slice = (flags & 2) != 0;
    if (slice && bytes % ((int64_t)groups * 4096)) return -2;
    hipStream_t st = (hipStream_t)stream;
    const u32x4* s = (const u32x4*)src;
    uint32_t* d = (uint32_t*)dst;
    const int64_t n16 = bytes / 16;
    switch (flags & 3) {
        case 0: probe_stream_read_kernel<false, false><<<groups, 256, 0, st>>>(s, n16, d); break;
        case 1: probe_stream_read_kernel<true, false><<<groups, 256, 0, st>>>(s, n16, d); break;
        case 2: probe_stream_read_kernel<false, true><<<groups, 256, 0, st>>>(s, n16, d); break;
        default: probe_stream_read_kernel<true, true><<<groups, 256, 0, st>>>(s, n16, d); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int mimo_probe_mfma(void* dst, int32_t groups, int32_t iters, void* stream) {
    if (!dst || groups < 1) return -1;
    if (iters < 1) return -2;
    probe_mfma_kernel<<<groups, 512, 0, (hipStream_t)stream>>>((float*)dst, iters);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
