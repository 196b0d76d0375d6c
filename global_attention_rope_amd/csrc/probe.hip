// probe.hip — latency references for the decode path (measurement aid, `libmimo_probe.so`).
//
// A decode call on a small batch is a chain that no bandwidth hides: the launch, one dependent
// read of each workgroup's key/value tile, a little arithmetic and the output store.  These two
// kernels time the floor of that chain with nothing of the layer in it, so the decode kernels can
// be stated against it (both graph-replayed the way a decode step runs):
//   * empty: every workgroup stores one word per thread (launch + completion);
//   * tile read: every workgroup reads its own contiguous slice of 4 KiB x NL with all of a
//     thread's 16-byte loads in flight at once, folds them and stores one word per thread.
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

}  // extern "C"
