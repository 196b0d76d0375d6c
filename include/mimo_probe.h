/*
 * mimo_probe.h — latency references of `libmimo_probe.so`, a measurement aid beside
 * `libmimo_attn.so` (not part of the layer's path).  The decode of a small batch is bound by the
 * latency of one dependent chain per workgroup (launch, one tile read, store); these kernels time
 * that chain with nothing else in it, so that a decode kernel's time can be stated against it.
 *
 * Both enqueue one kernel of `groups` workgroups of 256 threads on `stream` (a hipStream_t; NULL =
 * the default stream) and return 0, -1 for a NULL pointer or groups < 1, -2 for an unsupported
 * slice size, -4 when the launch fails.  Buffers are caller-owned device memory.
 */
#ifndef MIMO_PROBE_H
#define MIMO_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroup g stores one 32-bit word per thread at dst[g * 256 + thread] (dst: groups * 1 KiB). */
int mimo_probe_empty(void* dst, int32_t groups, void* stream);

/* Workgroup g reads bytes [g * S, (g + 1) * S) of src, S = kib_per_group KiB (20, 40 or 80), every
 * thread's 16-byte loads in flight at once, and stores one word per thread at dst[g * 256 + thread]
 * (src: groups * S bytes; dst: groups * 1 KiB). */
int mimo_probe_tile_read(const void* src, void* dst, int32_t groups, int32_t kib_per_group,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MIMO_PROBE_H */
