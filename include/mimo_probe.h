/*
 * mimo_probe.h — latency references and attainable ceilings of `libmimo_probe.so`, a measurement
 * aid beside `libmimo_attn.so` (not part of the layer's path).  The decode of a small batch is
 * bound by the latency of one dependent chain per workgroup (launch, one tile read, store); the
 * first two kernels time that chain with nothing else in it, so that a decode kernel's time can be
 * stated against it.  The last two measure the read bandwidth and the dense bf16 matrix rate that
 * code of this kind attains, beside the nominal peaks.
 *
 * Each enqueues one kernel of `groups` workgroups on `stream` (a hipStream_t; NULL = the default
 * stream) and returns 0, -1 for a NULL pointer or groups < 1, -2 for an unsupported size, -4 when
 * the launch fails.  Buffers are caller-owned device memory.
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

/* Read-only stream of bytes [0, bytes) of src (bytes a positive multiple of 16) in 16-byte loads,
 * consecutive lanes on consecutive addresses, 8 loads in flight per thread.  flags bit 0:
 * non-temporal loads; bit 1: workgroup g reads its own contiguous slice [g * bytes / groups,
 * (g + 1) * bytes / groups) (bytes then a multiple of groups * 4096), else the grid sweeps the
 * buffer together (grid-stride).  Stores one 32-bit word per thread at dst[g * 256 + thread]
 * (dst: groups * 1 KiB).  Returns -2 for a bad size. */
int mimo_probe_stream_read(const void* src, int64_t bytes, int32_t flags, void* dst,
                           int32_t groups, void* stream);

/* MFMA loop: `groups` workgroups of 8 waves (512 threads); every wave runs `iters` rounds of 4
 * independent v_mfma_f32_32x32x16_bf16 (32768 flop each) on register operands, then stores one
 * float per thread at dst[g * 512 + thread] (dst: groups * 2 KiB).  Flop per launch:
 * groups * 8 * iters * 4 * 32768.  Returns -2 for iters < 1. */
int mimo_probe_mfma(void* dst, int32_t groups, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MIMO_PROBE_H */
