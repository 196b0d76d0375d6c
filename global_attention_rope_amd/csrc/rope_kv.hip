// rope_kv.hip — rotate keys once and store them (and V) in cache-layout buffers [B, Hkv, n, d].
//
// Partial RoPE (pages: "Add Xiaomi MiMo-V2", "Additional useful info": the leading third of the
// head dim is rotated; "add Xiaomi MiMo v2 (mimo_v2_flash)", "Architecture, verified against
// upstream": rotated width int(partial_rotary_factor * head_dim), per-kind theta): pair
// (d, d + r/2), d < r/2, is turned by position * theta^(-2d/r); dims >= r are copied.
// Destinations: the rotated-K (and V) scratch of a prefill or an extend (row = a fixed offset +
// token index, or + position), the linear cache of global layers (slot = position) and the
// rotating cache of sliding layers (slot = position % window; "add Xiaomi MiMo v2
// (mimo_v2_flash)", "Implementation plan").  The cache-rows pass lays out by position the cached
// rows an extend reads in front of its new tokens (the ring's content; an fp8 cache's rows,
// widened to bf16).
#include "device_common.h"
#include "kernels.h"

namespace mimo {
namespace {

// Cache slot of token i at position pos, or -1 when it is not stored.
__device__ __forceinline__ int cache_slot(const RopeKVArgs& a, int i, int32_t pos) {
    if (!a.k_dst || pos < 0 || i < a.cache_i0) return -1;
    if (a.ring_window > 0) return pos % a.ring_window;
    return pos < a.cap ? pos : -1;
}

// Sequence b takes part (its start lies in the accepted range, when one is given).
__device__ __forceinline__ bool start_ok(int32_t start, int32_t max_start) {
    return max_start < 0 || (unsigned)start <= (unsigned)max_start;
}

// First token whose values are written: every token when a value workspace is given, else the
// tokens that get a cache slot (a ring keeps the last W), else none.
__host__ __device__ inline int rope_v_first(const RopeKVArgs& a) {
    if (a.v_ws) return a.i0;
    if (a.k_dst) {
        const int f = a.i0 > a.cache_i0 ? a.i0 : a.cache_i0;
        return f < a.S ? f : a.S;
    }
    return a.S;
}

// bf16: one thread per 8-element chunk of a K or V row, over a group of HG KV heads of one token
// (HG divides Hkv): the angles of a rotated chunk are evaluated once for the whole group.  The
// K chunks of every token come first, then the V chunks of the tokens whose values are written
// (on a sliding layer's prefill only the last W tokens), so that no thread idles on a value row
// nobody stores.
template <int HG>
__global__ __launch_bounds__(256) void rope_kv_bf16_kernel(const RopeKVArgs a) {
    const int kch = a.dqk / 8, vch = a.dv / 8;
    const int ntok = a.S - a.i0, ngrp = a.Hkv / HG;
    const int iv0 = rope_v_first(a), ntv = a.S - iv0;
    const int64_t total_k = (int64_t)a.B * ntok * ngrp * kch;
    const int64_t total = total_k + (int64_t)a.B * ntv * ngrp * vch;
    const int r = a.rope_dims, half = r >> 1;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const bool isk = e < total_k;
        const int64_t ev = isk ? e : e - total_k;
        const int per = isk ? kch : vch, nt = isk ? ntok : ntv;
        const int c = (int)(ev % per) + (isk ? 0 : kch);
        const int64_t grpid = ev / per;
        const int g0 = (int)(grpid % ngrp) * HG;
        const int64_t tok = grpid / ngrp;            // b * nt + (i - first token)
        const int i = (isk ? a.i0 : iv0) + (int)(tok % nt);
        const int b = (int)(tok / nt);
        const int32_t start = a.start_pos[b];
        if (!start_ok(start, a.max_start)) continue;
        const int32_t pos = start + i;
        const int slot = cache_slot(a, i, pos);
        const int64_t src0 = ((int64_t)b * a.S + i) * a.Hkv + g0;     // source row of head g0
        const int64_t bg0 = (int64_t)b * a.Hkv + g0;                  // [b, g0] of a [B, Hkv, n, d]
        const int64_t ws_r = (a.ws_rel ? start : 0) + a.ws_row0 + i;
        if (c < kch) {
            const int d0 = c * 8;
            const bool rot = d0 < r, lower = d0 < half;
            const int pd = lower ? d0 + half : d0 - half;
            float cs[8], sn[8];
            if (rot) {
                const int f0 = lower ? d0 : d0 - half;
#pragma unroll
                for (int t = 0; t < 8; ++t) rope_cos_sin_rev(pos, a.omega_rev[f0 + t], cs[t], sn[t]);
            }
#pragma unroll
            for (int j = 0; j < HG; ++j) {
                const uint16_t* krow = (const uint16_t*)a.k + (src0 + j) * a.dqk;
                u32x4 w = *(const u32x4*)(krow + d0);
                float x[8];
                unpack8(w, x);
                if (rot) {
                    float y[8];
                    unpack8(*(const u32x4*)(krow + pd), y);
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        x[t] = lower ? (x[t] * cs[t] - y[t] * sn[t]) : (x[t] * cs[t] + y[t] * sn[t]);
                    w = pack8(x);
                }
                if (a.k_ws) *(u32x4*)((uint16_t*)a.k_ws + ((bg0 + j) * a.ws_rows + ws_r) * a.dqk + d0) = w;
                if (slot >= 0) {
                    const int64_t slot_row = (bg0 + j) * a.cap + slot;
                    // (an fp8 cache codes the fp32 rotated key, not its bf16 rounding)
                    if (a.cache_fp8)
                        *(u32x2*)((uint8_t*)a.k_dst + slot_row * a.dqk + d0) = e4m3x8_from_f32(x, a.k_inv);
                    else
                        *(u32x4*)((uint16_t*)a.k_dst + slot_row * a.dqk + d0) = w;
                }
            }
        } else if (slot >= 0 || a.v_ws) {
            const int d0 = (c - kch) * 8;
#pragma unroll
            for (int j = 0; j < HG; ++j) {
                const u32x4 w = *(const u32x4*)((const uint16_t*)a.v + (src0 + j) * a.dv + d0);
                if (a.v_ws) *(u32x4*)((uint16_t*)a.v_ws + ((bg0 + j) * a.ws_rows + ws_r) * a.dv + d0) = w;
                if (slot >= 0) {
                    const int64_t slot_row = (bg0 + j) * a.cap + slot;
                    if (a.cache_fp8) {
                        float x[8];
                        unpack8(w, x);
                        *(u32x2*)((uint8_t*)a.v_dst + slot_row * a.dv + d0) = e4m3x8_from_f32(x, a.v_inv);
                    } else {
                        *(u32x4*)((uint16_t*)a.v_dst + slot_row * a.dv + d0) = w;
                    }
                }
            }
        }
    }
}

// fp32: one thread per element.
__global__ __launch_bounds__(256) void rope_kv_f32_kernel(const RopeKVArgs a) {
    const int per_row = a.dqk + ((a.k_dst || a.v_ws) ? a.dv : 0);
    const int ntok = a.S - a.i0;
    const int64_t total = (int64_t)a.B * ntok * a.Hkv * per_row;
    const int r = a.rope_dims, half = r >> 1;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(e % per_row);
        const int64_t rowid = e / per_row;
        const int g = (int)(rowid % a.Hkv);
        const int i = a.i0 + (int)((rowid / a.Hkv) % ntok);
        const int b = (int)(rowid / ((int64_t)a.Hkv * ntok));
        const int32_t start = a.start_pos[b];
        if (!start_ok(start, a.max_start)) continue;
        const int32_t pos = start + i;
        const int slot = cache_slot(a, i, pos);
        const int64_t src_row = ((int64_t)b * a.S + i) * a.Hkv + g;
        const int64_t ws_row =
            ((int64_t)b * a.Hkv + g) * a.ws_rows + (a.ws_rel ? start : 0) + a.ws_row0 + i;
        if (c < a.dqk) {
            const float* krow = (const float*)a.k + src_row * a.dqk;
            float x = krow[c];
            if (c < r) {
                const bool lower = c < half;
                float cs, sn;
                rope_cos_sin_rev(pos, a.omega_rev[lower ? c : c - half], cs, sn);
                x = lower ? (x * cs - krow[c + half] * sn) : (x * cs + krow[c - half] * sn);
            }
            if (a.k_ws) ((float*)a.k_ws)[ws_row * a.dqk + c] = x;
            if (slot >= 0) ((float*)a.k_dst)[(((int64_t)b * a.Hkv + g) * a.cap + slot) * a.dqk + c] = x;
        } else if (slot >= 0 || a.v_ws) {
            const int d = c - a.dqk;
            const float x = ((const float*)a.v)[src_row * a.dv + d];
            if (a.v_ws) ((float*)a.v_ws)[ws_row * a.dv + d] = x;
            if (slot >= 0) ((float*)a.v_dst)[(((int64_t)b * a.Hkv + g) * a.cap + slot) * a.dv + d] = x;
        }
    }
}

// bf16 cache rows: one thread per 8-element chunk of a K or V row.
__global__ __launch_bounds__(256) void cache_rows_bf16_kernel(const CacheRowsArgs a) {
    const int kch = a.dqk / 8, per_row = kch + a.dv / 8;
    const int64_t total = (int64_t)a.B * a.Hkv * a.rows * per_row;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(e % per_row);
        const int64_t rowid = e / per_row;
        const int r = (int)(rowid % a.rows);
        const int64_t bg = rowid / a.rows;         // b * Hkv + g
        const int b = (int)(bg / a.Hkv);
        const int32_t start = a.start_pos[b];
        if (!start_ok(start, a.max_start)) continue;
        const int32_t pos = a.W > 0 ? start - a.W + r : r;
        if (pos < 0 || (a.W == 0 && pos >= start)) continue;
        const int64_t slot_row = bg * a.cap + (a.W > 0 ? pos % a.W : pos);
        const int64_t ws_row = bg * a.ws_rows + r;
        const bool key = c < kch;
        const int d = 8 * (key ? c : c - kch), dim = key ? a.dqk : a.dv;
        uint16_t* dst = (key ? a.k_ws : a.v_ws) + ws_row * dim + d;
        if (a.cache_fp8) {
            const uint8_t* src = (const uint8_t*)(key ? a.k_cache : a.v_cache) + slot_row * dim + d;
            float x[8];
            unpack8(bf16x8_from_e4m3x8(*(const u32x2*)src), x);   // exact e4m3 values
            const float sc = key ? a.k_scale : a.v_scale;
#pragma unroll
            for (int t = 0; t < 8; ++t) x[t] *= sc;
            *(u32x4*)dst = pack8(x);
        } else {
            const uint16_t* src = (const uint16_t*)(key ? a.k_cache : a.v_cache) + slot_row * dim + d;
            *(u32x4*)dst = *(const u32x4*)src;
        }
    }
}

unsigned grid_for(int64_t total) {
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    return (unsigned)(blocks > 0 ? blocks : 1);
}

}  // namespace

hipError_t launch_rope_kv_bf16(const RopeKVArgs& a, hipStream_t st) {
    int64_t total = (int64_t)a.B * a.Hkv *
                    ((int64_t)(a.S - a.i0) * (a.dqk / 8) + (int64_t)(a.S - rope_v_first(a)) * (a.dv / 8));
    if (total <= 0 || (!a.k_ws && !a.k_dst && !a.v_ws)) return hipSuccess;
    // Heads per thread: the largest power of two up to 8 dividing Hkv that still leaves at least
    // 2^18 threads (4 waves of 256 threads per CU); small calls keep one head per thread, where a
    // smaller grid would cost more latency than the shared angles save.
    int hg = 1;
    while (hg < 8 && a.Hkv % (2 * hg) == 0 && total / (2 * hg) >= (int64_t{1} << 18)) hg *= 2;
    const unsigned grid = grid_for(total / hg);
    switch (hg) {
        case 8: rope_kv_bf16_kernel<8><<<grid, 256, 0, st>>>(a); break;
        case 4: rope_kv_bf16_kernel<4><<<grid, 256, 0, st>>>(a); break;
        case 2: rope_kv_bf16_kernel<2><<<grid, 256, 0, st>>>(a); break;
        default: rope_kv_bf16_kernel<1><<<grid, 256, 0, st>>>(a); break;
    }
    return hipGetLastError();
}

hipError_t launch_rope_kv_f32(const RopeKVArgs& a, hipStream_t st) {
    const int64_t total =
        (int64_t)a.B * (a.S - a.i0) * a.Hkv * (a.dqk + ((a.k_dst || a.v_ws) ? a.dv : 0));
    if (total <= 0 || (!a.k_ws && !a.k_dst && !a.v_ws)) return hipSuccess;
    rope_kv_f32_kernel<<<grid_for(total), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_cache_rows_bf16(const CacheRowsArgs& a, hipStream_t st) {
    if (a.dqk % 8 || a.dv % 8 || (a.W > 0 && a.cap != a.W)) return hipErrorInvalidValue;
    const int64_t total = (int64_t)a.B * a.Hkv * a.rows * (a.dqk / 8 + a.dv / 8);
    if (total <= 0) return hipSuccess;
    cache_rows_bf16_kernel<<<grid_for(total), 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace mimo
