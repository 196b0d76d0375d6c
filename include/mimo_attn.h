/*
 * mimo_attn.h — C ABI of the MI355X (gfx950) hybrid attention library `libmimo_attn.so`.
 *
 * The layer is the attention of the MiMo-V2-Flash decoder as the pages describe it:
 *   - "Add Xiaomi MiMo-V2" (transformers PR 45144), section "Additional useful info": sliding-
 *     window (SWA) and global (GA) layers use different RoPE bases and different KV-group counts;
 *     the V head dim is separate from the QK head dim; values are scaled by
 *     sqrt(hidden / (num_attention_heads * v_head_dim)); the attention sink is used on SWA layers
 *     only; partial RoPE rotates the leading third of the QK head dim.
 *   - Same PR, description: gpt-oss-style attention sinks together with dual theta and dual
 *     head dims.
 *   - "feat(models): add Xiaomi MiMo v2 (mimo_v2_flash) text model support" (mlxcel issue 842),
 *     "Architecture, verified against upstream": the layer kind comes from hybrid_layer_pattern
 *     (1 = sliding); theta is swa_rope_theta on sliding layers, rope_theta otherwise; the rotated
 *     width is int(partial_rotary_factor * head_dim); the window is sliding_window_size.
 *     "Implementation plan": sliding layers keep a rotating KV cache.
 *
 * Computed, per query head h of sequence b at position p_i:
 *   q', k' = q, k with pairs (d, d + r/2), d < r/2, turned by p * theta^(-2d/r); dims >= r as is.
 *   z_j    = tau * <q'_i, k'_j>, tau = softmax_scale (0 selects 1/sqrt(qk_head_dim)),
 *            k'_j from KV head h / (Hq / Hkv).
 *   visible j: 0 <= p_i - p_j (GA); 0 <= p_i - p_j < window (SWA).
 *   out    = v_scale * sum_j e^{z_j} v_j / (e^{s_h} + sum_j e^{z_j}),  s_h = -inf without sinks.
 *
 * Conventions for every entry point:
 *   - Tensors are caller-owned memory on the current HIP device, dense row-major, with the shapes
 *     given below.  dtype MIMO_BF16: q/k/v/out/caches are bf16, arithmetic fp32 with bf16 MFMA
 *     operands.  dtype MIMO_F32: all of them fp32, arithmetic fp32.
 *   - sinks is fp32 [Hq] or NULL (no sink).  Position arrays are int32 in device memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).  Nothing is
 *     synchronised, allocated, freed or printed by the library, and it keeps no global state;
 *     calls are thread-safe.  (Exception: mimo_attn_decode_noalloc keeps its partials in a device
 *     array of the library and that array's address per device.)  Calls that write the same cache
 *     or workspace must be ordered by the caller (same stream or events).
 *   - Arguments are checked on the host before anything is enqueued.  On error the function
 *     returns a negative MIMO_ERR_* code, writes nothing, and mimo_attn_last_error() returns a
 *     message (thread-local).  MIMO_ERR_HIP means a launch failed; the message holds HIP's text.
 */
#ifndef MIMO_ATTN_H
#define MIMO_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIMO_ATTN_ABI_VERSION 2

enum mimo_attn_status {
    MIMO_OK = 0,
    MIMO_ERR_INVALID_ARG = -1, /* a null pointer, a bad size or an inconsistent parameter    */
    MIMO_ERR_UNSUPPORTED = -2, /* a valid layer the compiled kernels do not cover            */
    MIMO_ERR_WORKSPACE = -3,   /* workspace missing or smaller than *_workspace_size()       */
    MIMO_ERR_HIP = -4          /* a HIP launch failed                                        */
};

enum mimo_attn_layer_kind { /* the value of hybrid_layer_pattern[layer] */
    MIMO_LAYER_GLOBAL = 0,
    MIMO_LAYER_SWA = 1
};

enum mimo_attn_dtype { MIMO_F32 = 0, MIMO_BF16 = 1 };

/* Element type of the KV caches (params.cache_dtype). */
enum mimo_attn_cache_dtype {
    MIMO_CACHE_SAME = 0,     /* the layer dtype (bf16 or fp32 caches)                        */
    MIMO_CACHE_FP8_E4M3 = 2  /* one-byte OCP e4m3 codes with one fp32 scale per cache tensor */
};

typedef struct mimo_attn_params {
    int32_t batch;         /* B >= 0 (0: nothing to do)                                      */
    int32_t num_q_heads;   /* Hq >= 1                                                        */
    int32_t num_kv_heads;  /* Hkv >= 1, divides Hq (GQA group = Hq / Hkv)                    */
    int32_t qk_head_dim;   /* dqk                                                            */
    int32_t v_head_dim;    /* dv                                                             */
    int32_t rope_dims;     /* r: even, 0 <= r <= dqk; 0 = no rotation                        */
    int32_t layer_kind;    /* MIMO_LAYER_GLOBAL or MIMO_LAYER_SWA                            */
    int32_t window;        /* SWA: >= 1, keys with 0 <= p_q - p_k < window; GLOBAL: 0         */
    double rope_theta;     /* base of the layer kind, > 0 when r > 0                         */
    float v_scale;         /* multiplies the output; sqrt(hidden / (Hq * dv)) in the model   */
    float softmax_scale;   /* 0 selects 1 / sqrt(dqk)                                        */
    int32_t dtype;         /* MIMO_BF16 or MIMO_F32                                          */
    int32_t cache_dtype;   /* MIMO_CACHE_SAME or MIMO_CACHE_FP8_E4M3 (bf16 layers)           */
    float k_cache_scale;   /* fp8 caches: stored key = e4m3(code) * k_cache_scale (> 0)      */
    float v_cache_scale;   /* fp8 caches: stored value = e4m3(code) * v_cache_scale (> 0)    */
} mimo_attn_params;

/*
 * Head-dim support.  MIMO_BF16 runs the bf16-MFMA kernels, compiled for (dqk, dv) = (192, 128),
 * the head shape of both layer kinds at full size.  MIMO_F32 runs fp32 vector kernels for any
 * dqk <= 256 and dv <= 256 (used for small fp32 layers).  Other combinations return
 * MIMO_ERR_UNSUPPORTED.
 *
 * fp8 KV caches (cache_dtype MIMO_CACHE_FP8_E4M3, bf16 layers; the pages only hint at quantized
 * storage — "Add Xiaomi MiMo-V2", "Additional useful info", a garbled note of three dtypes with one
 * quantized — and this is the reading taken): the caches are uint8 arrays of OCP e4m3 codes
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals; 0x7F/0xFF NaN; largest finite
 * 448) with the shapes of the bf16 caches.  A stored element is written as the e4m3 value nearest
 * (ties to even) to clamp(x * (1 / scale), -448, 448), x the fp32 rotated key or the value, the
 * product and 1 / scale in fp32; it is read as e4m3(code) * scale.  Prefill, decode and extend
 * support fp8 caches.  Decode attends the new token with its stored (coded) value, like every
 * other cached token; prefill and extend attend their new tokens at full precision (as without a
 * cache) and the cached positions through their codes, and store the new tokens as codes.
 */

/*
 * Prefill: attention of S new tokens per sequence over themselves.
 *   q [B,S,Hq,dqk], k [B,S,Hkv,dqk], v [B,S,Hkv,dv]; out [B,S,Hq,dv].
 *   start_pos [B] (device): token i of sequence b sits at position start_pos[b] + i (>= 0).
 *   Only the S given tokens are attended (no earlier cache content is read).
 *   Caches (optional; both NULL or both set; bf16 for MIMO_BF16, fp32 for MIMO_F32):
 *     GLOBAL: linear, k_cache [B,Hkv,cache_capacity,dqk], v_cache [B,Hkv,cache_capacity,dv];
 *             token i is stored at slot start_pos[b] + i, which must be < cache_capacity
 *             (checked by the kernel: a token whose slot would be out of range is not stored).
 *     SWA:    ring, cache_capacity == window; the last min(S, window) tokens are stored at slot
 *             position % window.
 *     K is stored rotated, V as given.
 *   workspace: device scratch of at least mimo_attn_prefill_workspace_size() bytes (may be NULL
 *   when that size is 0).  Its contents are not needed across calls.
 */
int mimo_attn_prefill(const mimo_attn_params* p, int32_t seq_len, const void* q, const void* k,
                      const void* v, const int32_t* start_pos, const float* sinks, void* out,
                      void* k_cache, void* v_cache, int32_t cache_capacity, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Workspace bytes mimo_attn_prefill needs for this layer and seq_len: bf16 layers keep their keys,
 * rotated once, there (B * Hkv * seq_len * dqk * 2 bytes); fp32 layers need none (0).  Returns 0
 * for invalid parameters. */
size_t mimo_attn_prefill_workspace_size(const mimo_attn_params* p, int32_t seq_len);

/*
 * Extend (chunked prefill): S new tokens per sequence against themselves and the tokens already
 * in the cache, which it also appends to.  The same attention as prefill, with every earlier
 * position of the sequence visible as well (subject to the window): splitting a prompt into
 * chunks, each extending the cache the previous chunks left, gives the prompt's prefill result.
 * (Layer as defined above; the caches are the ones prefill and decode keep, the rotating one of
 * "add Xiaomi MiMo v2 (mimo_v2_flash)", "Implementation plan", with its sliding prefill mask.)
 *   q [B,S,Hq,dqk], k [B,S,Hkv,dqk], v [B,S,Hkv,dv] (raw: not rotated); out [B,S,Hq,dv].
 *   start_pos [B] (device): token i of sequence b sits at position start_pos[b] + i; the cache
 *   holds that sequence's positions before start_pos[b].
 *   max_start (host): an upper bound of every start_pos[b] (>= 0).  A sequence whose start_pos
 *   lies outside [0, max_start] gets a zero output and nothing is stored for it.
 *   GLOBAL: linear cache [B,Hkv,cache_capacity,d], max_start + S <= cache_capacity; slots
 *           0..start_pos[b]-1 must hold positions 0..start_pos[b]-1; the new tokens are stored at
 *           slots start_pos[b] + i before they are attended.
 *   SWA:    ring cache [B,Hkv,window,d], cache_capacity == window; slot p % window must hold
 *           position p for the min(window, start_pos[b]) positions p before start_pos[b]; the last
 *           min(S, window) new tokens are stored at slot position % window.
 *   K is stored rotated, V as given (as prefill and decode store them); fp8 caches as above.
 *   bf16 only: MIMO_F32 returns MIMO_ERR_UNSUPPORTED.
 *   workspace: at least mimo_attn_extend_workspace_size() bytes (may be NULL when that is 0).
 *   Its contents are not needed across calls.
 */
int mimo_attn_extend(const mimo_attn_params* p, int32_t seq_len, const void* q, const void* k,
                     const void* v, const int32_t* start_pos, int32_t max_start,
                     const float* sinks, void* out, void* k_cache, void* v_cache,
                     int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Workspace bytes mimo_attn_extend needs for seq_len new tokens and starts up to max_start: SWA
 * bf16 layers lay the ring's content out in position order in front of the new tokens' rotated
 * keys and values (B * Hkv * (window + seq_len) * (dqk + dv) * 2 bytes, rounded up to 256);
 * GLOBAL layers read a bf16 cache in place, and lay an fp8 cache's rows out widened to bf16 in
 * front of the new tokens (B * Hkv * (max_start + seq_len) * (dqk + dv) * 2 bytes, rounded up to
 * 256; row = position).  Up to 16 new tokens per sequence run a tile kernel
 * whose query columns are the (query head, new token) pairs of a KV group, split over the key
 * rows, which adds split partials (B * seq_len * Hq * splits * (dv + 2) * 4 bytes) when the key
 * range is cut into several splits.
 * Returns 0 for invalid parameters. */
size_t mimo_attn_extend_workspace_size(const mimo_attn_params* p, int32_t seq_len,
                                       int32_t max_start);

/*
 * Decode: one new token per sequence against the KV cache, which it also appends to.
 *   q [B,Hq,dqk], k_new [B,Hkv,dqk], v_new [B,Hkv,dv] (raw: not rotated); out [B,Hq,dv].
 *   positions [B] (device): tokens already cached for sequence b = position of the new token.
 *   max_position (host): an upper bound of every positions[b]; it sizes the grid and the
 *   workspace.  A sequence whose position exceeds it, or whose slot exceeds the linear cache,
 *   produces a zero output and is not appended.
 *   GLOBAL: linear cache [B,Hkv,cache_capacity,d], cache_capacity > max_position; the new
 *           token goes to slot positions[b] and keys 0..positions[b] are attended.
 *   SWA:    ring cache [B,Hkv,window,d], cache_capacity == window; the new token overwrites
 *           slot positions[b] % window and the min(window, positions[b] + 1) most recent
 *           positions are attended.
 *   The new key is rotated at positions[b] before it is stored and used.
 *   bf16: one cache slice [cache_capacity, dqk] must stay below 4 GiB (cache_capacity <=
 *   11184810), else MIMO_ERR_UNSUPPORTED.
 *   workspace: at least mimo_attn_decode_workspace_size() bytes, for split-K partial results.
 */
int mimo_attn_decode(const mimo_attn_params* p, const void* q, const void* k_new,
                     const void* v_new, const int32_t* positions, int32_t max_position,
                     void* k_cache, void* v_cache, int32_t cache_capacity, const float* sinks,
                     void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mimo_attn_decode needs: B * Hq * splits * (dv + 2) * 4 when the cache range is
 * cut into several splits, else 0.  Returns 0 for invalid parameters. */
size_t mimo_attn_decode_workspace_size(const mimo_attn_params* p, int32_t max_position);

/*
 * Allocation-free decode, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): mimo_attn_decode without the
 * workspace arguments, on the same kernels.  The split partials go to a file-scope device array
 * of the library, mimo_attn_decode_noalloc_max_bytes() bytes (32 MiB), which each device the
 * library runs on holds until the process ends; its address is looked up once per device.  A call
 * whose partials (mimo_attn_decode_workspace_size) exceed it returns MIMO_ERR_WORKSPACE and
 * writes nothing.  Nothing is allocated, and no routine that allocates is called.  Every call on
 * one device shares that device's array, which keeps the last call's partials (nothing in it has
 * to start at zero): calls that overlap on one device (other streams, other threads) race and
 * must be ordered by the caller.  Arguments, results and errors otherwise as mimo_attn_decode.
 */
int mimo_attn_decode_noalloc(const mimo_attn_params* p, const void* q, const void* k_new,
                             const void* v_new, const int32_t* positions, int32_t max_position,
                             void* k_cache, void* v_cache, int32_t cache_capacity,
                             const float* sinks, void* out, void* stream);

/* Size in bytes of the array behind mimo_attn_decode_noalloc (its largest partials). */
size_t mimo_attn_decode_noalloc_max_bytes(void);

/*
 * Layer prefill: the attention layer with its projections ("Add Xiaomi MiMo-V2", "Additional
 * useful info": the value head dim is decoupled from the QK head dim and the attention output is
 * rescaled by v_scale before the output projection; here the rescale is folded into that
 * projection, which is the same by linearity).
 *   x [B,S,hidden]; w_q [hidden, Hq*dqk], w_k [hidden, Hkv*dqk], w_v [hidden, Hkv*dv] (row-major,
 *   heads contiguous in the columns); w_o [Hq*dv, out_dim]; out [B,S,out_dim].  All bf16
 *   (MIMO_BF16 layers only; fp8 caches as for prefill).  hidden % 64 == 0 and out_dim % 8 == 0,
 *   else MIMO_ERR_UNSUPPORTED.
 *   q = x w_q, v = x w_v (bf16 results of fp32-accumulated products); k = x w_k rotated in fp32
 *   from the products' fp32 results before its one rounding to bf16 (rope_dims 0 or 64; other
 *   widths round k first and rotate it as mimo_attn_prefill does); then the attention of
 *   mimo_attn_prefill (positions, sinks, caches as there) with v_scale 1, then
 *   out = v_scale * attn w_o.  Every product runs on this library's own bf16 matrix-core kernel.
 *   workspace: at least mimo_attn_layer_workspace_size() bytes (q, k, v, attention output and the
 *   prefill workspace); its contents are not needed across calls.
 *   Errors as for mimo_attn_prefill; every argument is checked before anything is enqueued.
 */
int mimo_attn_layer_prefill(const mimo_attn_params* p, int32_t hidden, int32_t seq_len,
                            const void* x, const void* w_q, const void* w_k, const void* w_v,
                            const void* w_o, int32_t out_dim, const int32_t* start_pos,
                            const float* sinks, void* out, void* k_cache, void* v_cache,
                            int32_t cache_capacity, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes of mimo_attn_layer_prefill (0 for invalid parameters or fp32 layers). */
size_t mimo_attn_layer_workspace_size(const mimo_attn_params* p, int32_t hidden, int32_t seq_len);

/* Host-only validation of a parameter block (no device access): MIMO_OK or a negative code. */
int mimo_attn_check_params(const mimo_attn_params* p);

/* Message of the last error on the calling thread ("" after success). */
const char* mimo_attn_last_error(void);

/* MIMO_ATTN_ABI_VERSION of the built library. */
int mimo_attn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MIMO_ATTN_H */
