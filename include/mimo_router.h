/*
 * mimo_router.h — C ABI of the MoE router kernel in `libmimo_attn.so` (the library of
 * mimo_attn.h; same status codes, same thread-local error message, mimo_attn_last_error()).
 *
 * The router of the MiMo-V2-Flash decoder as the pages describe it ("Add Xiaomi MiMo-V2", the
 * router notes: DeepSeek-V3's top-k router with its route-tokens-to-experts step, experts of the
 * groups that are not kept masked with -inf instead of 0; "add Xiaomi MiMo v2 (mimo_v2_flash)",
 * "Architecture, verified against upstream": the routing activation is a sigmoid of the gate
 * logits taken in float32).  Per token, over E experts in n_group equal consecutive groups:
 *   s_e = sigmoid(logit_e) (float32: the fp64 sigmoid rounded to float32);
 *   c_e = s_e + bias_e (float32; bias NULL = 0);
 *   group score = the sum of the group's two largest c (float32, largest first);
 *   the topk_group groups with the largest scores are kept, the others' experts get c = -inf;
 *   the top_k experts by c are chosen, in rank order; equal scores rank the lower index first;
 *   weight_k = s of chosen expert k, divided by the sum of the chosen s when norm_topk_prob,
 *   times routed_scaling_factor (float32).
 * Every selection compares the float32 values above.
 */
#ifndef MIMO_ROUTER_H
#define MIMO_ROUTER_H

#include <stddef.h>
#include <stdint.h>

#include "mimo_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mimo_router_params {
    int32_t num_tokens;             /* T >= 0 (0: nothing to do)                              */
    int32_t num_experts;            /* E in {64, 128, 256, 512}                               */
    int32_t n_group;                /* power of two, 1..64, E / n_group >= 2                  */
    int32_t topk_group;             /* 1..n_group                                             */
    int32_t top_k;                  /* 1..min(64, topk_group * E / n_group)                   */
    int32_t norm_topk_prob;         /* nonzero: weights divided by their sum                  */
    float routed_scaling_factor;    /* finite                                                 */
    int32_t reserved;               /* must be 0                                              */
} mimo_router_params;

/*
 * Route T tokens.
 *   logits [T, E] fp32 (device), bias [E] fp32 (device) or NULL;
 *   expert_idx [T, top_k] int32 and weights [T, top_k] fp32 (device, caller-owned) receive the
 *   chosen experts in rank order and their weights.
 * Work is enqueued on `stream` (hipStream_t; NULL = the null stream); nothing is allocated or
 * synchronised.  Invalid parameters return a negative MIMO_ERR_* code before anything is
 * enqueued (MIMO_ERR_UNSUPPORTED for a valid router the kernel does not cover), with the message
 * in mimo_attn_last_error().
 */
int mimo_router_topk(const mimo_router_params* p, const float* logits, const float* bias,
                     int32_t* expert_idx, float* weights, void* stream);

/* Host-only validation of a router parameter block: MIMO_OK or a negative code. */
int mimo_router_check_params(const mimo_router_params* p);

#ifdef __cplusplus
}
#endif
#endif /* MIMO_ROUTER_H */
