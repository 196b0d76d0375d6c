// router.hip — grouped sigmoid top-k routing of MoE tokens (the router of the MiMo-V2-Flash
// decoder; definition and citations in include/mimo_router.h).
//
// One wave per token: lane l holds experts [l * EPL, (l + 1) * EPL) (EPL = E / 64), so a group of
// E / n_group experts spans 64 / n_group whole lanes.  Group top-2 sums by a reduction ladder over
// the group's lanes, group ranks by reading every group's score by lane index, then top_k rounds
// of a wave-wide maximum score whose lowest holder is found by ballots.  Every cross-lane step is
// a DPP permute, a lane-pair swap or a ballot (no LDS round trips).
#include <math.h>
#include <string.h>

#include "device_common.h"
#include "kernels.h"
#include "mimo_router.h"

namespace mimo {
namespace {

struct RouterArgs {
    const float* logits;
    const float* bias;
    int32_t* idx;
    float* weights;
    int32_t T, n_group, topk_group, top_k, norm;
    float scale;
};

// Order-preserving 32-bit key of a score: a larger score is a larger key (0 is below every
// score, -inf included, and marks a chosen expert).
__device__ __forceinline__ uint32_t score_key(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// x from lane (lane ^ step partner) for the reduction ladder: step 0 pairs lanes l, l^1 and
// step 1 l, l^2 (quad permutes), step 2 l, 7-l within 8, step 3 l, 15-l within 16 (row mirrors),
// step 4 l, l^16, step 5 l, l^32 (lane-pair swaps).  After steps 0..n-1 every lane holds the
// reduction over its aligned group of 2^n lanes.
__device__ __forceinline__ uint32_t ladder(uint32_t x, int step) {
    switch (step) {
        case 0: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
        case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
        case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);
        case 3: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false);
        // (the swap hands every lane the pair {own, partner}: the partner's value is the second
        //  one in the lower row of the pair and the first one in the upper row)
        case 4: {
            const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
            return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
        }
        default: {
            const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
            return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
        }
    }
}

__device__ __forceinline__ float ladder_f(float x, int step) {
    return __uint_as_float(ladder(__float_as_uint(x), step));
}

__device__ __forceinline__ uint32_t ladder_max(uint32_t k) {
#pragma unroll
    for (int st = 0; st < 6; ++st) k = max(k, ladder(k, st));
    return k;
}

template <int EPL, int LPG>
__global__ __launch_bounds__(256) void router_kernel(const RouterArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;   // (whole waves: the token index is uniform in a wave)
    constexpr int E = 64 * EPL;
    constexpr int G = 64 / LPG;                    // groups
    constexpr int gsteps = __builtin_ctz(LPG);     // ladder steps that span a group
    float x[EPL], bias[EPL], s[EPL], c[EPL];
    const float* row = a.logits + (int64_t)t * E + lane * EPL;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        x[j] = row[j];
        bias[j] = a.bias ? a.bias[lane * EPL + j] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        s[j] = (float)(1.0 / (1.0 + exp(-(double)x[j])));
        c[j] = s[j] + bias[j];
    }
    // ---- group score: the two largest c of the group (values only; ties do not change the sum)
    float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        if (c[j] > m1) {
            m2 = m1;
            m1 = c[j];
        } else if (c[j] > m2) {
            m2 = c[j];
        }
    }
#pragma unroll
    for (int st = 0; st < gsteps; ++st) {
        const float o1 = ladder_f(m1, st), o2 = ladder_f(m2, st);
        const float hi = fmaxf(m1, o1);
        const float lo = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
        m1 = hi;
        m2 = lo;
    }
    const float gscore = m1 + m2;
    const int g = lane / LPG;
    // ---- rank of this lane's group among all groups (every group score read by lane index)
    int rank = 0;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gscore), j * LPG));
        rank += (o > gscore || (o == gscore && j < g)) ? 1 : 0;
    }
    const bool kept = rank < a.topk_group;
    uint32_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) key[j] = score_key(kept ? c[j] : -INFINITY);
    // ---- top_k rounds: the largest key over the wave, then the lowest expert index holding it
    //      (ballots per register slot: lane-major order within a slot, slot order within a lane)
    int my_idx = -1;   // lane k keeps the k-th choice
    float my_s = 0.0f, sum = 0.0f;
    for (int k = 0; k < a.top_k; ++k) {
        uint32_t best = key[0];
#pragma unroll
        for (int j = 1; j < EPL; ++j) best = max(best, key[j]);
        const uint32_t M = __builtin_amdgcn_readfirstlane(ladder_max(best));
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const uint64_t hit = __ballot(key[j] == M);
            if (hit) bi = min(bi, (int)__builtin_ctzll(hit) * EPL + j);
        }
        const int owner = bi / EPL, slot = bi - owner * EPL;
        float sv = s[0];
#pragma unroll
        for (int j = 1; j < EPL; ++j) sv = slot == j ? s[j] : sv;
        const float bs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), owner));
        if (lane == owner) {   // retire the chosen expert
#pragma unroll
            for (int j = 0; j < EPL; ++j)
                if (j == slot) key[j] = 0;
        }
        if (lane == k) {
            my_idx = bi;
            my_s = bs;
        }
        sum += bs;   // in rank order, the same on every lane
    }
    if (lane < a.top_k) {
        const float w = (a.norm ? my_s / sum : my_s) * a.scale;
        a.idx[(int64_t)t * a.top_k + lane] = my_idx;
        a.weights[(int64_t)t * a.top_k + lane] = w;
    }
}

}  // namespace

template <int EPL>
void launch_router(const RouterArgs& a, int n_group, dim3 grid, dim3 block, hipStream_t st) {
    switch (n_group) {   // lanes per group = 64 / n_group
        case 1: router_kernel<EPL, 64><<<grid, block, 0, st>>>(a); break;
        case 2: router_kernel<EPL, 32><<<grid, block, 0, st>>>(a); break;
        case 4: router_kernel<EPL, 16><<<grid, block, 0, st>>>(a); break;
        case 8: router_kernel<EPL, 8><<<grid, block, 0, st>>>(a); break;
        case 16: router_kernel<EPL, 4><<<grid, block, 0, st>>>(a); break;
        case 32: router_kernel<EPL, 2><<<grid, block, 0, st>>>(a); break;
        default: router_kernel<EPL, 1><<<grid, block, 0, st>>>(a); break;
    }
}

}  // namespace mimo

extern "C" {

int mimo_router_check_params(const mimo_router_params* p) {
    if (!p) return mimo::set_error(MIMO_ERR_INVALID_ARG, "router params is NULL");
    if (p->reserved != 0) return mimo::set_error(MIMO_ERR_INVALID_ARG, "reserved must be 0");
    const int E = p->num_experts, G = p->n_group;
    if (p->num_tokens < 0 || E < 1 || G < 1 || E % G || E / G < 2 || p->topk_group < 1 ||
        p->topk_group > G || p->top_k < 1 || p->top_k > p->topk_group * (E / G) ||
        !isfinite(p->routed_scaling_factor))
        return mimo::set_error(MIMO_ERR_INVALID_ARG,
                               "router: need T >= 0, E % n_group == 0 with groups of >= 2 "
                               "experts, 1 <= topk_group <= n_group, 1 <= top_k <= kept experts, "
                               "a finite scale");
    if ((E != 64 && E != 128 && E != 256 && E != 512) || (G & (G - 1)) || G > 64 || p->top_k > 64)
        return mimo::set_error(MIMO_ERR_UNSUPPORTED,
                               "router kernel covers E in {64,128,256,512}, n_group a power of "
                               "two up to 64, top_k up to 64");
    mimo::clear_error();
    return MIMO_OK;
}

int mimo_router_topk(const mimo_router_params* p, const float* logits, const float* bias,
                     int32_t* expert_idx, float* weights, void* stream) {
    const int rc = mimo_router_check_params(p);
    if (rc != MIMO_OK) return rc;
    if (p->num_tokens == 0) return MIMO_OK;
    if (!logits || !expert_idx || !weights)
        return mimo::set_error(MIMO_ERR_INVALID_ARG, "logits, expert_idx and weights must be non-NULL");
    mimo::RouterArgs a;
    memset(&a, 0, sizeof a);
    a.logits = logits;
    a.bias = bias;
    a.idx = expert_idx;
    a.weights = weights;
    a.T = p->num_tokens;
    a.n_group = p->n_group;
    a.topk_group = p->topk_group;
    a.top_k = p->top_k;
    a.norm = p->norm_topk_prob != 0;
    a.scale = p->routed_scaling_factor;
    const dim3 grid((unsigned)((p->num_tokens + 3) / 4)), block(256);
    hipStream_t st = (hipStream_t)stream;
    switch (p->num_experts) {
        case 64: mimo::launch_router<1>(a, p->n_group, grid, block, st); break;
        case 128: mimo::launch_router<2>(a, p->n_group, grid, block, st); break;
        case 256: mimo::launch_router<4>(a, p->n_group, grid, block, st); break;
        default: mimo::launch_router<8>(a, p->n_group, grid, block, st); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return mimo::set_error(MIMO_ERR_HIP, hipGetErrorString(e));
    mimo::clear_error();
    return MIMO_OK;
}

}  // extern "C"
