/*
 * router_oracle.c — plain CPU oracle of the MoE router of the MiMo-V2-Flash decoder.
 *
 * TEST INFRASTRUCTURE ONLY, like mimo_oracle.c (same library, same rules: only the test-suite,
 * the smoke check and the CPU-baseline leg of the benchmark load it; the product shares no code
 * with it).
 *
 * What the pages state ("Add Xiaomi MiMo-V2", the router notes; "add Xiaomi MiMo v2
 * (mimo_v2_flash)", "Architecture, verified against upstream"):
 *   - the routing activation is a sigmoid of the gate logits taken in float32;
 *   - the router is DeepSeek-V3's top-k router together with its route-tokens-to-experts step,
 *     except that experts of the groups that are not selected are masked with -inf (not 0);
 *   - the model has 256 routed experts.
 * Readings for the steps the pages leave to that router (each listed in the design notes):
 *   selection score c_e = s_e + bias_e (a per-expert correction bias); experts split into
 *   n_group equal consecutive groups; group score = sum of the group's two largest c; the
 *   topk_group groups with the largest scores are kept; the top_k experts by c among the kept
 *   groups are chosen; weights are the chosen experts' s (without bias), divided by their sum
 *   when norm_topk_prob, times routed_scaling_factor.  Equal scores: the lower index ranks first.
 *
 * Precision: s_e = 1 / (1 + e^{-x}) evaluated in fp64 and rounded to fp32 (the float32 score the
 * pages name), c_e = s_e + bias_e in fp32, group score = top1 + top2 in fp32; every selection
 * compares these fp32 values.  Weights are formed in fp64 from the fp32 s values.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t num_tokens, num_experts, n_group, topk_group, top_k, norm_topk_prob;
    double routed_scaling_factor;
} oracle_router_params;

/* a ranks before b: larger value, or equal value and lower index */
static int ranks_before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

/* Indices of the n largest of v[0..m) by ranks_before, in rank order (selection by repeated
 * scanning: plain and obviously correct for the sizes at hand). */
static void top_n(const float* v, int m, int n, int* out) {
    unsigned char* taken = (unsigned char*)calloc((size_t)m, 1);
    for (int r = 0; r < n; ++r) {
        int best = -1;
        for (int i = 0; i < m; ++i)
            if (!taken[i] && (best < 0 || ranks_before(v[i], i, v[best], best))) best = i;
        out[r] = best;
        taken[best] = 1;
    }
    free(taken);
}

float oracle_router_sigmoid(float x) { return (float)(1.0 / (1.0 + exp(-(double)x))); }

int oracle_router(const oracle_router_params* p, const float* logits, const float* bias,
                  int32_t* idx, double* weights) {
    if (!p || p->num_tokens < 0 || p->num_experts < 1 || p->n_group < 1 ||
        p->num_experts % p->n_group || p->topk_group < 1 || p->topk_group > p->n_group ||
        p->top_k < 1 || p->top_k > (p->num_experts / p->n_group) * p->topk_group ||
        p->num_experts / p->n_group < 2 || (p->num_tokens > 0 && (!logits || !idx || !weights)))
        return -1;
    const int E = p->num_experts, G = p->n_group, gs = E / G;
    float* s = (float*)malloc(sizeof(float) * E);
    float* c = (float*)malloc(sizeof(float) * E);
    float* gscore = (float*)malloc(sizeof(float) * G);
    int* gsel = (int*)malloc(sizeof(int) * G);
    int* sel = (int*)malloc(sizeof(int) * E);
    int top2[2];
    for (int32_t t = 0; t < p->num_tokens; ++t) {
        const float* x = logits + (int64_t)t * E;
        for (int e = 0; e < E; ++e) {
            s[e] = oracle_router_sigmoid(x[e]);
            c[e] = s[e] + (bias ? bias[e] : 0.0f);
        }
        for (int g = 0; g < G; ++g) {
            top_n(c + g * gs, gs, 2, top2);
            gscore[g] = c[g * gs + top2[0]] + c[g * gs + top2[1]];
        }
        top_n(gscore, G, p->topk_group, gsel);
        /* experts outside the kept groups: -inf */
        float* cm = (float*)malloc(sizeof(float) * E);
        for (int e = 0; e < E; ++e) cm[e] = -INFINITY;
        for (int r = 0; r < p->topk_group; ++r)
            for (int e = gsel[r] * gs; e < (gsel[r] + 1) * gs; ++e) cm[e] = c[e];
        top_n(cm, E, p->top_k, sel);
        free(cm);
        double sum = 0.0;
        for (int r = 0; r < p->top_k; ++r) sum += (double)s[sel[r]];
        for (int r = 0; r < p->top_k; ++r) {
            idx[(int64_t)t * p->top_k + r] = sel[r];
            double w = (double)s[sel[r]];
            if (p->norm_topk_prob) w /= sum;
            weights[(int64_t)t * p->top_k + r] = w * p->routed_scaling_factor;
        }
    }
    free(s);
    free(c);
    free(gscore);
    free(gsel);
    free(sel);
    return 0;
}
