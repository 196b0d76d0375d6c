/*
 * mimo_oracle.c — plain fp64 CPU oracle for the MiMo-V2-Flash hybrid attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load this library.  The product path (the HIP library and its Python
 * binding) never calls it and shares no code, header, table or helper with it.
 *
 * What is computed, and where the pages state it:
 *   - "Add Xiaomi MiMo-V2" (transformers PR 45144), section "Additional useful info":
 *       RoPE base differs between sliding-window (SWA) and global (GA) layers; the KV-group
 *       count differs per kind (GQA); the value head dim is independent of the QK head dim;
 *       values are scaled by sqrt(hidden / (heads * v_head_dim)); the attention sink exists on
 *       SWA layers only; partial RoPE rotates the leading third of the head dim.
 *   - Same PR, description: the model combines dual RoPE theta, dual head dims and
 *     gpt-oss-style attention sinks.
 *   - "feat(models): add Xiaomi MiMo v2 (mimo_v2_flash) text model support" (mlxcel issue 842),
 *     section "Architecture, verified against upstream": the rotated width is
 *     int(partial_rotary_factor * head_dim); theta is swa_rope_theta on sliding layers and
 *     rope_theta otherwise; the window is sliding_window_size.  Section "Implementation plan":
 *     sliding layers keep a rotating KV cache.
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   rotation pairs (d, d + r/2) inside the first r dims, frequency theta^(-2d/r);
 *   softmax scale 1/sqrt(qk_head_dim); the sink is one raw logit per query head that adds
 *   exp(s_h) to the softmax denominator and carries no value; window = keys with
 *   0 <= p_i - p_j < W; GQA head h reads KV head h / (Hq/Hkv); the value scale multiplies the
 *   output; caches hold rotated K and raw V.
 *
 * Arithmetic: every input is read as float (bf16 and fp32 values are exact in float) and all
 * computation is fp64, two-pass exact softmax, no tiling, no online rescaling.
 *
 * Error behaviour: every entry point returns 0 on success and a negative code on invalid
 * arguments (same meaning as the product library's codes, re-implemented here):
 *   -1 invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

typedef struct {
    int32_t batch, num_q_heads, num_kv_heads, qk_head_dim, v_head_dim;
    int32_t rope_dims;   /* even, 0 <= rope_dims <= qk_head_dim                       */
    int32_t layer_kind;  /* 0 = global causal, 1 = sliding window                      */
    int32_t window;      /* sliding: >= 1; global: ignored                            */
    double rope_theta;   /* the theta of this layer kind                              */
    double v_scale;      /* multiplies the output                                     */
    double softmax_scale;/* 0 => 1/sqrt(qk_head_dim)                                  */
} oracle_params;

static int check_params(const oracle_params* p) {
    if (!p) return ORACLE_EINVAL;
    if (p->batch < 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0) return ORACLE_EINVAL;
    if (p->num_q_heads % p->num_kv_heads) return ORACLE_EINVAL;
    if (p->qk_head_dim <= 0 || p->v_head_dim <= 0) return ORACLE_EINVAL;
    if (p->rope_dims < 0 || p->rope_dims > p->qk_head_dim || (p->rope_dims & 1)) return ORACLE_EINVAL;
    if (p->layer_kind != 0 && p->layer_kind != 1) return ORACLE_EINVAL;
    if (p->layer_kind == 1 && p->window < 1) return ORACLE_EINVAL;
    if (p->rope_dims > 0 && !(p->rope_theta > 0.0)) return ORACLE_EINVAL;
    return ORACLE_OK;
}

static double score_scale(const oracle_params* p) {
    return p->softmax_scale != 0.0 ? p->softmax_scale : 1.0 / sqrt((double)p->qk_head_dim);
}

/* Threads the oracle's parallel loops use (reported beside its timings). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Frequencies of the rotated slice: omega_d = theta^(-2d/r), d in [0, r/2). */
int oracle_rope_omega(int32_t rope_dims, double theta, double* omega) {
    if (rope_dims < 0 || (rope_dims & 1) || !omega) return ORACLE_EINVAL;
    for (int32_t d = 0; d < rope_dims / 2; ++d)
        omega[d] = pow(theta, -2.0 * (double)d / (double)rope_dims);
    return ORACLE_OK;
}

/* Rotate one head vector x (length dim) at position pos.  Pair (d, d + r/2) for d < r/2 is
 * turned by the angle pos*omega_d; dims >= r are copied unchanged. */
static void rotate_row(const double* x, double* y, int32_t dim, int32_t r, const double* omega,
                       double pos) {
    const int32_t h = r / 2;
    for (int32_t d = 0; d < h; ++d) {
        const double a = pos * omega[d];
        const double c = cos(a), s = sin(a);
        y[d] = x[d] * c - x[d + h] * s;
        y[d + h] = x[d + h] * c + x[d] * s;
    }
    for (int32_t d = r; d < dim; ++d) y[d] = x[d];
}

/* Public form of the rotation for tests: n rows of length dim, one position per row. */
int oracle_rope_rotate(const double* x, double* y, int64_t n, int32_t dim, int32_t rope_dims,
                       double theta, const int32_t* positions) {
    if (!x || !y || !positions || dim <= 0 || rope_dims < 0 || rope_dims > dim || (rope_dims & 1))
        return ORACLE_EINVAL;
    double omega[4096];
    if (rope_dims / 2 > 4096) return ORACLE_EINVAL;
    oracle_rope_omega(rope_dims, theta, omega);
    for (int64_t i = 0; i < n; ++i)
        rotate_row(x + i * dim, y + i * dim, dim, rope_dims, omega, (double)positions[i]);
    return ORACLE_OK;
}

/* A key at position pk is visible to a query at position pq. */
static int visible(const oracle_params* p, int64_t pq, int64_t pk) {
    const int64_t diff = pq - pk;
    if (diff < 0) return 0;
    if (p->layer_kind == 1) return diff < (int64_t)p->window;
    return 1;
}

/* Softmax-with-sink over one query row.  z: n scores (already scaled); vals: n value rows of
 * length dv (stride dv); sink: raw logit or -INFINITY.  Writes dv outputs scaled by v_scale. */
static void attend_row(const double* z, const double* const* vals, int64_t n, int32_t dv,
                       double sink, double v_scale, double* out) {
    double m = sink;
    for (int64_t j = 0; j < n; ++j)
        if (z[j] > m) m = z[j];
    for (int32_t e = 0; e < dv; ++e) out[e] = 0.0;
    if (m == -INFINITY) return; /* nothing visible and no sink: define the row as zero */
    double den = (sink == -INFINITY) ? 0.0 : exp(sink - m);
    for (int64_t j = 0; j < n; ++j) {
        const double w = exp(z[j] - m);
        den += w;
        for (int32_t e = 0; e < dv; ++e) out[e] += w * vals[j][e];
    }
    for (int32_t e = 0; e < dv; ++e) out[e] = v_scale * out[e] / den;
}

static double dot(const double* a, const double* b, int32_t n) {
    double s = 0.0;
    for (int32_t d = 0; d < n; ++d) s += a[d] * b[d];
    return s;
}

/*
 * Prefill: one layer over S new tokens per sequence.
 *   q [B,S,Hq,dqk], k [B,S,Hkv,dqk], v [B,S,Hkv,dv] (float, row-major), positions [B,S],
 *   sinks [Hq] or NULL (no sink), out [B,S,Hq,dv] (double).
 *   rows: optional list of query indices (nrows entries) to compute; NULL computes all S rows.
 *   Rows not listed are left untouched.
 *   k_rot_out: optional [B,S,Hkv,dqk] double, receives the rotated keys.
 */
/* Element i of a q/k/v input given as float (f64 = 0) or double (f64 = 1). */
static double in_elem(const void* a, int64_t i, int f64) {
    return f64 ? ((const double*)a)[i] : (double)((const float*)a)[i];
}

static int prefill_core(const oracle_params* p, int32_t S, const void* q, const void* k,
                        const void* v, int f64, const int32_t* positions, const float* sinks,
                        double* out, const int32_t* rows, int32_t nrows, double* k_rot_out) {
    if (check_params(p) != ORACLE_OK || S < 0 || !q || !k || !v || !positions || !out)
        return ORACLE_EINVAL;
    const int32_t B = p->batch, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
    const int32_t dqk = p->qk_head_dim, dv = p->v_head_dim, r = p->rope_dims;
    const int32_t group = Hq / Hkv;
    const int32_t nr = rows ? nrows : S;
    if (rows)
        for (int32_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= S) return ORACLE_EINVAL;
    const double tau = score_scale(p);
    double omega[4096];
    if (r / 2 > 4096) return ORACLE_EINVAL;
    oracle_rope_omega(r, p->rope_theta, omega);

    /* Rotate every key once (fp64), and widen every value. */
    const int64_t nk = (int64_t)B * S * Hkv;
    double* kr = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * dqk);
    double* vd = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * dv);
    if (!kr || !vd) { free(kr); free(vd); return ORACLE_EINVAL; }
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nk; ++t) {
        const int64_t b = t / ((int64_t)S * Hkv), s = (t / Hkv) % S;
        double tmp[4096];
        for (int32_t d = 0; d < dqk; ++d) tmp[d] = in_elem(k, t * dqk + d, f64);
        rotate_row(tmp, kr + t * dqk, dqk, r, omega, (double)positions[b * S + s]);
        for (int32_t e = 0; e < dv; ++e) vd[t * dv + e] = in_elem(v, t * dv + e, f64);
    }
    if (k_rot_out) memcpy(k_rot_out, kr, sizeof(double) * (size_t)nk * dqk);

    const int64_t work = (int64_t)B * Hq * nr;
    int bad = 0;
    #pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
        const double** vals = (const double**)malloc(sizeof(double*) * (size_t)(S > 0 ? S : 1));
        double qraw[4096], qrot[4096];
        if (!z || !vals) {
            #pragma omp atomic write
            bad = 1;
        } else {
            #pragma omp for schedule(dynamic, 4)
            for (int64_t w = 0; w < work; ++w) {
                const int32_t b = (int32_t)(w / ((int64_t)Hq * nr));
                const int32_t h = (int32_t)((w / nr) % Hq);
                const int32_t i = rows ? rows[w % nr] : (int32_t)(w % nr);
                const int32_t g = h / group;
                const int64_t qoff = (((int64_t)b * S + i) * Hq + h) * dqk;
                for (int32_t d = 0; d < dqk; ++d) qraw[d] = in_elem(q, qoff + d, f64);
                const int64_t pi = positions[(int64_t)b * S + i];
                rotate_row(qraw, qrot, dqk, r, omega, (double)pi);
                int64_t n = 0;
                for (int32_t j = 0; j < S; ++j) {
                    const int64_t pj = positions[(int64_t)b * S + j];
                    if (!visible(p, pi, pj)) continue;
                    const int64_t kv = ((int64_t)b * S + j) * Hkv + g;
                    z[n] = tau * dot(qrot, kr + kv * dqk, dqk);
                    vals[n] = vd + kv * dv;
                    ++n;
                }
                const double sink = sinks ? (double)sinks[h] : -INFINITY;
                attend_row(z, vals, n, dv, sink, p->v_scale,
                           out + (((int64_t)b * S + i) * Hq + h) * dv);
            }
        }
        free(z);
        free(vals);
    }
    free(kr);
    free(vd);
    return bad ? ORACLE_EINVAL : ORACLE_OK;
}

int oracle_prefill(const oracle_params* p, int32_t S, const float* q, const float* k,
                   const float* v, const int32_t* positions, const float* sinks, double* out,
                   const int32_t* rows, int32_t nrows, double* k_rot_out) {
    return prefill_core(p, S, q, k, v, 0, positions, sinks, out, rows, nrows, k_rot_out);
}

/* Prefill with q, k, v given in double (e.g. fp64 projections of a layer input). */
int oracle_prefill_f64(const oracle_params* p, int32_t S, const double* q, const double* k,
                       const double* v, const int32_t* positions, const float* sinks,
                       double* out, const int32_t* rows, int32_t nrows, double* k_rot_out) {
    return prefill_core(p, S, q, k, v, 1, positions, sinks, out, rows, nrows, k_rot_out);
}

/*
 * Raw score matrix of one (batch, query head): z[i][j] = tau * <rot(q_i), rot(k_j)> for all
 * i, j in [0,S) with no mask applied.  Used by the brute-force pin on tiny inputs.
 */
int oracle_scores(const oracle_params* p, int32_t S, const float* q, const float* k,
                  const int32_t* positions, int32_t b, int32_t h, double* z) {
    if (check_params(p) != ORACLE_OK || !q || !k || !positions || !z) return ORACLE_EINVAL;
    if (b < 0 || b >= p->batch || h < 0 || h >= p->num_q_heads) return ORACLE_EINVAL;
    const int32_t Hq = p->num_q_heads, Hkv = p->num_kv_heads, dqk = p->qk_head_dim;
    const int32_t g = h / (Hq / Hkv);
    double omega[4096], a[4096], ar[4096], c[4096], cr[4096];
    if (p->rope_dims / 2 > 4096 || dqk > 4096) return ORACLE_EINVAL;
    oracle_rope_omega(p->rope_dims, p->rope_theta, omega);
    const double tau = score_scale(p);
    for (int32_t i = 0; i < S; ++i) {
        for (int32_t d = 0; d < dqk; ++d) a[d] = q[(((int64_t)b * S + i) * Hq + h) * dqk + d];
        rotate_row(a, ar, dqk, p->rope_dims, omega, (double)positions[(int64_t)b * S + i]);
        for (int32_t j = 0; j < S; ++j) {
            for (int32_t d = 0; d < dqk; ++d) c[d] = k[(((int64_t)b * S + j) * Hkv + g) * dqk + d];
            rotate_row(c, cr, dqk, p->rope_dims, omega, (double)positions[(int64_t)b * S + j]);
            z[(int64_t)i * S + j] = tau * dot(ar, cr, dqk);
        }
    }
    return ORACLE_OK;
}

/*
 * Decode: one new token per sequence against previously cached keys.
 *   The cache is given as a position -> (rotated key, value) map per (sequence, KV head):
 *     kc [B,Hkv,L,dqk] rotated keys, vc [B,Hkv,L,dv] values, kpos [B,L] their positions,
 *     count [B] number of valid entries (entries beyond count are ignored).
 *   q [B,Hq,dqk], k_new [B,Hkv,dqk] (raw, not rotated), v_new [B,Hkv,dv], pos [B] = position of
 *   the new token.  The new key is rotated at pos[b] and joins the visible set.
 *   Visible: cached entries at positions before pos[b] that the mask admits, plus the new
 *   token itself (entries at positions >= pos[b] are ignored).
 *   out [B,Hq,dv]; k_new_rot [B,Hkv,dqk] optional, receives the rotated new key.
 *   batch_rows: optional list of sequences to compute (others untouched); NULL = all.
 */
/*
 * The cache of a decode: either float entries (rotated keys, values) or fp8 e4m3 codes with
 * one scale per tensor (see the fp8 section below).  For fp8 caches the new token is quantized
 * the way the cache stores it and attended with its stored value.
 */
typedef struct {
    const float* kf;
    const float* vf;
    const uint8_t* k8;
    const uint8_t* v8;
    double k_scale, v_scale;   /* fp8: stored value = e4m3(code) * scale */
    float k_inv, v_inv;        /* fp8: 1 / scale rounded to fp32 */
} decode_cache;

double oracle_e4m3_value(uint8_t c);
uint8_t oracle_e4m3_code(float y);

static int decode_core(const oracle_params* p, const float* q, const float* k_new,
                       const float* v_new, const int32_t* pos, const decode_cache* c,
                       const int32_t* kpos, const int32_t* count, int32_t L, const float* sinks,
                       double* out, double* k_new_rot, uint8_t* k_code_new, uint8_t* v_code_new,
                       const int32_t* batch_rows, int32_t nbatch_rows) {
    const int fp8 = c->k8 != NULL;
    if (check_params(p) != ORACLE_OK || !q || !k_new || !v_new || !pos || !out || L < 0)
        return ORACLE_EINVAL;
    if (L > 0 && (!kpos || !count || (fp8 ? (!c->k8 || !c->v8) : (!c->kf || !c->vf))))
        return ORACLE_EINVAL;
    const int32_t B = p->batch, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
    const int32_t dqk = p->qk_head_dim, dv = p->v_head_dim, r = p->rope_dims;
    const int32_t group = Hq / Hkv;
    const int32_t nb = batch_rows ? nbatch_rows : B;
    if (batch_rows)
        for (int32_t t = 0; t < nbatch_rows; ++t)
            if (batch_rows[t] < 0 || batch_rows[t] >= B) return ORACLE_EINVAL;
    for (int32_t b = 0; b < B; ++b)
        if (L > 0 && (count[b] < 0 || count[b] > L)) return ORACLE_EINVAL;
    const double tau = score_scale(p);
    double omega[4096];
    if (r / 2 > 4096) return ORACLE_EINVAL;
    oracle_rope_omega(r, p->rope_theta, omega);

    const int64_t work = (int64_t)nb * Hq;
    int bad = 0;
    #pragma omp parallel
    {
        const int64_t cap = (int64_t)L + 1;
        double* z = (double*)malloc(sizeof(double) * (size_t)cap);
        double* vrows = (double*)malloc(sizeof(double) * (size_t)cap * dv);
        const double** vals = (const double**)malloc(sizeof(double*) * (size_t)cap);
        double tmp[4096], qrot[4096], knew[4096], kj[4096];
        if (!z || !vrows || !vals) {
            #pragma omp atomic write
            bad = 1;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t w = 0; w < work; ++w) {
                const int32_t b = batch_rows ? batch_rows[w / Hq] : (int32_t)(w / Hq);
                const int32_t h = (int32_t)(w % Hq);
                const int32_t g = h / group;
                const int64_t pq = pos[b];
                const int64_t kv_row = (int64_t)b * Hkv + g;
                for (int32_t d = 0; d < dqk; ++d) tmp[d] = (double)q[((int64_t)b * Hq + h) * dqk + d];
                rotate_row(tmp, qrot, dqk, r, omega, (double)pq);
                for (int32_t d = 0; d < dqk; ++d) tmp[d] = (double)k_new[kv_row * dqk + d];
                rotate_row(tmp, knew, dqk, r, omega, (double)pq);
                if (k_new_rot && h % group == 0)
                    memcpy(k_new_rot + kv_row * dqk, knew, sizeof(double) * dqk);
                if (fp8) {
                    /* the new key as the cache stores it: fp32 of the rotated key, times the
                     * fp32 inverse scale, to the nearest code */
                    for (int32_t d = 0; d < dqk; ++d) {
                        const uint8_t code = oracle_e4m3_code((float)knew[d] * c->k_inv);
                        if (k_code_new && h % group == 0) k_code_new[kv_row * dqk + d] = code;
                        knew[d] = oracle_e4m3_value(code) * c->k_scale;
                    }
                }
                int64_t n = 0;
                const int32_t cnt = L > 0 ? count[b] : 0;
                for (int32_t j = 0; j < cnt; ++j) {
                    const int64_t pk = kpos[(int64_t)b * L + j];
                    /* only keys strictly in the past of the new token; it is itself at pq */
                    if (pk >= pq || !visible(p, pq, pk)) continue;
                    const int64_t off = kv_row * L + j;
                    for (int32_t d = 0; d < dqk; ++d)
                        kj[d] = fp8 ? oracle_e4m3_value(c->k8[off * dqk + d]) * c->k_scale
                                    : (double)c->kf[off * dqk + d];
                    z[n] = tau * dot(qrot, kj, dqk);
                    for (int32_t e = 0; e < dv; ++e)
                        vrows[n * dv + e] = fp8 ? oracle_e4m3_value(c->v8[off * dv + e]) * c->v_scale
                                                : (double)c->vf[off * dv + e];
                    vals[n] = vrows + n * dv;
                    ++n;
                }
                z[n] = tau * dot(qrot, knew, dqk);
                for (int32_t e = 0; e < dv; ++e) {
                    const float x = v_new[kv_row * dv + e];
                    if (fp8) {
                        const uint8_t code = oracle_e4m3_code(x * c->v_inv);
                        if (v_code_new && h % group == 0) v_code_new[kv_row * dv + e] = code;
                        vrows[n * dv + e] = oracle_e4m3_value(code) * c->v_scale;
                    } else {
                        vrows[n * dv + e] = (double)x;
                    }
                }
                vals[n] = vrows + n * dv;
                ++n;
                const double sink = sinks ? (double)sinks[h] : -INFINITY;
                attend_row(z, vals, n, dv, sink, p->v_scale, out + ((int64_t)b * Hq + h) * dv);
            }
        }
        free(z);
        free(vrows);
        free(vals);
    }
    return bad ? ORACLE_EINVAL : ORACLE_OK;
}

int oracle_decode(const oracle_params* p, const float* q, const float* k_new, const float* v_new,
                  const int32_t* pos, const float* kc, const float* vc, const int32_t* kpos,
                  const int32_t* count, int32_t L, const float* sinks, double* out,
                  double* k_new_rot, const int32_t* batch_rows, int32_t nbatch_rows) {
    decode_cache c;
    memset(&c, 0, sizeof c);
    c.kf = kc;
    c.vf = vc;
    return decode_core(p, q, k_new, v_new, pos, &c, kpos, count, L, sinks, out, k_new_rot, NULL,
                       NULL, batch_rows, nbatch_rows);
}

/*
 * fp8 KV cache.  The pages only hint at quantized storage ("Add Xiaomi MiMo-V2", "Additional
 * useful info": a garbled note of three dtypes with one quantized); the reading taken here:
 * the caches hold OCP e4m3 codes with one fp32 scale per cache tensor (K and V), rotated K and
 * raw V as before.
 *   e4m3: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 holds the
 *   subnormals m * 2^-9; codes 0x7F and 0xFF are NaN; there are no infinities; the largest
 *   finite magnitude is 448.
 *   Stored value of a code: e4m3(code) * scale.
 *   Code of a value x: y = fp32(x) * fp32(1 / scale) in fp32, clamped to [-448, 448], then the
 *   nearest e4m3 value, ties to the even mantissa (the sign of y is kept, also for zero).
 */
double oracle_e4m3_value(uint8_t c) {
    const int sgn = c >> 7, E = (c >> 3) & 15, M = c & 7;
    if (E == 15 && M == 7) return NAN;
    const double v = E == 0 ? ldexp((double)M, -9) : ldexp((double)(8 + M), E - 10);
    return sgn ? -v : v;
}

uint8_t oracle_e4m3_code(float y) {
    if (isnan(y)) return 0x7F;
    const uint8_t sgn = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    if (a > 448.0) a = 448.0;
    /* spacing of the e4m3 values around a: 2^(e-3) in the binade [2^e, 2^(e+1)), e >= -6;
     * below 2^-6 the subnormal spacing 2^-9 */
    int ex = 0;
    frexp(a, &ex);            /* a = f * 2^ex, f in [0.5, 1) (a > 0) */
    int e = a > 0.0 ? ex - 1 : -6;
    if (e < -6) e = -6;
    const double quantum = ldexp(1.0, e - 3);
    const double v = nearbyint(a / quantum) * quantum;   /* default rounding: ties to even */
    if (v == 0.0) return sgn;
    frexp(v, &ex);
    const int ev = ex - 1;    /* binade of the rounded value (a carry may have moved it up) */
    if (ev < -6) return (uint8_t)(sgn | (uint8_t)(v / ldexp(1.0, -9)));   /* subnormal: m */
    const int mant = (int)((v / ldexp(1.0, ev) - 1.0) * 8.0);
    return (uint8_t)(sgn | ((ev + 7) << 3) | mant);
}

/* Array forms: codes of x[i] * inv_scale (fp32 product), and stored values code * scale. */
int oracle_e4m3_encode(const float* x, int64_t n, float inv_scale, uint8_t* out) {
    if ((n > 0 && (!x || !out)) || n < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_code(x[i] * inv_scale);
    return ORACLE_OK;
}

int oracle_e4m3_decode(const uint8_t* c, int64_t n, double scale, double* out) {
    if ((n > 0 && (!c || !out)) || n < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_value(c[i]) * scale;
    return ORACLE_OK;
}

/*
 * Decode against fp8 caches: as oracle_decode, with the cache entries given as codes
 * kc8 [B,Hkv,L,dqk], vc8 [B,Hkv,L,dv] and their scales, and the new token quantized as the
 * cache stores it before it is attended.  k_code_new [B,Hkv,dqk], v_code_new [B,Hkv,dv]
 * (optional) receive the new token's codes.  Scales must be finite and > 0.
 */
int oracle_decode_fp8(const oracle_params* p, const float* q, const float* k_new,
                      const float* v_new, const int32_t* pos, const uint8_t* kc8,
                      const uint8_t* vc8, const int32_t* kpos, const int32_t* count, int32_t L,
                      double k_scale, double v_scale, const float* sinks, double* out,
                      double* k_new_rot, uint8_t* k_code_new, uint8_t* v_code_new,
                      const int32_t* batch_rows, int32_t nbatch_rows) {
    if (!(k_scale > 0.0 && isfinite(k_scale) && v_scale > 0.0 && isfinite(v_scale)))
        return ORACLE_EINVAL;
    static const uint8_t none = 0;
    decode_cache c;
    memset(&c, 0, sizeof c);
    c.k8 = kc8 ? kc8 : &none;   /* (marks the cache as fp8 also when L = 0) */
    c.v8 = vc8 ? vc8 : &none;
    c.k_scale = (double)(float)k_scale;
    c.v_scale = (double)(float)v_scale;
    c.k_inv = 1.0f / (float)k_scale;
    c.v_inv = 1.0f / (float)v_scale;
    if (L > 0 && (!kc8 || !vc8)) return ORACLE_EINVAL;
    return decode_core(p, q, k_new, v_new, pos, &c, kpos, count, L, sinks, out, k_new_rot,
                       k_code_new, v_code_new, batch_rows, nbatch_rows);
}

/*
 * Extend (chunked prefill): S new tokens per sequence against previously cached keys.
 *   The cache is the position -> (rotated key, value) map of oracle_decode: kc [B,Hkv,L,dqk],
 *   vc [B,Hkv,L,dv], kpos [B,L], count [B].
 *   q [B,S,Hq,dqk], k [B,S,Hkv,dqk] (raw, not rotated), v [B,S,Hkv,dv]; start [B]: new token i
 *   of sequence b sits at position start[b] + i, and its key is rotated there.
 *   Visible to new token i: the cached entries at positions before start[b] that the mask
 *   admits (entries at positions >= start[b] are ignored), and the new tokens j <= i that the
 *   mask admits.  Same definition as prefill, with the cached entries as extra keys.
 *   out [B,S,Hq,dv]; k_rot_out [B,S,Hkv,dqk] optional (rotated new keys); rows/nrows: optional
 *   subset of query indices (others untouched).
 */
int oracle_extend(const oracle_params* p, int32_t S, const float* q, const float* k,
                  const float* v, const int32_t* start, const float* kc, const float* vc,
                  const int32_t* kpos, const int32_t* count, int32_t L, const float* sinks,
                  double* out, const int32_t* rows, int32_t nrows, double* k_rot_out) {
    if (check_params(p) != ORACLE_OK || S < 0 || !q || !k || !v || !start || !out || L < 0)
        return ORACLE_EINVAL;
    if (L > 0 && (!kc || !vc || !kpos || !count)) return ORACLE_EINVAL;
    const int32_t B = p->batch, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
    const int32_t dqk = p->qk_head_dim, dv = p->v_head_dim, r = p->rope_dims;
    const int32_t group = Hq / Hkv;
    const int32_t nr = rows ? nrows : S;
    if (rows)
        for (int32_t t = 0; t < nrows; ++t)
            if (rows[t] < 0 || rows[t] >= S) return ORACLE_EINVAL;
    for (int32_t b = 0; b < B; ++b)
        if (start[b] < 0 || (L > 0 && (count[b] < 0 || count[b] > L))) return ORACLE_EINVAL;
    const double tau = score_scale(p);
    double omega[4096];
    if (r / 2 > 4096) return ORACLE_EINVAL;
    oracle_rope_omega(r, p->rope_theta, omega);

    /* rotate every new key once at its own position; widen the new values */
    const int64_t nk = (int64_t)B * S * Hkv;
    double* kr = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * dqk);
    double* vd = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * dv);
    if (!kr || !vd) { free(kr); free(vd); return ORACLE_EINVAL; }
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < nk; ++t) {
        const int64_t b = t / ((int64_t)S * Hkv), s = (t / Hkv) % S;
        double tmp[4096];
        for (int32_t d = 0; d < dqk; ++d) tmp[d] = (double)k[t * dqk + d];
        rotate_row(tmp, kr + t * dqk, dqk, r, omega, (double)(start[b] + s));
        for (int32_t e = 0; e < dv; ++e) vd[t * dv + e] = (double)v[t * dv + e];
    }
    if (k_rot_out) memcpy(k_rot_out, kr, sizeof(double) * (size_t)nk * dqk);

    const int64_t work = (int64_t)B * Hq * nr;
    int bad = 0;
    #pragma omp parallel
    {
        const int64_t cap = (int64_t)L + S + 1;
        double* z = (double*)malloc(sizeof(double) * (size_t)cap);
        double* crow = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * dv);
        const double** vals = (const double**)malloc(sizeof(double*) * (size_t)cap);
        double qraw[4096], qrot[4096], kj[4096];
        if (!z || !crow || !vals) {
            #pragma omp atomic write
            bad = 1;
        } else {
            #pragma omp for schedule(dynamic, 4)
            for (int64_t w = 0; w < work; ++w) {
                const int32_t b = (int32_t)(w / ((int64_t)Hq * nr));
                const int32_t h = (int32_t)((w / nr) % Hq);
                const int32_t i = rows ? rows[w % nr] : (int32_t)(w % nr);
                const int32_t g = h / group;
                const int64_t pq = (int64_t)start[b] + i;
                for (int32_t d = 0; d < dqk; ++d)
                    qraw[d] = (double)q[(((int64_t)b * S + i) * Hq + h) * dqk + d];
                rotate_row(qraw, qrot, dqk, r, omega, (double)pq);
                int64_t n = 0;
                const int32_t cnt = L > 0 ? count[b] : 0;
                for (int32_t j = 0; j < cnt; ++j) {   /* cached keys */
                    const int64_t pk = kpos[(int64_t)b * L + j];
                    if (pk >= start[b] || !visible(p, pq, pk)) continue;
                    const int64_t off = ((int64_t)b * Hkv + g) * L + j;
                    for (int32_t d = 0; d < dqk; ++d) kj[d] = (double)kc[off * dqk + d];
                    z[n] = tau * dot(qrot, kj, dqk);
                    for (int32_t e = 0; e < dv; ++e) crow[n * dv + e] = (double)vc[off * dv + e];
                    vals[n] = crow + n * dv;
                    ++n;
                }
                for (int32_t j = 0; j <= i; ++j) {    /* new keys */
                    if (!visible(p, pq, (int64_t)start[b] + j)) continue;
                    const int64_t kv = ((int64_t)b * S + j) * Hkv + g;
                    z[n] = tau * dot(qrot, kr + kv * dqk, dqk);
                    vals[n] = vd + kv * dv;
                    ++n;
                }
                const double sink = sinks ? (double)sinks[h] : -INFINITY;
                attend_row(z, vals, n, dv, sink, p->v_scale,
                           out + (((int64_t)b * S + i) * Hq + h) * dv);
            }
        }
        free(z);
        free(crow);
        free(vals);
    }
    free(kr);
    free(vd);
    return bad ? ORACLE_EINVAL : ORACLE_OK;
}
