/*
 * Plain C CPU oracle of the Quant Experts (QE) linear-layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct definition
 * of what the hot path computes, written as straight loops over tokens, channels and
 * output channels in the order the definition states.  Only the test suite, the smoke
 * check of the package entry file and the CPU-baseline leg of the benchmark load the
 * shared library built from it; the product path never does.  It shares no code with
 * the HIP library (no header, helper or table in common) and none with the numpy oracle
 * beside it; the tests compare the two.
 *
 * Sources (the pages, cited by title and section):
 *   DeepRead   MCISLAB DeepRead summary "Quant Experts: Token-aware Adaptive Error
 *              Reconstruction with Mixture of Experts for Large Vision-Language Models
 *              Quantization", section "Method".
 *   PaperDaily longzhangge PaperDaily post "西交大提出Quant Experts：token级量化补偿",
 *              sections "从观察到创新" and "核心设计".
 *   WisPaper   wispaper.ai post on Quant Experts, "Critical Analysis & Insight".
 *   Listing    thelatestinai.com listing of arXiv 2602.24059, Tables 1-3 (bit settings)
 *              and Table 7 (cost of a QE linear).
 *
 * Readings (the same as the numpy oracle's): per-token symmetric activation RTN of x/s
 * with qmax = 2^(b-1)-1; per-output-channel symmetric weight RTN of W_f diag(s) with
 * qmax 7 (W4) or 3 (W3); round half to even; an all-zero token or row has scale 0 and
 * codes 0.  Quantization decisions are taken in float32 with IEEE division, the
 * precision the kernels use.  The shared expert, the router and the routed experts read
 * bf16(x) (unsmoothed); the router picks the smallest score of x.R, lower index on ties;
 * the three terms are summed in parallel.  Integer sums are exact (int64); every other
 * reduction is accumulated in double in index order.  Top-k orders channels by
 * (score desc, index asc) with score = fabsf(x) * w in float32.
 *
 * OpenMP runs over tokens only; each output element is computed by one thread in a
 * fixed order, so results do not depend on the thread count.
 */

#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 rounding of a float32 (round to nearest, ties to even), returned as float32. */
static float bf16_round(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u = (uint32_t)(((uint64_t)u + 0x7FFFu + lsb) & 0xFFFF0000u);
    float r;
    memcpy(&r, &u, 4);
    return r;
}

static int qmax_act(int a_bits) { return a_bits == 6 ? 31 : a_bits == 8 ? 127 : -1; }
static int qmax_w(int w_bits) { return w_bits == 4 ? 7 : w_bits == 3 ? 3 : -1; }

int qo_num_threads(void) { return omp_get_max_threads(); }

void qo_set_threads(int n) { omp_set_num_threads(n); }

/* One token of the activation quantizer (DeepRead "Method": x is divided by the
 * channel-wise smoothing factor before activation quantization). */
static void quant_token(const float* x, const float* s, int64_t d_in, int qmax, int8_t* codes, float* s_x,
                        float* tmp) {
    float amax = 0.0f;
    for (int64_t j = 0; j < d_in; ++j) {
        float v = s ? x[j] / s[j] : x[j];
        tmp[j] = v;
        float a = fabsf(v);
        if (a > amax) amax = a;
    }
    float scale = amax / (float)qmax;
    *s_x = scale;
    for (int64_t j = 0; j < d_in; ++j) {
        if (amax == 0.0f) {
            codes[j] = 0;
            continue;
        }
        float q = rintf(tmp[j] / scale);
        if (q > (float)qmax) q = (float)qmax;
        if (q < -(float)qmax) q = -(float)qmax;
        codes[j] = (int8_t)q;
    }
}

/* Activation codes and per-token scales.  x [T, d_in] float32, s [d_in] or NULL. */
int qo_quant_act(const float* x, const float* s, int64_t T, int64_t d_in, int a_bits, int8_t* codes, float* s_x) {
    int qmax = qmax_act(a_bits);
    if (qmax < 0) return -1;
#pragma omp parallel
    {
        float* tmp = (float*)malloc(sizeof(float) * (size_t)(d_in > 0 ? d_in : 1));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) quant_token(x + t * d_in, s, d_in, qmax, codes + t * d_in, s_x + t, tmp);
        free(tmp);
    }
    return 0;
}

/* Weight codes and per-output-channel scales of W' = W_f diag(s) (DeepRead "Method": the
 * weights are amplified by the factor the activations are divided by). */
int qo_quant_weights(const float* W, const float* s, int64_t d_out, int64_t d_in, int w_bits, int8_t* codes,
                     float* s_w) {
    int qmax = qmax_w(w_bits);
    if (qmax < 0) return -1;
#pragma omp parallel
    {
        float* tmp = (float*)malloc(sizeof(float) * (size_t)(d_in > 0 ? d_in : 1));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < d_out; ++i) {
            const float* row = W + i * d_in;
            float amax = 0.0f;
            for (int64_t j = 0; j < d_in; ++j) {
                float v = s ? row[j] * s[j] : row[j];
                tmp[j] = v;
                if (fabsf(v) > amax) amax = fabsf(v);
            }
            float scale = amax / (float)qmax;
            s_w[i] = scale;
            for (int64_t j = 0; j < d_in; ++j) {
                int8_t c = 0;
                if (amax != 0.0f) {
                    float q = rintf(tmp[j] / scale);
                    if (q > (float)qmax) q = (float)qmax;
                    if (q < -(float)qmax) q = -(float)qmax;
                    c = (int8_t)q;
                }
                codes[i * d_in + j] = c;
            }
        }
        free(tmp);
    }
    return 0;
}

/* Integer accumulators acc[t][i] = sum_j qx[t][j] qw[i][j] (Listing Table 7: the s d^2 term).
 * Returns 1 if any sum leaves the int32 range (the value is then not stored exactly). */
int qo_main_acc(const int8_t* qx, const int8_t* qw, int64_t T, int64_t d_in, int64_t d_out, int32_t* acc) {
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t i = 0; i < d_out; ++i) {
            int64_t a = 0;
            for (int64_t j = 0; j < d_in; ++j) a += (int64_t)qx[t * d_in + j] * (int64_t)qw[i * d_in + j];
            if (a > INT32_MAX || a < INT32_MIN) overflow = 1;
            acc[t * d_out + i] = (int32_t)a;
        }
    }
    return overflow;
}

/* Router of one token: scores sc[e] = sum_j xb[j] R[j][e] in double; the expert is the
 * first smallest score (DeepRead "Method", routed experts: the router estimates each
 * expert's remaining error and picks the smallest; Listing Table 7: one d x N_r map).
 * margin = second smallest minus smallest; scale = max(|smallest|, |second|). */
static int route_token(const float* xb, const float* R, int64_t d_in, int n_r, double* sc, double* margin,
                       double* scale) {
    for (int e = 0; e < n_r; ++e) sc[e] = 0.0;
    for (int64_t j = 0; j < d_in; ++j)
        for (int e = 0; e < n_r; ++e) sc[e] += (double)xb[j] * (double)R[j * n_r + e];
    int best = 0;
    for (int e = 1; e < n_r; ++e)
        if (sc[e] < sc[best]) best = e;
    if (n_r >= 2) {
        int second = -1;
        for (int e = 0; e < n_r; ++e) {
            if (e == best) continue;
            if (second < 0 || sc[e] < sc[second]) second = e;
        }
        *margin = sc[second] - sc[best];
        *scale = fmax(fabs(sc[best]), fabs(sc[second]));
    } else {
        *margin = INFINITY;
        *scale = 0.0;
    }
    return best;
}

/* Bucketing of the routes: counts per expert, exclusive offsets, and the tokens listed in
 * (expert, token) order. */
static void bucket(const int32_t* expert, int64_t T, int n_r, int32_t* counts, int32_t* offsets, int32_t* perm) {
    for (int e = 0; e < n_r; ++e) counts[e] = 0;
    for (int64_t t = 0; t < T; ++t) counts[expert[t]]++;
    offsets[0] = 0;
    for (int e = 0; e < n_r; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t pos = 0;
    for (int e = 0; e < n_r; ++e)
        for (int64_t t = 0; t < T; ++t)
            if (expert[t] == e) perm[pos++] = (int32_t)t;
}

/* Router and bucketing over T tokens of bf16-valued x.  scores [T, n_r] (nullable). */
int qo_route(const float* xb, const float* R, int64_t T, int64_t d_in, int n_r, double* scores, int32_t* expert,
             double* margin, double* margin_scale, int32_t* counts, int32_t* offsets, int32_t* perm) {
    if (n_r <= 0) return -1;
#pragma omp parallel
    {
        double* sc = (double*)malloc(sizeof(double) * (size_t)n_r);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            expert[t] = route_token(xb + t * d_in, R, d_in, n_r, sc, margin + t, margin_scale + t);
            if (scores)
                for (int e = 0; e < n_r; ++e) scores[t * n_r + e] = sc[e];
        }
        free(sc);
    }
    bucket(expert, T, n_r, counts, offsets, perm);
    return 0;
}

/* (x.A).B of one token in double: u[m] = sum_j xb[j] A[j][m]; out[i] += sum_m u[m] B[m][i]. */
static void lowrank_token(const float* xb, int64_t d_in, const float* A, const float* B, int r, int64_t d_out,
                          double* u, double* out) {
    for (int m = 0; m < r; ++m) u[m] = 0.0;
    for (int64_t j = 0; j < d_in; ++j)
        for (int m = 0; m < r; ++m) u[m] += (double)xb[j] * (double)A[j * r + m];
    for (int64_t i = 0; i < d_out; ++i) {
        double a = 0.0;
        for (int m = 0; m < r; ++m) a += u[m] * (double)B[(int64_t)m * d_out + i];
        out[i] = a;
    }
}

/*
 * One QE linear (DeepRead "Method": every token uses the fixed shared expert plus the one
 * routed expert the router picks; PaperDaily "核心设计": the compensations are added):
 *   y[t] = main[t] + SE(bf16(x_t)) + RE_{e_t}(bf16(x_t)).
 * main[t][i] = acc[t][i] * s_x[t] * s_w[i] for A6/A8 (acc over the activation codes), or
 * s_w[i] * sum_j bf16(x)[t][j] qw[i][j] for A16 (no smoothing, no activation quantization).
 * x [T, d_in] float32 values (bf16-representable when x_is_bf16); qw [d_out, d_in] codes;
 * A_s [d_in, r_s], B_s [r_s, d_out], A_r [n_r, d_in, r_r], B_r [n_r, r_r, d_out],
 * R [d_in, n_r] (float32 arrays of bf16 values; r_s = 0 or n_r = 0 drops the term).
 * expert_override [T] (nullable) replaces the router's choice.  Outputs: y [T, d_out]
 * double; expert, margin, margin_scale [T] (when n_r > 0); codes [T, d_in], s_x [T] and
 * acc [T, d_out] (each nullable, A6/A8 only).  Returns 1 if an accumulator overflows int32.
 */
int qo_qe_linear(const float* x, int x_is_bf16, const float* s, const int8_t* qw, const float* s_w, int64_t T,
                 int64_t d_in, int64_t d_out, int a_bits, int r_s, const float* A_s, const float* B_s, int n_r,
                 int r_r, const float* A_r, const float* B_r, const float* R, const int32_t* expert_override,
                 double* y, int32_t* expert, double* margin, double* margin_scale, int8_t* codes, float* s_x,
                 int32_t* acc) {
    int qmax = a_bits == 16 ? 0 : qmax_act(a_bits);
    if (qmax < 0) return -1;
    int overflow = 0;
    int rmax = (r_s > r_r ? r_s : r_r) + 1;
#pragma omp parallel reduction(| : overflow)
    {
        float* xb = (float*)malloc(sizeof(float) * (size_t)d_in);
        float* tmp = (float*)malloc(sizeof(float) * (size_t)d_in);
        int8_t* q = (int8_t*)malloc((size_t)d_in);
        double* u = (double*)malloc(sizeof(double) * (size_t)rmax);
        double* sc = (double*)malloc(sizeof(double) * (size_t)(n_r > 0 ? n_r : 1));
        double* term = (double*)malloc(sizeof(double) * (size_t)d_out);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const float* xt = x + t * d_in;
            double* yt = y + t * d_out;
            for (int64_t j = 0; j < d_in; ++j) xb[j] = x_is_bf16 ? xt[j] : bf16_round(xt[j]);
            if (a_bits == 16) {
                for (int64_t i = 0; i < d_out; ++i) {
                    double a = 0.0;
                    for (int64_t j = 0; j < d_in; ++j) a += (double)xb[j] * (double)qw[i * d_in + j];
                    yt[i] = a * (double)s_w[i];
                }
            } else {
                float sx;
                quant_token(xt, s, d_in, qmax, q, &sx, tmp);
                if (codes) memcpy(codes + t * d_in, q, (size_t)d_in);
                if (s_x) s_x[t] = sx;
                for (int64_t i = 0; i < d_out; ++i) {
                    int64_t a = 0;
                    for (int64_t j = 0; j < d_in; ++j) a += (int64_t)q[j] * (int64_t)qw[i * d_in + j];
                    if (a > INT32_MAX || a < INT32_MIN) overflow = 1;
                    if (acc) acc[t * d_out + i] = (int32_t)a;
                    yt[i] = (double)a * (double)sx * (double)s_w[i];
                }
            }
            if (r_s > 0) {
                lowrank_token(xb, d_in, A_s, B_s, r_s, d_out, u, term);
                for (int64_t i = 0; i < d_out; ++i) yt[i] += term[i];
            }
            if (n_r > 0) {
                double mg, ms;
                int e = route_token(xb, R, d_in, n_r, sc, &mg, &ms);
                if (expert) expert[t] = e;
                if (margin) margin[t] = mg;
                if (margin_scale) margin_scale[t] = ms;
                if (expert_override) e = expert_override[t];
                if (r_r > 0) {
                    lowrank_token(xb, d_in, A_r + (int64_t)e * d_in * r_r, B_r + (int64_t)e * r_r * d_out, r_r, d_out,
                                  u, term);
                    for (int64_t i = 0; i < d_out; ++i) yt[i] += term[i];
                }
            }
        }
        free(xb);
        free(tmp);
        free(q);
        free(u);
        free(sc);
        free(term);
    }
    return overflow;
}

typedef struct {
    float score;
    int32_t index;
} scored_channel;

/* (score desc, index asc) */
static int by_score_then_index(const void* a, const void* b) {
    const scored_channel* p = (const scored_channel*)a;
    const scored_channel* q = (const scored_channel*)b;
    if (p->score > q->score) return -1;
    if (p->score < q->score) return 1;
    return (p->index > q->index) - (p->index < q->index);
}

/*
 * Per-token Top-k(|x_t| * w) and the channel-frequency histogram (DeepRead "Method", first
 * paragraph; PaperDaily "从观察到创新").  score = fabsf(x) * w in float32; the k first
 * channels of the full sort under (score desc, index asc).  topk [T, k] (nullable);
 * hist [d_in] is overwritten with the selection counts.
 */
int qo_channel_topk(const float* x, const float* w, int64_t T, int64_t d_in, int k, int32_t* topk, int64_t* hist) {
    if (k < 1 || k > d_in) return -1;
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * (size_t)k);
#pragma omp parallel
    {
        scored_channel* buf = (scored_channel*)malloc(sizeof(scored_channel) * (size_t)d_in);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t j = 0; j < d_in; ++j) {
                buf[j].score = fabsf(x[t * d_in + j]) * w[j];
                buf[j].index = (int32_t)j;
            }
            qsort(buf, (size_t)d_in, sizeof(scored_channel), by_score_then_index);
            for (int m = 0; m < k; ++m) sel[t * k + m] = buf[m].index;
        }
        free(buf);
    }
    for (int64_t j = 0; j < d_in; ++j) hist[j] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int m = 0; m < k; ++m) hist[sel[t * k + m]]++;
    if (topk) memcpy(topk, sel, sizeof(int32_t) * (size_t)T * (size_t)k);
    free(sel);
    return 0;
}

/* Mean over output rows of |W_f|: one value per input channel, summed in double, divided
 * by d_out and rounded once to float32 (DeepRead "Method": w = Mean_row(|W_f|)). */
int qo_colmean_abs(const float* W, int64_t d_out, int64_t d_in, float* w) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < d_in; ++j) {
        double a = 0.0;
        for (int64_t i = 0; i < d_out; ++i) a += fabs((double)W[i * d_in + j]);
        w[j] = (float)(a / (double)d_out);
    }
    return 0;
}
