/*
 * moe_oracle.c -- plain CPU reference for the sparse mixture-of-experts
 * feed-forward layer, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  The GPU library
 * never includes, links or calls it, and the two share no code.
 *
 * What is computed, per token (Mixtral of Experts, wikillm.com card,
 * "Method", sparse MoE layer of section 2.1 and the two pseudocode blocks):
 *   1. router: one logit per expert from a bias-free linear map of the token
 *      (section 2.1, steps-for-one-token item 2);
 *   2. keep the K largest logits and take a softmax over those K only, so the
 *      kept weights sum to one and the other experts add nothing
 *      (section 2.1 display 2; "Pitfalls": renormalised top-2 weights);
 *   3. each kept expert is a SwiGLU block: SiLU on the w1 branch, times the
 *      linear w3 branch, then the w2 down-projection (SwiGLU pseudocode);
 *   4. output = sum over the kept experts of gate * expert(x), starting from
 *      zero (section 2.1 displays 1 and 3; moe_feed_forward pseudocode).
 *
 * Storage is row-major with the products written as x.W:
 *   x [T,d], w_router [d,E], w1 and w3 [E,d,f], w2 [E,f,d].
 * The pages write the same products as W.x with the transposed shapes
 * (router (n_experts, dim); w1, w3 (hidden, dim); w2 (dim, hidden)).
 *
 * Readings taken where the pages are silent:
 *   - top-k ties break toward the lower expert index, and the kept experts
 *     are listed by descending logit;
 *   - the selection compares logits rounded to binary32, the precision the
 *     GPU kernel keeps them in, so both sides take that decision in the same
 *     precision; the softmax itself uses the double-precision logits;
 *   - an optional per-expert additive logit bias is supported for a skewed-
 *     routing workload; with bias == NULL the router is bias-free as stated.
 *
 * Inputs are either binary32 (dtype 0) or bfloat16 bit patterns (dtype 1);
 * both widen to double exactly, so the oracle consumes the same values the
 * GPU does.  Every result is double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_oracle.h"
#ifdef _OPENMP
#include <omp.h>
#endif

/* Widen element i of a binary32 or bfloat16 array to double (exact). */
static double elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float v;
    memcpy(&v, &bits, sizeof v);
    return (double)v;
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)). */
static double silu(double z)
{
    return z / (1.0 + exp(-z));
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Router logits for token t: l[e] = sum_i x[t,i] * w_router[i,e] (+ bias[e]).
 */
static void router_logits_one(const void *x, const void *w_router, const float *bias,
                              int dtype, int64_t t, int64_t d, int64_t E, double *l)
{
    for (int64_t e = 0; e < E; ++e)
        l[e] = 0.0;
    for (int64_t i = 0; i < d; ++i) {
        double xi = elem(x, dtype, t * d + i);
        for (int64_t e = 0; e < E; ++e)
            l[e] += xi * elem(w_router, dtype, i * E + e);
    }
    if (bias)
        for (int64_t e = 0; e < E; ++e)
            l[e] += (double)bias[e];
}

/*
 * Top-k selection and softmax over the kept logits (section 2.1 display 2).
 * The j-th pick is the largest binary32-rounded logit among the experts not
 * yet picked; a strict '>' while scanning experts in ascending order makes
 * the lowest index win a tie.  Gates: g_j = exp(l_j - l_max) / sum_m exp(l_m - l_max)
 * over the k picks, in double.
 */
static void topk_softmax_one(const double *l, int64_t E, int64_t k, int32_t *ids, double *gates)
{
    unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
    for (int64_t j = 0; j < k; ++j) {
        int64_t best = -1;
        float best_v = 0.0f;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            float v = (float)l[e];
            if (best < 0 || v > best_v) {
                best = e;
                best_v = v;
            }
        }
        taken[best] = 1;
        ids[j] = (int32_t)best;
    }
    free(taken);
    double lmax = l[ids[0]];
    for (int64_t j = 1; j < k; ++j)
        if (l[ids[j]] > lmax)
            lmax = l[ids[j]];
    double z = 0.0;
    for (int64_t j = 0; j < k; ++j) {
        gates[j] = exp(l[ids[j]] - lmax);
        z += gates[j];
    }
    for (int64_t j = 0; j < k; ++j)
        gates[j] /= z;
}

/*
 * Routing for every token: logits [T,E] (optional), ids [T,k], gates [T,k].
 */
int oracle_route(const void *x, const void *w_router, const float *bias, int dtype,
                 int64_t T, int64_t d, int64_t E, int64_t k,
                 double *logits, int32_t *ids, double *gates)
{
    if (k < 1 || k > E || T < 0)
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double *l = (double *)malloc((size_t)E * sizeof(double));
        router_logits_one(x, w_router, bias, dtype, t, d, E, l);
        topk_softmax_one(l, E, k, ids + t * k, gates + t * k);
        if (logits)
            memcpy(logits + t * E, l, (size_t)E * sizeof(double));
        free(l);
    }
    return 0;
}

/*
 * One SwiGLU expert e on one token row xr (SwiGLU pseudocode):
 *   a = xr . w1[e]   (length f)      b = xr . w3[e]   (length f)
 *   h = SiLU(a) * b                  y = h . w2[e]    (length d)
 * xr is a row of x given as (base, row index).  h may be NULL.
 */
static void swiglu_expert_one(const void *x, int64_t row, const void *w1, const void *w3,
                              const void *w2, int dtype, int64_t d, int64_t f, int64_t e,
                              double *h, double *y)
{
    double *a = (double *)calloc((size_t)f, sizeof(double));
    double *b = (double *)calloc((size_t)f, sizeof(double));
    const int64_t w13_base = e * d * f;
    for (int64_t i = 0; i < d; ++i) {
        double xi = elem(x, dtype, row * d + i);
        for (int64_t j = 0; j < f; ++j) {
            a[j] += xi * elem(w1, dtype, w13_base + i * f + j);
            b[j] += xi * elem(w3, dtype, w13_base + i * f + j);
        }
    }
    for (int64_t j = 0; j < f; ++j)
        a[j] = silu(a[j]) * b[j]; /* a now holds h */
    const int64_t w2_base = e * f * d;
    for (int64_t c = 0; c < d; ++c)
        y[c] = 0.0;
    for (int64_t j = 0; j < f; ++j) {
        double hj = a[j];
        for (int64_t c = 0; c < d; ++c)
            y[c] += hj * elem(w2, dtype, w2_base + j * d + c);
    }
    if (h)
        memcpy(h, a, (size_t)f * sizeof(double));
    free(a);
    free(b);
}

/*
 * The whole layer for a list of tokens (tokens == NULL means 0..n-1).
 *   out   [n,d]    layer output per listed token
 *   ids   [n,k]    selected experts (written when routing here, read when forced)
 *   gates [n,k]    their weights    (same)
 *   y     [n,k,d]  optional: expert outputs before gating, per slot
 *   h     [n,k,f]  optional: SwiGLU activations per slot
 * forced != 0 skips the router and uses the caller's ids/gates, so a token can
 * be checked against a selection made elsewhere (x and the weights are still
 * this layer's).
 */
int oracle_moe_tokens(const void *x, const void *w_router, const float *bias,
                      const void *w1, const void *w3, const void *w2, int dtype,
                      int64_t T, int64_t d, int64_t f, int64_t E, int64_t k,
                      const int64_t *tokens, int64_t n, int forced,
                      int32_t *ids, double *gates, double *out, double *y, double *h)
{
    if (k < 1 || k > E || n < 0)
        return 1;
    for (int64_t s = 0; s < n; ++s) {
        int64_t t = tokens ? tokens[s] : s;
        if (t < 0 || t >= T)
            return 2;
        if (forced)
            for (int64_t j = 0; j < k; ++j)
                if (ids[s * k + j] < 0 || ids[s * k + j] >= E)
                    return 3;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < n; ++s) {
        int64_t t = tokens ? tokens[s] : s;
        int32_t *id = ids + s * k;
        double *g = gates + s * k;
        if (!forced) {
            double *l = (double *)malloc((size_t)E * sizeof(double));
            router_logits_one(x, w_router, bias, dtype, t, d, E, l);
            topk_softmax_one(l, E, k, id, g);
            free(l);
        }
        double *ye = (double *)malloc((size_t)d * sizeof(double));
        double *o = out + s * d;
        for (int64_t c = 0; c < d; ++c)
            o[c] = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            double *hj = h ? h + (s * k + j) * f : NULL;
            swiglu_expert_one(x, t, w1, w3, w2, dtype, d, f, id[j], hj, ye);
            for (int64_t c = 0; c < d; ++c)
                o[c] += g[j] * ye[c];
            if (y)
                memcpy(y + (s * k + j) * d, ye, (size_t)d * sizeof(double));
        }
        free(ye);
    }
    return 0;
}

/*
 * RMSNorm with unit gain, used by the stacked-block workload
 * h = h + MoE(RMSNorm(h)):  out[t,i] = h[t,i] / sqrt(mean_i(h[t,i]^2) + eps).
 * The pages leave the normalisation to the code; eps is the caller's.
 */
int oracle_rmsnorm(const void *hsrc, int dtype, int64_t T, int64_t d, double eps, double *out)
{
    if (T < 0 || d < 1)
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int64_t i = 0; i < d; ++i) {
            double v = elem(hsrc, dtype, t * d + i);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)d + eps);
        for (int64_t i = 0; i < d; ++i)
            out[t * d + i] = elem(hsrc, dtype, t * d + i) * r;
    }
    return 0;
}
