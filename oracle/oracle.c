/*
 * oracle.c -- plain, slow CPU oracle of the fused MoE-LoRA layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two meet only through
 * the seeded inputs handed to both.
 *
 * What it computes (all accumulation in IEEE fp64, fixed left-to-right
 * order, no blocking or fusion):
 *
 *  route   top-K experts per token from fp32 router logits, softmax weights
 *          over the selected logits, then S always-on shared slots appended
 *          after the routed ones with ids E..E+S-1 and weight 1/rsf.
 *          (aitrends.kr summary of the AWS multi-LoRA MoE post, "section
 *          details": a router sends each token to its experts;
 *          secrett2633 analysis of vLLM PR 46545, "code analysis" part 1:
 *          shared ids start at the routed expert count and every shared slot
 *          carries one constant weight; "lessons" item 2: that weight is
 *          1/routed_scaling_factor.)
 *  route (biased variant) sigmoid or full-softmax expert scores in fp64, a
 *          per-expert bias added for the choice only, the weights taken from
 *          the unbiased scores of the chosen experts (route_token_bias).
 *  align   stable counting sort of the (token, slot) pairs by expert, the
 *          expert count being the number of stacked w13 rows (same analysis,
 *          "code analysis" part 2), each expert group padded to a multiple of
 *          the block size.  Inside an expert group the pairs are ordered by
 *          adapter (no-LoRA first) and then by pair index; the LoRA work
 *          items are the (adapter, expert) runs cut into pieces of at most
 *          the LoRA block size.  The in-group order, sentinel and padding are
 *          not on the pages; this is the layout contract with the kernels.
 *  forward per token and slot: g = W13[e] x (+ B13[a,e] A13[a,e] x when the
 *          token has an adapter), h = silu(g[:I]) * g[I:], y = W2[e] h
 *          (+ B2[a,e] A2[a,e] h), out = rsf * sum_j w_j y_j.  LoRA shrink (A)
 *          and expand (B) sit on both the gate_up and the down projection
 *          (AWS post summary, "image analysis", diagram).
 *
 *  mxfp8   decode of MXFP8 expert weights (the experts module of the ROCm
 *          path in the PR 46545 analysis, "code analysis" part 2, is the
 *          mxfp8 one; the pages do not define the format, and the reading
 *          taken is the MX one): every element is an FP8 E4M3 code (sign,
 *          4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
 *          subnormal, exponent 15 with mantissa 7 is NaN, no infinities)
 *          times 2^(s - 127) for the E8M0 scale byte s of its block of 32
 *          consecutive elements along the reduction.  The layer forward then
 *          runs on the decoded weights unchanged.
 *
 * Floating point inputs arrive either as fp32 or as raw bf16 bit patterns
 * (uint16); both are widened exactly to fp64 before use.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

static double widen_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double ld(const void *p, int64_t i, int dtype)
{
    if (dtype == ORACLE_BF16)
        return widen_bf16(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

/* ---------------------------------------------------------------- route */

/* Route one token.  Selection: repeat K times "take the largest logit not yet
 * taken; on an exact tie the lower expert index wins" (a strict > scan in
 * index order does exactly that; +0 and -0 compare equal).  Slot order is
 * selection order.  Weights: softmax of the selected logits (renormalize=1)
 * or the full softmax over all E logits restricted to the selected ones
 * (renormalize=0), exp and sums in fp64 after subtracting the top logit,
 * rounded once to fp32. */
static void route_token(const float *l, int64_t E, int64_t K, int64_t S, float rsf, int renorm,
                        int32_t *ids, float *w, unsigned char *taken, double *ex)
{
    int64_t Kp = K + S;
    memset(taken, 0, (size_t)E);
    for (int64_t j = 0; j < K; ++j) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || l[e] > l[best])
                best = e;
        }
        taken[best] = 1;
        ids[j] = (int32_t)best;
    }
    double m = (double)l[ids[0]];
    double s = 0.0;
    for (int64_t j = 0; j < K; ++j)
        ex[j] = exp((double)l[ids[j]] - m);
    if (renorm) {
        for (int64_t j = 0; j < K; ++j)
            s += ex[j];
    } else {
        for (int64_t e = 0; e < E; ++e)
            s += exp((double)l[e] - m);
    }
    for (int64_t j = 0; j < K; ++j)
        w[j] = (float)(ex[j] / s);
    for (int64_t q = 0; q < S; ++q) {
        ids[K + q] = (int32_t)(E + q);
        w[K + q] = 1.0f / rsf;
    }
    (void)Kp;
}

/* Biased router (the router module named in the PR 46545 analysis, "code
 * analysis" part 1, is a top-k router with a bias; the page does not define
 * it, and the reading taken is the plainest one that keeps the routing
 * weights meaningful):
 *   score  s_e = 1 / (1 + exp(-l_e))                      scoring = sigmoid
 *          s_e = exp(l_e - m) / sum_e' exp(l_e' - m)       scoring = softmax
 *          (m the largest logit, the sum in expert index order)
 *   key    k_e = s_e + b_e    (b the per-expert bias, 0 when absent)
 *   choose K experts by repeated "largest key not yet taken, lower expert
 *          index on an exact tie"; slot order = selection order
 *   weight w_j = s_j / sum_{j' < K} s_j'   (renormalize = 1, slot order)
 *          w_j = s_j                       (renormalize = 0)
 * The bias steers the choice only; the weights use the unbiased scores.
 * Everything is fp64; each weight is rounded once to fp32.  Shared slots
 * are appended as in route_token. */
static void route_token_bias(const float *l, const float *bias, int64_t E, int64_t K, int64_t S, float rsf,
                             int renorm, int scoring, int32_t *ids, float *w, unsigned char *taken,
                             double *score)
{
    double den = 1.0, m = 0.0;
    if (scoring == 0) {
        m = (double)l[0];
        for (int64_t e = 1; e < E; ++e)
            if ((double)l[e] > m)
                m = (double)l[e];
        den = 0.0;
        for (int64_t e = 0; e < E; ++e)
            den += exp((double)l[e] - m);
    }
    for (int64_t e = 0; e < E; ++e)
        score[e] = scoring == 0 ? exp((double)l[e] - m) / den : 1.0 / (1.0 + exp(-(double)l[e]));
    memset(taken, 0, (size_t)E);
    for (int64_t j = 0; j < K; ++j) {
        int64_t best = -1;
        double bk = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            double k = score[e] + (bias ? (double)bias[e] : 0.0);
            if (best < 0 || k > bk) {
                best = e;
                bk = k;
            }
        }
        taken[best] = 1;
        ids[j] = (int32_t)best;
    }
    double s = 0.0;
    for (int64_t j = 0; j < K; ++j)
        s += score[ids[j]];
    for (int64_t j = 0; j < K; ++j)
        w[j] = (float)(renorm ? score[ids[j]] / s : score[ids[j]]);
    for (int64_t q = 0; q < S; ++q) {
        ids[K + q] = (int32_t)(E + q);
        w[K + q] = 1.0f / rsf;
    }
}

/* scoring: -1 = the plain router (route_token; bias must be NULL), 0 =
 * softmax scores, 1 = sigmoid scores (route_token_bias; bias may be NULL). */
int oracle_route_bias(int64_t T, int64_t E, int64_t K, int64_t S, float rsf, int renorm, int scoring,
                      const float *logits, const float *bias, int32_t *topk_ids, float *topk_w)
{
    if (T < 0 || E <= 0 || K <= 0 || K > E || S < 0 || scoring < -1 || scoring > 1 ||
        (scoring < 0 && bias != NULL))
        return -1;
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    double *sc = (double *)malloc(sizeof(double) * (size_t)(E > K ? E : K));
    if (!taken || !sc) {
        free(taken);
        free(sc);
        return -2;
    }
    int64_t Kp = K + S;
    for (int64_t t = 0; t < T; ++t) {
        if (scoring < 0)
            route_token(logits + t * E, E, K, S, rsf, renorm, topk_ids + t * Kp, topk_w + t * Kp, taken, sc);
        else
            route_token_bias(logits + t * E, bias, E, K, S, rsf, renorm, scoring, topk_ids + t * Kp,
                             topk_w + t * Kp, taken, sc);
    }
    free(taken);
    free(sc);
    return 0;
}

int oracle_route(int64_t T, int64_t E, int64_t K, int64_t S, float rsf, int renorm,
                 const float *logits, int32_t *topk_ids, float *topk_w)
{
    if (T < 0 || E <= 0 || K <= 0 || K > E || S < 0)
        return -1;
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    double *ex = (double *)malloc(sizeof(double) * (size_t)K);
    if (!taken || !ex) {
        free(taken);
        free(ex);
        return -2;
    }
    int64_t Kp = K + S;
    for (int64_t t = 0; t < T; ++t)
        route_token(logits + t * E, E, K, S, rsf, renorm, topk_ids + t * Kp, topk_w + t * Kp, taken, ex);
    free(taken);
    free(ex);
    return 0;
}

/* ---------------------------------------------------------------- align */

/* Capacity bounds used by both sides of the layout contract:
 *   blocks <= ceil(P/bm) + min(Ep, P),  sorted capacity = blocks * bm,
 *   items  <= ceil(P/lbm) + min(P, La*Ep). */
int64_t oracle_max_blocks(int64_t P, int64_t Ep, int64_t bm)
{
    int64_t nz = Ep < P ? Ep : P;
    return (P + bm - 1) / bm + nz;
}

int64_t oracle_max_items(int64_t P, int64_t Ep, int64_t La, int64_t lbm)
{
    int64_t bins = La * Ep;
    int64_t nz = bins < P ? bins : P;
    return (P + lbm - 1) / lbm + nz;
}

/* Stable counting sort of pairs f = t*Kp + j by key = e*(La+1) + (a+1),
 * a = adapter of token t (or -1; La = 0 when LoRA is off).  Expert groups
 * (all keys of one e) are padded to a multiple of bm with the sentinel P.
 * Outputs:
 *   sorted_ids[cap]            pair index or P (padding and tail)
 *   block_expert[max_blocks]   expert of each block of bm rows, -1 in the tail
 *   num_post_pad[0]            padded row count
 *   items[max_items][4]        LoRA work items (start row, rows, adapter,
 *                              expert) in key order, each at most lbm rows;
 *                              tail filled with (0, 0, -1, -1)
 *   num_items[0]               item count */
int oracle_align(int64_t T, int64_t Kp, int64_t Ep, int64_t La, int64_t bm, int64_t lbm,
                 const int32_t *topk_ids, const int32_t *adapter_ids,
                 int32_t *sorted_ids, int64_t cap, int32_t *block_expert, int64_t max_blocks,
                 int32_t *num_post_pad, int32_t *items, int64_t max_items, int32_t *num_items)
{
    int64_t P = T * Kp;
    int64_t NK = Ep * (La + 1);
    if (bm <= 0 || lbm <= 0 || Ep <= 0 || La < 0)
        return -1;
    if (max_blocks < oracle_max_blocks(P, Ep, bm) || cap < max_blocks * bm)
        return -3;
    if (La > 0 && max_items < oracle_max_items(P, Ep, La, lbm))
        return -3;
    int64_t *cnt = (int64_t *)calloc((size_t)NK, sizeof(int64_t));
    int64_t *bin_off = (int64_t *)calloc((size_t)NK, sizeof(int64_t));
    int64_t *cursor = (int64_t *)calloc((size_t)NK, sizeof(int64_t));
    if (!cnt || !bin_off || !cursor) {
        free(cnt);
        free(bin_off);
        free(cursor);
        return -2;
    }
    for (int64_t f = 0; f < P; ++f) {
        int64_t e = topk_ids[f];
        int64_t a = (La > 0) ? adapter_ids[f / Kp] : -1;
        if (e < 0 || e >= Ep || a < -1 || a >= (La > 0 ? La : 0)) {
            free(cnt);
            free(bin_off);
            free(cursor);
            return -1;
        }
        cnt[e * (La + 1) + (a + 1)] += 1;
    }
    for (int64_t i = 0; i < cap; ++i)
        sorted_ids[i] = (int32_t)P;
    for (int64_t b = 0; b < max_blocks; ++b)
        block_expert[b] = -1;
    int64_t off = 0, nblk = 0;
    for (int64_t e = 0; e < Ep; ++e) {
        int64_t ce = 0, run = off;
        for (int64_t j = 0; j <= La; ++j) {
            bin_off[e * (La + 1) + j] = run;
            run += cnt[e * (La + 1) + j];
            ce += cnt[e * (La + 1) + j];
        }
        int64_t pad = (ce + bm - 1) / bm * bm;
        for (int64_t b = 0; b < pad / bm; ++b)
            block_expert[nblk++] = (int32_t)e;
        off += pad;
    }
    *num_post_pad = (int32_t)off;
    for (int64_t k = 0; k < NK; ++k)
        cursor[k] = bin_off[k];
    for (int64_t f = 0; f < P; ++f) {
        int64_t e = topk_ids[f];
        int64_t a = (La > 0) ? adapter_ids[f / Kp] : -1;
        int64_t k = e * (La + 1) + (a + 1);
        sorted_ids[cursor[k]++] = (int32_t)f;
    }
    int64_t ni = 0;
    if (items) {
        for (int64_t i = 0; i < max_items; ++i) {
            items[4 * i + 0] = 0;
            items[4 * i + 1] = 0;
            items[4 * i + 2] = -1;
            items[4 * i + 3] = -1;
        }
        for (int64_t e = 0; e < Ep && La > 0; ++e) {
            for (int64_t a = 0; a < La; ++a) {
                int64_t k = e * (La + 1) + (a + 1);
                for (int64_t q = 0; q < cnt[k]; q += lbm) {
                    int64_t len = cnt[k] - q < lbm ? cnt[k] - q : lbm;
                    items[4 * ni + 0] = (int32_t)(bin_off[k] + q);
                    items[4 * ni + 1] = (int32_t)len;
                    items[4 * ni + 2] = (int32_t)a;
                    items[4 * ni + 3] = (int32_t)e;
                    ++ni;
                }
            }
        }
    }
    if (num_items)
        *num_items = (int32_t)ni;
    free(cnt);
    free(bin_off);
    free(cursor);
    return 0;
}

/* -------------------------------------------------------------- forward */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One (token, slot) expert MLP with the token's adapter, in fp64.
 * g[n] = sum_h W13[e,n,h] x[h]                     n < 2I
 * u[k] = sum_h A13[a,e,k,h] x[h];  g[n] += sum_k B13[a,e,n,k] u[k]   (a >= 0)
 * hv[i] = silu(g[i]) * g[I+i]
 * y[n] = sum_i W2[e,n,i] hv[i]                     n < H
 * v[k] = sum_i A2[a,e,k,i] hv[i];  y[n] += sum_k B2[a,e,n,k] v[k]    (a >= 0) */
static void expert_mlp(int64_t H, int64_t I, int64_t Ep, int64_t r, int dtype,
                       const double *x, int64_t e, int64_t a,
                       const void *w13, const void *w2, const void *a13, const void *b13,
                       const void *a2, const void *b2, double *g, double *hv, double *uv, double *y)
{
    for (int64_t n = 0; n < 2 * I; ++n) {
        double acc = 0.0;
        int64_t base = (e * 2 * I + n) * H;
        for (int64_t h = 0; h < H; ++h)
            acc += ld(w13, base + h, dtype) * x[h];
        g[n] = acc;
    }
    if (a >= 0 && r > 0) {
        int64_t ae = a * Ep + e;
        for (int64_t k = 0; k < r; ++k) {
            double acc = 0.0;
            int64_t base = (ae * r + k) * H;
            for (int64_t h = 0; h < H; ++h)
                acc += ld(a13, base + h, dtype) * x[h];
            uv[k] = acc;
        }
        for (int64_t n = 0; n < 2 * I; ++n) {
            double acc = 0.0;
            int64_t base = (ae * 2 * I + n) * r;
            for (int64_t k = 0; k < r; ++k)
                acc += ld(b13, base + k, dtype) * uv[k];
            g[n] += acc;
        }
    }
    for (int64_t i = 0; i < I; ++i)
        hv[i] = silu(g[i]) * g[I + i];
    for (int64_t n = 0; n < H; ++n) {
        double acc = 0.0;
        int64_t base = (e * H + n) * I;
        for (int64_t i = 0; i < I; ++i)
            acc += ld(w2, base + i, dtype) * hv[i];
        y[n] = acc;
    }
    if (a >= 0 && r > 0) {
        int64_t ae = a * Ep + e;
        for (int64_t k = 0; k < r; ++k) {
            double acc = 0.0;
            int64_t base = (ae * r + k) * I;
            for (int64_t i = 0; i < I; ++i)
                acc += ld(a2, base + i, dtype) * hv[i];
            uv[k] = acc;
        }
        for (int64_t n = 0; n < H; ++n) {
            double acc = 0.0;
            int64_t base = (ae * H + n) * r;
            for (int64_t k = 0; k < r; ++k)
                acc += ld(b2, base + k, dtype) * uv[k];
            y[n] += acc;
        }
    }
}

/* Full layer output for the tokens listed in `tokens` (all T when tokens is
 * NULL), written as fp64 rows of `out` in list order.  LoRA is applied when
 * L > 0, r > 0 and adapter_ids is non-NULL; adapter -1 means no LoRA.
 * Routing is recomputed here from the logits: the plain router for
 * scoring = -1 (bias NULL), else the biased router of oracle_route_bias.
 * nthreads <= 0 uses the OpenMP default. */
int oracle_forward(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, int64_t S,
                   int64_t L, int64_t r, float rsf, int renorm, int dtype, int scoring,
                   const float *bias,
                   const void *x, const float *logits, const int32_t *adapter_ids,
                   const void *w13, const void *w2, const void *a13, const void *b13,
                   const void *a2, const void *b2,
                   const int64_t *tokens, int64_t ntok, double *out, int nthreads)
{
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || K > E || S < 0 || rsf <= 0.0f ||
        scoring < -1 || scoring > 1 || (scoring < 0 && bias != NULL))
        return -1;
    int lora = (L > 0 && r > 0 && adapter_ids != NULL && a13 && b13 && a2 && b2);
    int64_t Ep = E + S, Kp = K + S;
    if (!tokens)
        ntok = T;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *xv = (double *)malloc(sizeof(double) * (size_t)H);
        double *g = (double *)malloc(sizeof(double) * (size_t)(2 * I));
        double *hv = (double *)malloc(sizeof(double) * (size_t)I);
        double *uv = (double *)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        double *y = (double *)malloc(sizeof(double) * (size_t)H);
        double *ex = (double *)malloc(sizeof(double) * (size_t)(E > K ? E : K));
        unsigned char *taken = (unsigned char *)malloc((size_t)E);
        int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)Kp);
        float *w = (float *)malloc(sizeof(float) * (size_t)Kp);
        if (!xv || !g || !hv || !uv || !y || !ex || !taken || !ids || !w) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t q = 0; q < ntok; ++q) {
                int64_t t = tokens ? tokens[q] : q;
                double *o = out + q * H;
                if (t < 0 || t >= T) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                for (int64_t hh = 0; hh < H; ++hh) {
                    xv[hh] = ld(x, t * H + hh, dtype);
                    o[hh] = 0.0;
                }
                if (scoring < 0)
                    route_token(logits + t * E, E, K, S, rsf, renorm, ids, w, taken, ex);
                else
                    route_token_bias(logits + t * E, bias, E, K, S, rsf, renorm, scoring, ids, w, taken, ex);
                int64_t a = lora ? adapter_ids[t] : -1;
                if (a < -1 || a >= L) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                for (int64_t j = 0; j < Kp; ++j) {
                    expert_mlp(H, I, Ep, lora ? r : 0, dtype, xv, ids[j], a, w13, w2, a13, b13, a2,
                               b2, g, hv, uv, y);
                    for (int64_t hh = 0; hh < H; ++hh)
                        o[hh] += (double)w[j] * y[hh];
                }
                for (int64_t hh = 0; hh < H; ++hh)
                    o[hh] *= (double)rsf;
            }
        }
        free(xv);
        free(g);
        free(hv);
        free(uv);
        free(y);
        free(ex);
        free(taken);
        free(ids);
        free(w);
    }
    return bad ? -1 : 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One FP8 E4M3 code as a double; NaN for the two NaN codes. */
static double e4m3_value(uint8_t b)
{
    const int sign = b >> 7, ex = (b >> 3) & 15, man = b & 7;
    double v;
    if (ex == 15 && man == 7)
        return NAN;
    if (ex == 0)
        v = ldexp((double)man, -9);              /* (man / 8) * 2^(1 - 7) */
    else
        v = ldexp(8.0 + (double)man, ex - 10);   /* (1 + man / 8) * 2^(ex - 7) */
    return sign ? -v : v;
}

/* MXFP8 rows -> fp64: out[r][k] = e4m3(codes[r][k]) * 2^(scales[r][k/32] - 127).
 * K must be a multiple of 32.  Returns -1 for a NaN code or a scale byte
 * outside [1, 254] (NaN scale 255; 0 is left out as the layer's
 * precondition), else 0. */
int oracle_mxfp8_decode(int64_t rows, int64_t K, const uint8_t *codes, const uint8_t *scales, double *out)
{
    int64_t r, k;
    if (K % 32 != 0)
        return -1;
    for (r = 0; r < rows; ++r) {
        for (k = 0; k < K; ++k) {
            const uint8_t s = scales[r * (K / 32) + k / 32];
            const double v = e4m3_value(codes[r * K + k]);
            if (s == 0 || s == 255 || isnan(v))
                return -1;
            out[r * K + k] = ldexp(v, (int)s - 127);
        }
    }
    return 0;
}
