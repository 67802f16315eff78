/*
 * moe_oracle.c -- the plain CPU oracle of the quantised MoE layer.
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h): no product code links this.
 *
 * Each function writes out the definition of one step in the most direct
 * form: sequential loops, fp64 sums, no blocking or reordering.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Scalar conversions, from the IEEE 754 / OCP MX v1.0 format definitions.    */
/* ------------------------------------------------------------------------- */

float orc_bf16_to_f32(uint16_t b)
{
    /* bfloat16 is the upper half of a binary32 */
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float orc_f16_to_f32(uint16_t h)
{
    /* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits */
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return (float)(sign ? -v : v);                 /* exact in binary32 */
}

uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);    /* NaN stays NaN, made quiet */
    /* round to nearest, ties to even, on the 16 dropped bits */
    uint32_t lower = u & 0xffffu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

float orc_e2m1_value(uint8_t code)
{
    /* E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit.  Exponent field 0
     * is subnormal (0 or 0.5); otherwise (1 + m/2) * 2^(e-1). */
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    float v = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return sign ? -v : v;
}

double orc_e8m0_value(uint8_t e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* ------------------------------------------------------------------------- */
/* Activation quantisation.                                                   */
/* The integer-dot scheme of the Colibri guide (table "Points techniques      */
/* cles", integer dot-product row) multiplies int8 activations by int8 /      */
/* packed-int4 weights.  Reading: symmetric per-row scale amax/127, codes in  */
/* [-127,127], the code decided in fp32 with one rounded multiply by 127/amax */
/* and rint (ties to even).                                                   */
/* ------------------------------------------------------------------------- */

void orc_quant_row(const float *v, int K, int8_t *q, float *s)
{
    float amax = 0.0f;
    for (int i = 0; i < K; ++i) {
        float a = fabsf(v[i]);
        if (a > amax)
            amax = a;
    }
    if (amax == 0.0f) {
        for (int i = 0; i < K; ++i)
            q[i] = 0;
        *s = 0.0f;
        return;
    }
    float inv = 127.0f / amax;
    *s = amax / 127.0f;
    for (int i = 0; i < K; ++i) {
        float p = v[i] * inv;          /* one fp32 rounding */
        float r = rintf(p);            /* ties to even */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
}

/* ------------------------------------------------------------------------- */
/* Router.  DeepSeek-V3 style (Colibri guide, table "Points techniques cles", */
/* router row): sigmoid affinities, a bias that only steers selection, the    */
/* k best experts per token (kongchang article, MoE section: only the few     */
/* experts the light router picks run), weights normalised over the selected */
/* experts and multiplied by the routed scale.                                */
/* ------------------------------------------------------------------------- */

static double sigmoid64(double l)
{
    return 1.0 / (1.0 + exp(-l));
}

/* the value a biased score is ranked by: itself, or -inf for NaN */
static double rank_key(double c)
{
    return isnan(c) ? -INFINITY : c;
}

void orc_router(int T, int H, int E, int k, float r,
                const uint16_t *x, const float *Wr, const float *b,
                int32_t *idx, float *w,
                double *logits, double *scores, double *choice)
{
    double *l = (double *)malloc(sizeof(double) * (size_t)E);
    double *s = (double *)malloc(sizeof(double) * (size_t)E);
    double *c = (double *)malloc(sizeof(double) * (size_t)E);
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const uint16_t *xt = x + (size_t)t * H;
        for (int e = 0; e < E; ++e) {
            const float *we = Wr + (size_t)e * H;
            double acc = 0.0;
            for (int j = 0; j < H; ++j)
                acc += (double)orc_bf16_to_f32(xt[j]) * (double)we[j];
            l[e] = acc;
            s[e] = sigmoid64(acc);
            c[e] = s[e] + (double)b[e];
            taken[e] = 0;
            if (logits) logits[(size_t)t * E + e] = l[e];
            if (scores) scores[(size_t)t * E + e] = s[e];
            if (choice) choice[(size_t)t * E + e] = c[e];
        }
        /* k rounds of "largest c among the experts not yet taken"; scanning
         * e upwards with a strict > keeps the lowest index on ties.  A NaN c
         * ranks as -inf (reading: an undefined score never wins a place over
         * a defined one). */
        for (int i = 0; i < k; ++i) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || rank_key(c[e]) > rank_key(c[best]))
                    best = e;
            }
            taken[best] = 1;
            idx[(size_t)t * k + i] = best;
        }
        double den = 0.0;
        for (int i = 0; i < k; ++i)
            den += s[idx[(size_t)t * k + i]];
        for (int i = 0; i < k; ++i) {
            double wi = (den > 0.0) ? (s[idx[(size_t)t * k + i]] / den) * (double)r : 0.0;
            w[(size_t)t * k + i] = (float)wi;
        }
    }
    free(l); free(s); free(c); free(taken);
}

/* ------------------------------------------------------------------------- */
/* Router lookahead (Colibri guide, section "Router-Lookahead prefetch"): the  */
/* next layer's router applied to the current layer's input.  The weights are */
/* not needed for a prediction, only the selection.                           */
/* ------------------------------------------------------------------------- */

void orc_lookahead(int T, int H, int E, int k, const uint16_t *x_l, const float *Wr_next,
                   const float *b_next, int32_t *idx_pred)
{
    float *w = (float *)malloc(sizeof(float) * (size_t)T * (size_t)k);
    orc_router(T, H, E, k, 1.0f, x_l, Wr_next, b_next, idx_pred, w, NULL, NULL, NULL);
    free(w);
}

void orc_residual_bf16(int n, const uint16_t *x, const float *y, float gamma, uint16_t *x_next)
{
    for (int i = 0; i < n; ++i) {
        float t = gamma * y[i];                     /* rounded to fp32 */
        float r = orc_bf16_to_f32(x[i]) + t;        /* rounded to fp32 */
        x_next[i] = orc_f32_to_bf16(r);
    }
}

/* ------------------------------------------------------------------------- */
/* int4 x int8 projection (the integer dot-product kernel of the Colibri      */
/* guide, table "Points techniques cles"; group-scaled int4 of the            */
/* aifrontierpost tutorial, "Step 3").  Inside a group the dot product is an  */
/* exact integer; the groups are then combined with their fp16 scales.        */
/* Every product acc*S is exact in fp64 and so is their sum as long as the    */
/* scale exponents of a row span at most 19 binades (orc_rows_exact_fp64), so */
/* the fp64 sum below is the exact real number, whatever the order.           */
/* ------------------------------------------------------------------------- */

void orc_group_dots(const int8_t *q_in, const int8_t *qw, int N, int K, int g,
                    int32_t *acc)
{
    int G = K / g;
    for (int n = 0; n < N; ++n)
        for (int j = 0; j < G; ++j) {
            int32_t a = 0;
            for (int i = 0; i < g; ++i)
                a += (int32_t)qw[(size_t)n * K + (size_t)j * g + i] * (int32_t)q_in[j * g + i];
            acc[(size_t)n * G + j] = a;
        }
}

static double row_dot_exact(const int8_t *q_in, const int8_t *qw_row,
                            const uint16_t *S_row, int K, int g)
{
    int G = K / g;
    double sum = 0.0;
    for (int j = 0; j < G; ++j) {
        int32_t a = 0;
        for (int i = 0; i < g; ++i)
            a += (int32_t)qw_row[j * g + i] * (int32_t)q_in[j * g + i];
        sum += (double)a * (double)orc_f16_to_f32(S_row[j]);
    }
    return sum;
}

void orc_proj_i4i8(const int8_t *q_in, float s_in, const int8_t *qw,
                   const uint16_t *S, int N, int K, int g,
                   const int32_t *rows, int n_rows, float *y)
{
    int G = K / g;
    int cnt = rows ? n_rows : N;
    for (int i = 0; i < cnt; ++i) {
        int n = rows ? rows[i] : i;
        double p = row_dot_exact(q_in, qw + (size_t)n * K, S + (size_t)n * G, K, g);
        y[i] = (float)(p * (double)s_in);
    }
}

int orc_rows_exact_fp64(const uint16_t *S, int N, int K, int g)
{
    /* A term acc*S is an integer of at most 15 + 11 bits times 2^(E-25)
     * (E = biased fp16 exponent, 1 for subnormals); G terms add log2(G) bits.
     * The sum is exact in fp64 when 26 + ceil(log2 G) + (Emax - Emin) <= 53. */
    int G = K / g;
    int lg = 0;
    while ((1 << lg) < G)
        ++lg;
    for (int n = 0; n < N; ++n) {
        int emin = 99, emax = -99;
        for (int j = 0; j < G; ++j) {
            uint16_t h = S[(size_t)n * G + j];
            int e = (h >> 10) & 31;
            if ((h & 0x7fff) == 0)
                continue;                   /* zero scale: term is 0 */
            if (e == 31)
                return 0;
            if (e == 0)
                e = 1;
            if (e < emin) emin = e;
            if (e > emax) emax = e;
        }
        if (emax >= emin && 26 + lg + (emax - emin) > 53)
            return 0;
    }
    return 1;
}

/* ------------------------------------------------------------------------- */
/* One SwiGLU expert.  The activation function is not on the pages; SwiGLU is */
/* the plainest reading for DeepSeek-V3-family experts: h = silu(G) * U,      */
/* silu(v) = v / (1 + exp(-v)).  h is requantised per (token, expert) row.    */
/* ------------------------------------------------------------------------- */

static double proj_fp64(const int8_t *q_in, float s_in, const int8_t *qw_row,
                        const uint16_t *S_row, int K, int g)
{
    return row_dot_exact(q_in, qw_row, S_row, K, g) * (double)s_in;
}

void orc_expert(int H, int F, int g, const int8_t *qa, float sa,
                const orc_expert_w *w, const int32_t *down_rows, int n_down,
                float *y, float *h, int8_t *qh, float *sh)
{
    int GH = H / g;
    float *hv = (float *)malloc(sizeof(float) * (size_t)F);
    int8_t *qv = (int8_t *)malloc((size_t)F);
    float s_h;
    for (int n = 0; n < F; ++n) {
        double G = proj_fp64(qa, sa, w->q_gate + (size_t)n * H, w->s_gate + (size_t)n * GH, H, g);
        double U = proj_fp64(qa, sa, w->q_up + (size_t)n * H, w->s_up + (size_t)n * GH, H, g);
        double silu = G / (1.0 + exp(-G));
        hv[n] = (float)(silu * U);
    }
    orc_quant_row(hv, F, qv, &s_h);
    orc_proj_i4i8(qv, s_h, w->q_down, w->s_down, H, F, g, down_rows, n_down, y);
    if (h) memcpy(h, hv, sizeof(float) * (size_t)F);
    if (qh) memcpy(qh, qv, (size_t)F);
    if (sh) *sh = s_h;
    free(hv);
    free(qv);
}

/* ------------------------------------------------------------------------- */
/* Whole layer: quantise each token, route, run the shared expert and the k   */
/* routed experts, combine.  Reading: the shared expert enters with weight 1  */
/* (DeepSeek-V3 convention; the Colibri guide only says shared experts are    */
/* supported), the routed experts with their gate weights, summed in fp64 in  */
/* the order shared, rank 0 .. k-1 and rounded once to fp32.                  */
/* ------------------------------------------------------------------------- */

void orc_layer(int T, int H, int F, int E, int k, int g, float r,
               const uint16_t *x, const float *Wr, const float *b,
               const orc_expert_w *experts, const orc_expert_w *shared,
               const int32_t *out_rows, int n_out,
               int32_t *idx, float *w, float *out)
{
    int cnt = out_rows ? n_out : H;
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    int8_t *qa = (int8_t *)malloc((size_t)H);
    float *ysh = (float *)malloc(sizeof(float) * (size_t)cnt);
    float *ye = (float *)malloc(sizeof(float) * (size_t)cnt * (size_t)k);
    float sa;
    orc_router(T, H, E, k, r, x, Wr, b, idx, w, NULL, NULL, NULL);
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < H; ++j)
            xf[j] = orc_bf16_to_f32(x[(size_t)t * H + j]);
        orc_quant_row(xf, H, qa, &sa);
        if (shared)
            orc_expert(H, F, g, qa, sa, shared, out_rows, n_out, ysh, NULL, NULL, NULL);
        for (int i = 0; i < k; ++i) {
            int e = idx[(size_t)t * k + i];
            orc_expert(H, F, g, qa, sa, &experts[e], out_rows, n_out,
                       ye + (size_t)i * cnt, NULL, NULL, NULL);
        }
        for (int n = 0; n < cnt; ++n) {
            double o = shared ? (double)ysh[n] : 0.0;
            for (int i = 0; i < k; ++i)
                o += (double)w[(size_t)t * k + i] * (double)ye[(size_t)i * cnt + n];
            out[(size_t)t * cnt + n] = (float)o;
        }
    }
    free(xf); free(qa); free(ysh); free(ye);
}

/* ------------------------------------------------------------------------- */
/* MXFP4 variant (kongchang article, model-family list: Kimi K3 streams its   */
/* native MXFP4 experts; aifrontierpost tutorial, "Step 3").  Weights are     */
/* E2M1 codes with one E8M0 power-of-two scale per 32 inputs (OCP MX v1.0);   */
/* activations stay bf16; sums of exact products in fp64, rounded to fp32.    */
/* Reading: h is rounded to bf16 before the down projection.                  */
/* ------------------------------------------------------------------------- */

void orc_proj_mx(const float *a, const uint8_t *codes, const uint8_t *e8m0,
                 int N, int K, const int32_t *rows, int n_rows, float *y)
{
    int G = K / 32;
    int cnt = rows ? n_rows : N;
    for (int i = 0; i < cnt; ++i) {
        int n = rows ? rows[i] : i;
        double sum = 0.0;
        for (int j = 0; j < K; ++j) {
            double wv = (double)orc_e2m1_value(codes[(size_t)n * K + j] & 15)
                      * orc_e8m0_value(e8m0[(size_t)n * G + j / 32]);
            sum += (double)a[j] * wv;
        }
        y[i] = (float)sum;
    }
}

void orc_mx_expert(int H, int F, const float *a, const orc_mx_expert_w *w,
                   const int32_t *down_rows, int n_down, float *y,
                   uint16_t *h_bf16)
{
    float *G = (float *)malloc(sizeof(float) * (size_t)F);
    float *U = (float *)malloc(sizeof(float) * (size_t)F);
    float *hv = (float *)malloc(sizeof(float) * (size_t)F);
    orc_proj_mx(a, w->c_gate, w->e_gate, F, H, NULL, 0, G);
    orc_proj_mx(a, w->c_up, w->e_up, F, H, NULL, 0, U);
    for (int n = 0; n < F; ++n) {
        double gv = (double)G[n];
        double hn = gv / (1.0 + exp(-gv)) * (double)U[n];
        uint16_t hb = orc_f32_to_bf16((float)hn);
        if (h_bf16) h_bf16[n] = hb;
        hv[n] = orc_bf16_to_f32(hb);
    }
    orc_proj_mx(hv, w->c_down, w->e_down, H, F, down_rows, n_down, y);
    free(G); free(U); free(hv);
}

void orc_mx_layer(int T, int H, int F, int E, int k, float r,
                  const uint16_t *x, const float *Wr, const float *b,
                  const orc_mx_expert_w *experts, const orc_mx_expert_w *shared,
                  const int32_t *out_rows, int n_out,
                  int32_t *idx, float *w, float *out)
{
    int cnt = out_rows ? n_out : H;
    float *xf = (float *)malloc(sizeof(float) * (size_t)H);
    float *ysh = (float *)malloc(sizeof(float) * (size_t)cnt);
    float *ye = (float *)malloc(sizeof(float) * (size_t)cnt * (size_t)k);
    orc_router(T, H, E, k, r, x, Wr, b, idx, w, NULL, NULL, NULL);
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < H; ++j)
            xf[j] = orc_bf16_to_f32(x[(size_t)t * H + j]);
        if (shared)
            orc_mx_expert(H, F, xf, shared, out_rows, n_out, ysh, NULL);
        for (int i = 0; i < k; ++i) {
            int e = idx[(size_t)t * k + i];
            orc_mx_expert(H, F, xf, &experts[e], out_rows, n_out, ye + (size_t)i * cnt, NULL);
        }
        for (int n = 0; n < cnt; ++n) {
            double o = shared ? (double)ysh[n] : 0.0;
            for (int i = 0; i < k; ++i)
                o += (double)w[(size_t)t * k + i] * (double)ye[(size_t)i * cnt + n];
            out[(size_t)t * cnt + n] = (float)o;
        }
    }
    free(xf); free(ysh); free(ye);
}
