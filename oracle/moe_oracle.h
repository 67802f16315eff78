/*
 * moe_oracle.h -- plain, slow, single-threaded CPU oracle for one quantised
 * Mixture-of-Experts layer forward (router + top-k + int4 x int8 SwiGLU
 * expert FFNs + combine), its MXFP4 variant, and the expert-cache state
 * machine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link or call this code; only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no code, header, table or
 * constant with the HIP path.
 *
 * Sources (the method as described on the Colibri pages):
 *  - "Guide Complet de Colibri" (dashen-tech.com), table "Points techniques
 *    cles": the router is the DeepSeek-V3 sigmoid router with shared experts;
 *    matrix products run as integer dot products of int8 / packed int4 values.
 *  - same page, "Analyse approfondie": decode and prefill use the integer kernel.
 *  - "Colibri纯C引擎爆火" (kongchang.com), section on MoE: a light router picks
 *    a few experts per token and only those compute.
 *  - "Run a 744B-parameter model on your own machine" (aifrontierpost.com),
 *    "Step 3": group-scaled int4 expert weights; MXFP4 experts for Kimi K3.
 * Where the pages leave a step open the plainest reading is taken; every such
 * reading is listed in the design notes of the repository.
 *
 * Floating point: fp64 wherever the pages fix no precision.  Where floating
 * point decides an integer (an int8 code), the decision is taken in fp32 -- the
 * precision of the GPU kernels -- with the same IEEE operations.
 * Build: gcc -O2 -ffp-contract=off, no fast-math, no intrinsics, no threads.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- scalar conversions (IEEE 754 definitions) ---------------------------- */
float orc_bf16_to_f32(uint16_t b);
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);          /* round to nearest even, NaN kept quiet */
float orc_e2m1_value(uint8_t code);         /* OCP MX v1.0 FP4 E2M1, code in low nibble */
double orc_e8m0_value(uint8_t e);           /* 2^(e-127); e == 255 is NaN */

/* ---- activation quantisation ---------------------------------------------- */
/* Symmetric per-row int8: amax = max|v|; amax == 0 -> q = 0, s = 0;
 * else inv = 127/amax, s = amax/127 (fp32, correctly rounded) and
 * q = clamp(rint(v * inv), -127, 127) with the product rounded to fp32. */
void orc_quant_row(const float *v, int K, int8_t *q, float *s);

/* ---- router ----------------------------------------------------------------- */
/* For T tokens x[T,H] (bf16 bits), router weights Wr[E,H] (fp32) and selection
 * bias b[E] (fp32):  l = x . Wr_e (fp64), s = 1/(1+exp(-l)), c = s + b.
 * idx[T,k] = the k experts with the largest c, ties to the lower index, in rank
 * order (a NaN c ranks as -inf); w[T,k] = s_idx / sum(s_idx) * r.  logits/scores/choice may be NULL
 * ([T,E] fp64 each). */
void orc_router(int T, int H, int E, int k, float r,
                const uint16_t *x, const float *Wr, const float *b,
                int32_t *idx, float *w,
                double *logits, double *scores, double *choice);

/* ---- router lookahead ------------------------------------------------------- */
/* Source: "Guide Complet de Colibri", section "Router-Lookahead prefetch"
 * (the next layer's routing is largely predictable from the current state, and
 * a worker prefetches the predicted experts); kongchang article, storage-tier
 * section (one-layer-ahead prefetch).  Reading: the prediction for layer l+1
 * is layer l+1's own router applied to layer l's input x_l, before layer l's
 * output is known: idx_pred [T,k] = the k experts with the largest
 * sigmoid(x_l . Wr_next) + b_next, ties to the lower index, in rank order. */
void orc_lookahead(int T, int H, int E, int k, const uint16_t *x_l, const float *Wr_next,
                   const float *b_next, int32_t *idx_pred);
/* The residual composition of a stack of MoE layers (reading: no norm):
 * x_next = bf16(fp32(x) + fp32(gamma * y)) with both fp32 operations rounded
 * to nearest and the bf16 rounding to nearest even; n elements. */
void orc_residual_bf16(int n, const uint16_t *x, const float *y, float gamma, uint16_t *x_next);

/* ---- int4 x int8 projection ---------------------------------------------------- */
/* y[n] = fp32( fp64(sum_g acc[n,g] * S[n,g]) * s_in ),
 * acc[n,g] = sum_{k in group g} qw[n,k] * q_in[k]  (exact int32),
 * qw[N,K] int8 in [-8,7], S[N,K/g] fp16 bits.  rows (may be NULL = all rows
 * 0..N-1) selects which n to compute; y has n_rows entries. */
void orc_proj_i4i8(const int8_t *q_in, float s_in, const int8_t *qw,
                   const uint16_t *S, int N, int K, int g,
                   const int32_t *rows, int n_rows, float *y);
/* The raw int32 group sums acc[n,g] for all n, g (N x K/g). */
void orc_group_dots(const int8_t *q_in, const int8_t *qw, int N, int K, int g,
                    int32_t *acc);
/* 1 if sum_g acc*S of every row is exactly representable in fp64 for every
 * possible int8 input (a bound on the spread of the row's scale exponents). */
int orc_rows_exact_fp64(const uint16_t *S, int N, int K, int g);

/* ---- one expert ------------------------------------------------------------------ */
typedef struct orc_expert_w {
    const int8_t *q_gate;   const uint16_t *s_gate;   /* [F,H], [F,H/g] */
    const int8_t *q_up;     const uint16_t *s_up;     /* [F,H], [F,H/g] */
    const int8_t *q_down;   const uint16_t *s_down;   /* [H,F], [H,F/g] */
} orc_expert_w;

/* SwiGLU expert on one quantised token row (qa[H], sa):
 *   G, U = proj(gate), proj(up) kept in fp64 (exact sum times sa),
 *   h = fp32( G/(1+exp(-G)) * U ),  (q_h, s_h) = quant_row(h),
 *   y = proj(down) on (q_h, s_h).
 * down_rows (NULL = all H rows) / n_down select output rows of y.
 * h, qh, sh may be NULL. */
void orc_expert(int H, int F, int g, const int8_t *qa, float sa,
                const orc_expert_w *w, const int32_t *down_rows, int n_down,
                float *y, float *h, int8_t *qh, float *sh);

/* ---- whole layer ------------------------------------------------------------------ */
/* out[T, n_out] fp32 = Y_shared + sum_i w_i * Y_{idx_i}, summed in fp64 in that
 * order (shared first, then rank order) and rounded once to fp32.
 * experts[E]: weights of each routed expert (entries never selected may be
 * zeroed); shared may be NULL.  out_rows (NULL = all H) selects output columns.
 * idx/w receive the routing ([T,k]). */
void orc_layer(int T, int H, int F, int E, int k, int g, float r,
               const uint16_t *x, const float *Wr, const float *b,
               const orc_expert_w *experts, const orc_expert_w *shared,
               const int32_t *out_rows, int n_out,
               int32_t *idx, float *w, float *out);

/* ---- MXFP4 variant ------------------------------------------------------------------ */
/* y[n] = fp32( sum_k a[k] * E2M1(codes[n,k]) * 2^(e8m0[n,k/32]-127) ) with the
 * sum of exact products taken in fp64.  codes: one code per byte, low nibble. */
void orc_proj_mx(const float *a, const uint8_t *codes, const uint8_t *e8m0,
                 int N, int K, const int32_t *rows, int n_rows, float *y);

typedef struct orc_mx_expert_w {
    const uint8_t *c_gate; const uint8_t *e_gate;   /* [F,H], [F,H/32] */
    const uint8_t *c_up;   const uint8_t *e_up;
    const uint8_t *c_down; const uint8_t *e_down;   /* [H,F], [H,F/32] */
} orc_mx_expert_w;

/* MXFP4 expert on bf16 activations: G,U fp32 as above; h = fp32(silu(G)*U)
 * rounded to bf16; y = proj_mx(down) on h.  h_bf16 may be NULL. */
void orc_mx_expert(int H, int F, const float *a, const orc_mx_expert_w *w,
                   const int32_t *down_rows, int n_down, float *y,
                   uint16_t *h_bf16);

void orc_mx_layer(int T, int H, int F, int E, int k, float r,
                  const uint16_t *x, const float *Wr, const float *b,
                  const orc_mx_expert_w *experts, const orc_mx_expert_w *shared,
                  const int32_t *out_rows, int n_out,
                  int32_t *idx, float *w, float *out);

/* ---- expert cache state machine ------------------------------------------------------ */
enum { ORC_EV_HIT = 0, ORC_EV_MISS = 1, ORC_EV_PF_ISSUE = 2, ORC_EV_PF_HIT = 3,
       ORC_EV_PF_SKIP = 4, ORC_EV_EVICT = 5, ORC_EV_PIN_FILL = 6, ORC_EV_PIN_KEEP = 7 };

typedef struct orc_cache_event {
    int32_t kind, layer, expert, slot;
} orc_cache_event;

typedef struct orc_cache_stats {
    int64_t demand_hits, demand_misses;
    int64_t prefetch_issued, prefetch_used, prefetch_wasted, prefetch_skipped;
    int64_t prefetch_resident;
    int64_t evictions;
    int64_t pinned, pin_fills;
} orc_cache_stats;

/* Replays a trace through the LRU slot pool.  For step s and layer l the
 * demanded experts are demand[(s*L + l)*k + i] (k distinct ids, rank order);
 * when predict != NULL, after the demand of layer l the predicted set
 * predict[(s*L + l)*k + i] for layer l+1 (or layer 0 of step s+1 when
 * l == L-1 and wrap != 0) is prefetched.  Slots used by a layer are locked
 * until that layer is released, which happens right after its prefetch.
 * per_layer != 0 partitions the pool: layer l owns slots
 * [l*cap/L, (l+1)*cap/L).  Events go to ev (capacity ev_cap); returns the
 * number of events written, or -1 if ev_cap is too small / capacity < k. */
int64_t orc_cache_sim(int L, int E, int k, int n_slots, int n_steps,
                      const int32_t *demand, const int32_t *predict, int wrap,
                      int per_layer, orc_cache_event *ev, int64_t ev_cap,
                      orc_cache_stats *st);

/* The same replay with the learned pinned hot-store: usage counts start from
 * usage_init [L*E] (NULL: zeros) and count every DEMAND access; before step t
 * with pin_before[t] >= 0 (pin_before may be NULL), PIN(pin_before[t]) unpins
 * every slot and pins the hottest keys (count descending, key ascending, at
 * most partition size - k per partition; missing keys are filled).  Pinned
 * slots are never victims.  usage_out [L*E] (may be NULL) receives the final
 * counts.  Events ORC_EV_PIN_FILL / ORC_EV_PIN_KEEP record a pinned key that
 * was copied in / already resident. */
int64_t orc_cache_sim_hot(int L, int E, int k, int n_slots, int n_steps,
                          const int32_t *demand, const int32_t *predict, int wrap,
                          int per_layer, const int64_t *usage_init,
                          const int32_t *pin_before, orc_cache_event *ev, int64_t ev_cap,
                          orc_cache_stats *st, int64_t *usage_out);

#ifdef __cplusplus
}
#endif
#endif
