/*
 * moe.h -- C ABI of the MI355X (gfx950) quantised Mixture-of-Experts layer.
 *
 * One MoE layer forward as the Colibri pages describe it: a DeepSeek-V3-style
 * sigmoid router with a selection bias and top-k, routed and shared SwiGLU
 * expert FFNs over packed-int4 weights with int8 activations and exact int32
 * group sums, an MXFP4 variant, and an HBM expert cache filled from pinned host
 * memory.  Every step runs in hand-written HIP kernels for gfx950.
 *
 * Conventions
 *  - Row-major arrays.  Pointers are DEVICE pointers unless the name ends in
 *    _host.  The caller owns every array it passes; the library owns the
 *    workspace inside a moe_ctx and the slot pool inside a moe_cache.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Hot
 *    calls only enqueue work; they allocate nothing and do not synchronise the
 *    host, except moe_layer_forward with a cache (documented there).
 *  - Every call validates its arguments before enqueuing anything and returns
 *    a status; nothing aborts or throws across the ABI.  moe_last_error()
 *    gives the message of the last non-OK status of the calling thread.
 *  - Outputs are bitwise identical for identical inputs and the same kernel
 *    path, whatever the grid, the cache state or the stream timing (every sum
 *    has a fixed order).  Across the int4 paths (one-token, GEMV, MFMA) the
 *    expert projections and the combine give the same bits too (their sums
 *    are exact); the router's fp64 logits are summed in an order of each
 *    router kernel, so two paths may differ in the logits' last bits and,
 *    where two biased scores lie that close, in the routing.  The two MXFP4
 *    kernels differ in their sums (moe_ctx_set_path).
 *  - A moe_ctx is used by one host thread at a time.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK             0
#define MOE_E_INVAL        1   /* bad argument; nothing was enqueued */
#define MOE_E_UNSUPPORTED  2   /* shape/format/device this library does not run */
#define MOE_E_NOMEM        3   /* device or pinned allocation failed */
#define MOE_E_HIP          4   /* a HIP runtime call failed */
#define MOE_E_CAPACITY     5   /* cache has fewer free slots than the request */

#define MOE_WFMT_INT4   0      /* group-scaled int4, fp16 scales */
#define MOE_WFMT_MXFP4  1      /* E2M1 + E8M0 per 32 (OCP MX v1.0) */

#define MOE_DT_F32   0
#define MOE_DT_BF16  1

#define MOE_PATH_AUTO  0       /* GEMV kernels for few tokens, MFMA otherwise */
#define MOE_PATH_GEMV  1
#define MOE_PATH_MFMA  2
#define MOE_PATH_MX_BF16 3     /* MXFP4 layers: weights widened to exact bf16 on the bf16 MFMA
                                  instead of the MX MFMA (exact products, plain fp32 sums) */

/* Shape and numerics of one MoE layer.
 *  hidden H, ffn F: multiples of 256.  n_experts E in [1, 1024].
 *  top_k k in [1, min(E, 32)].  n_shared in {0, 1}.
 *  group: 32 or 64 for INT4 (inputs per fp16 scale), 32 for MXFP4.
 *  routed_scale r: multiplies the normalised routed gate weights.
 *  out_dtype: MOE_DT_F32 or MOE_DT_BF16 (round to nearest even of the fp32). */
typedef struct moe_layer_desc {
    int32_t hidden;
    int32_t ffn;
    int32_t n_experts;
    int32_t top_k;
    int32_t n_shared;
    int32_t group;
    float   routed_scale;
    int32_t wfmt;
    int32_t out_dtype;
} moe_layer_desc;

/* Weights of one layer (all device memory, caller-owned):
 *  router_w [E,H] fp32, router_bias [E] fp32,
 *  expert_ptrs: device array [E] of device blob pointers (moe_blob_bytes()
 *  bytes each, 256-byte aligned); entries of experts that are never selected
 *  may be NULL; ignored by moe_layer_forward when a cache supplies them.
 *  shared: device blob of the shared expert, or NULL when n_shared == 0. */
typedef struct moe_layer_weights {
    const float *router_w;
    const float *router_bias;
    const void *const *expert_ptrs;
    const void *shared;
} moe_layer_weights;

typedef struct moe_ctx moe_ctx;
typedef struct moe_cache moe_cache;

/* ---- context ----------------------------------------------------------------
 * Validates desc, checks that `device` is a gfx950 GPU, and allocates all
 * workspace for up to max_tokens tokens per call (activation codes, router
 * logits, routing lists, SwiGLU outputs, per-expert outputs).  Hot calls never
 * allocate.  Errors: E_INVAL (desc), E_UNSUPPORTED (device), E_NOMEM, E_HIP. */
moe_status moe_ctx_create(int32_t device, const moe_layer_desc *desc,
                          int32_t max_tokens, moe_ctx **out);
void moe_ctx_destroy(moe_ctx *ctx);
/* Kernel path for the expert FFNs (MOE_PATH_*).  For int4 layers results do
 * not depend on it (every path gives the same bits).  MXFP4 layers run on the
 * gfx950 MX MFMA by default (activations split into two E4M3 parts; its
 * internal sums measured to ~3e-4 of the largest output on the test layers)
 * or, with MOE_PATH_MX_BF16, on the bf16 MFMA with exact bf16 weights (~1e-7);
 * both within the 2e-3 output bar. */
moe_status moe_ctx_set_path(moe_ctx *ctx, int32_t path);

/* ---- weight packing (host only, no GPU needed) -----------------------------
 * Source: "Run a 744B-parameter model on your own machine" (aifrontierpost),
 * "Step 3": experts are stored as group-scaled int4; Kimi K3's experts as
 * native MXFP4.  The blob is this library's own in-memory format.
 *
 * moe_blob_bytes: size of one expert blob for desc (0 if desc is invalid).
 *
 * moe_pack_expert_int4: q_gate, q_up [F,H] and q_down [H,F] are int8 codes in
 * [-8,7]; s_gate, s_up [F,H/group] and s_down [H,F/group] are fp16 scale bits
 * (finite).  Writes the blob to blob_host (caller-owned, moe_blob_bytes()
 * bytes); copy it to device or pinned memory afterwards.  Errors: E_INVAL on a
 * code outside [-8,7], a non-finite scale, or a row whose nonzero scales span
 * more than 19 binades (the layer's exact group sums need that bound).
 *
 * moe_pack_expert_mxfp4: c_* are E2M1 codes (one per byte, low nibble) with the
 * same shapes, e_* the E8M0 bytes per 32 inputs.  E_INVAL on E8M0 0xFF (NaN). */
size_t moe_blob_bytes(const moe_layer_desc *desc);
moe_status moe_pack_expert_int4(const moe_layer_desc *desc,
                                const int8_t *q_gate, const uint16_t *s_gate,
                                const int8_t *q_up, const uint16_t *s_up,
                                const int8_t *q_down, const uint16_t *s_down,
                                void *blob_host);
moe_status moe_pack_expert_mxfp4(const moe_layer_desc *desc,
                                 const uint8_t *c_gate, const uint8_t *e_gate,
                                 const uint8_t *c_up, const uint8_t *e_up,
                                 const uint8_t *c_down, const uint8_t *e_down,
                                 void *blob_host);

/* ---- router -------------------------------------------------------------------
 * Source: "Guide Complet de Colibri" (dashen-tech), table "Points techniques
 * cles", router row: the DeepSeek-V3 sigmoid router with shared experts;
 * "Colibri纯C引擎爆火" (kongchang), MoE section: a light router picks a few
 * experts per token.
 * For x [T,H] bf16: logit l[t,e] = x[t].Wr[e] (fp64), score s = sigmoid(l),
 * choice c = s + bias[e] (the bias only steers selection).  idx [T,k] int32 =
 * the k experts with the largest c, ties to the lower index, in rank order;
 * gate_w [T,k] fp32 = s[idx]/sum(s[idx]) * routed_scale.
 * T in [0, max_tokens] (T == 0 does nothing).  Asynchronous on `stream`.
 * Errors: E_INVAL (NULL pointer, T out of range), E_HIP (launch failed). */
moe_status moe_router_topk(moe_ctx *ctx, const void *x, int32_t T,
                           const moe_layer_weights *w, int32_t *idx,
                           float *gate_w, void *stream);

/* ---- expert FFNs ----------------------------------------------------------------
 * Source: "Guide Complet de Colibri", table "Points techniques cles", integer
 * dot-product row (int8 and packed int4 matmul as exact integer dot products)
 * and section "Analyse approfondie" (step 3: loaded experts go to that
 * kernel); kongchang article, MoE section (only the selected experts compute).
 * For each token: int8 quantisation (per token, scale amax/127), the shared
 * expert and the k routed experts idx[t,:] as SwiGLU FFNs
 *   G,U = exact int4 x int8 group sums scaled by the fp16 group scales and the
 *         token scale (fp64), h = fp32(silu(G)*U), h requantised to int8 per
 *         (token, expert), Y = down projection (fp32),
 * then out[t] = Y_shared + sum_i gate_w[t,i] * Y_idx[t,i] (fp64, in that
 * order, rounded once).  idx/gate_w may come from moe_router_topk or from the
 * caller (indices must be distinct per token and < E).  out [T,H] fp32 or
 * bf16 (desc.out_dtype).  Every referenced expert pointer must be resident.
 * Asynchronous.  Errors: E_INVAL, E_HIP. */
moe_status moe_expert_ffn(moe_ctx *ctx, const void *x, int32_t T,
                          const moe_layer_weights *w, const int32_t *idx,
                          const float *gate_w, void *out, void *stream);

/* ---- whole layer ------------------------------------------------------------------
 * moe_router_topk then moe_expert_ffn.  idx_out/gate_w_out may be NULL (the
 * context's own buffers are used).  With cache == NULL: fully asynchronous.
 * With a cache: routed experts come from the cache's slots for `layer`; the
 * call synchronises the host on the router result (T*k ids), stages misses on
 * the cache's copy stream (moe_cache_stage, DEMAND), makes `stream` wait for
 * them and enqueues the FFNs.  The slots stay locked: the caller may then
 * prefetch the next layer (moe_cache_stage, PREFETCH) and must call
 * moe_cache_release(cache, layer, stream).  Errors with a cache: E_INVAL
 * (layer out of range, a cache of another shape or backend, T*k above the
 * cache's id buffer) before anything is enqueued; E_CAPACITY when the call's
 * distinct experts need more slots than the layer's partition can give: the
 * router has then run (idx_out, gate_w_out written), the cache is unchanged
 * and no slot is locked, so the call can be split into fewer tokens.  Source for the
 * staging: "Guide Complet de Colibri", section "Qu'est-ce que Colibri ?"
 * (experts loaded on demand behind an LRU cache); aifrontierpost tutorial,
 * "Honest limitations" (placement decides speed only: results are identical
 * with or without the cache). */
moe_status moe_layer_forward(moe_ctx *ctx, const void *x, int32_t T,
                             const moe_layer_weights *w, moe_cache *cache,
                             int32_t layer, int32_t *idx_out, float *gate_w_out,
                             void *out, void *stream);

/* ---- whole layer without allocation ------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, hosts that forbid hipMalloc.
 * moe_layer_forward_noalloc computes exactly what moe_layer_forward computes
 * with cache == NULL and the automatic kernel path (same kernels, same bits),
 * but takes no context: desc is passed per call, and the workspace is one
 * static device array of MOE_NOALLOC_SCRATCH_BYTES per GPU, which the library
 * holds on each GPU it runs on until the process ends.  It runs on the
 * current device.  It calls no hipMalloc/hipFree and allocates no host
 * memory; its first call on a device looks up that GPU's copy of the array.
 * x, w, idx_out (may be NULL), gate_w_out (may be NULL) and out are as for
 * moe_layer_forward.  Errors: E_INVAL (bad desc or arguments, or a call whose
 * workspace for T tokens at this shape exceeds the array -- e.g. more than
 * ~40 tokens of a hidden 6144, top-8 + shared layer -- nothing is enqueued
 * then), E_UNSUPPORTED (not a gfx950 device), E_HIP.
 * Every call on one GPU shares that GPU's array and leaves its contents for
 * the next: calls that overlap in time on one GPU (different streams without
 * ordering, or several host threads) race and give wrong results; order them
 * on one stream or synchronise them.  The call's first kernel clears the
 * array's counters. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
moe_status moe_layer_forward_noalloc(const moe_layer_desc *desc, const void *x, int32_t T,
                                     const moe_layer_weights *w, int32_t *idx_out,
                                     float *gate_w_out, void *out, void *stream);

/* ---- expert cache ---------------------------------------------------------------
 * Source: "Guide Complet de Colibri", sections "Qu'est-ce que Colibri ?" (LRU
 * expert cache, experts loaded on demand) and "Router-Lookahead prefetch" (the
 * next layer's experts are predictable and prefetched by a dedicated I/O
 * worker while the current layer computes); kongchang article, storage-tier
 * section (one-layer-ahead prefetch hides the load latency).
 * Keys are (layer, expert).  The pool has capacity_bytes / blob_bytes slots of
 * device memory.  host_blobs [n_layers*n_experts] are caller-owned pinned
 * host blobs (moe_host_alloc_pinned), key (l,e) at index l*n_experts+e.
 * policy: MOE_CACHE_GLOBAL_LRU (one pool) or MOE_CACHE_PER_LAYER_LRU (layer l
 * owns slots [l*S/L, (l+1)*S/L)).  backend: MOE_CACHE_BACKEND_HIP copies with
 * hipMemcpyAsync on the cache's own copy stream; MOE_CACHE_BACKEND_HOST keeps
 * slots in host memory and copies with memcpy (no GPU; for tests of the
 * logic).
 *
 * moe_cache_stage(DEMAND): ids_host [n] in rank order.  A resident key is a hit
 * (touched); a missing key takes the least-recently-used unlocked slot (never
 * used slots first, ties to the lowest slot), is copied, and counts as
 * resident at once; `compute` (a hipStream_t) is made to wait for every fill
 * it depends on; slots used are locked until moe_cache_release(layer).
 * dev_ptrs_host_out [n] receives the slot addresses.  E_CAPACITY if fewer than
 * n slots are unlocked (nothing changes).
 * moe_cache_stage(PREFETCH): same lookup for a predicted set, but never waits,
 * never evicts a locked slot, and skips (counted) when no unlocked slot is
 * left; prefetched slots are not locked.
 * moe_cache_stage(PREFETCH_IDLE): PREFETCH only while the copy engine is idle:
 * when copies issued earlier are still running on the cache's copy stream, the
 * whole request is skipped (each id counted in prefetch_skipped, event kind
 * 8), so a guess never delays a demand copy.  Where one layer computes in far
 * less time than one expert takes to cross PCIe, streaming is copy-bound and
 * prefetching wrong guesses only costs copy time; this form prefetches into
 * the idle gaps alone.  Which requests run depends on timing (the HOST backend
 * copies synchronously and is never busy: there it equals PREFETCH).
 * moe_cache_release: unlocks the slots of `layer`; before a released slot is
 * refilled, the copy stream waits until the work enqueued on `compute` up to
 * the release has finished (no write-after-read hazard).
 * moe_cache_table: device array [n_experts] of the current slot address of
 * each resident (layer, e), NULL elsewhere; valid on `compute` after a DEMAND
 * stage of that layer.
 * Errors: E_INVAL (ids out of range, NULL blobs), E_CAPACITY, E_HIP (a failed
 * copy leaves its slot empty; the next stage retries), E_NOMEM. */
#define MOE_CACHE_GLOBAL_LRU     0
#define MOE_CACHE_PER_LAYER_LRU  1
#define MOE_CACHE_BACKEND_HIP    0
#define MOE_CACHE_BACKEND_HOST   1
#define MOE_STAGE_DEMAND   0
#define MOE_STAGE_PREFETCH 1
#define MOE_STAGE_PREFETCH_IDLE 2

typedef struct moe_cache_desc {
    int32_t device;
    int32_t n_layers;
    int32_t n_experts;
    size_t blob_bytes;
    size_t capacity_bytes;
    const void *const *host_blobs;
    int32_t policy;
    int32_t backend;
} moe_cache_desc;

/* Counters since creation or the last reset.  copy_busy_ms: the summed
 * durations of the host-to-device copies (HIP backend; the copy stream runs
 * them one at a time, so this is the copy engine's busy time), timed by event
 * pairs around each copy; copies_timed: how many.  moe_cache_stats_get waits
 * for the copies issued so far to finish before it reads them. */
typedef struct moe_cache_stats {
    int64_t demand_hits, demand_misses;
    int64_t prefetch_issued, prefetch_used, prefetch_wasted, prefetch_skipped;
    int64_t prefetch_resident;
    int64_t evictions;
    int64_t bytes_copied;
    int64_t n_slots;
    int64_t pinned, pin_fills;
    double copy_busy_ms;
    int64_t copies_timed;
} moe_cache_stats;

/* One logical cache event (kind: 0 hit, 1 miss, 2 prefetch issued, 3 prefetch
 * already resident, 4 prefetch skipped, 5 eviction, 6 pinned key copied in,
 * 7 pinned key already resident, 8 prefetch skipped: copy engine busy). */
typedef struct moe_cache_event {
    int32_t kind, layer, expert, slot;
} moe_cache_event;

moe_status moe_cache_create(const moe_cache_desc *desc, moe_cache **out);
void moe_cache_destroy(moe_cache *cache);
moe_status moe_cache_stage(moe_cache *cache, int32_t layer,
                           const int32_t *ids_host, int32_t n, int32_t mode,
                           void *compute, const void **dev_ptrs_host_out);
moe_status moe_cache_release(moe_cache *cache, int32_t layer, void *compute);
const void *const *moe_cache_table(moe_cache *cache, int32_t layer);
moe_status moe_cache_stats_get(const moe_cache *cache, moe_cache_stats *out);
void moe_cache_reset_stats(moe_cache *cache);
/* Copies up to cap events of the log (oldest first) and returns how many were
 * written; the log is kept only when enabled. */
moe_status moe_cache_log_enable(moe_cache *cache, int32_t on);
int64_t moe_cache_event_log(const moe_cache *cache, moe_cache_event *out, int64_t cap);
/* Learned pinned hot-store.  Source: aifrontierpost tutorial, introduction
 * (measured routing heat drives the LRU cache and a learned pinned hot-store)
 * and "Step 4 -- Run it" (the usage file records which experts the workload
 * routes to and the hottest are pinned); kongchang article, storage-tier
 * section (expert usage is recorded, hit rates grow with use).
 * Every DEMAND access of key (l, e) adds one to usage[l*n_experts + e]
 * (prefetches do not count).  moe_cache_pin_hot: between layers (no slot
 * locked; else E_INVAL and nothing changes) unpins every slot, then takes the
 * keys with a nonzero count by count descending, key ascending, and pins them
 * until n are pinned: a resident key's slot as it is, a missing key copied
 * into the LRU unlocked unpinned slot of its partition (on the copy stream,
 * waited for by the next DEMAND of the key as any fill).  At most (partition
 * slots - reserve) slots of a partition are pinned (reserve >= 1: pass at
 * least the number of distinct experts one layer call demands), so a layer
 * always finds room; keys whose partition is full are passed over.  A pinned
 * slot is never evicted by DEMAND, PREFETCH or a later pin until the next
 * moe_cache_pin_hot.  moe_cache_usage_get / _set copy the [n_layers *
 * n_experts] counts out / in (host memory), so a caller can keep them across
 * runs.  Errors: E_INVAL, E_CAPACITY, E_HIP (a failed copy). */
moe_status moe_cache_pin_hot(moe_cache *cache, int32_t n, int32_t reserve);
moe_status moe_cache_usage_get(const moe_cache *cache, int64_t *usage_host);
moe_status moe_cache_usage_set(moe_cache *cache, const int64_t *usage_host);
/* Test hook: the next copy fails as if the runtime had reported an error. */
moe_status moe_cache_debug_fail_next_copy(moe_cache *cache);

/* ---- helpers ------------------------------------------------------------------- */
moe_status moe_host_alloc_pinned(size_t bytes, void **out);
moe_status moe_host_free_pinned(void *p);
const char *moe_last_error(void);

/* ---- kernel timing (measurement) ---------------------------------------------------
 * When on, every hot call on ctx has each kernel it enqueues (on the call's
 * stream) stamped with a HIP event pair taken from the kernel's own dispatch
 * (hipExtLaunchKernelGGL), from a ring of 256 pairs per kind.  Calls do not wait for the events, so
 * profiled calls run back to back like unprofiled ones; only when a kind's
 * ring is full does the next call of that kind wait for its oldest records.
 * moe_ctx_profile_read waits for every recorded kernel, copies the totals
 * (milliseconds) and launch counts for the MOE_PROF_N kinds below and resets
 * them; it returns MOE_E_HIP if an event could not be read.  Results of the
 * hot calls are unchanged.  Not for use while a stream is being captured. */
#define MOE_PROF_ROUTER  0    /* router logits */
#define MOE_PROF_TOPK    1
#define MOE_PROF_QUANT   2
#define MOE_PROF_PERMUTE 3
#define MOE_PROF_GATEUP  4    /* gate/up projections + SwiGLU */
#define MOE_PROF_REQUANT 5
#define MOE_PROF_DOWN    6
#define MOE_PROF_COMBINE 7
#define MOE_PROF_TILES   8    /* MFMA tile list */
#define MOE_PROF_N       9
moe_status moe_ctx_profile(moe_ctx *ctx, int32_t on);
moe_status moe_ctx_profile_read(moe_ctx *ctx, double *ms, int64_t *counts);

/* ---- inspection (tests) ---------------------------------------------------------
 * Copies a workspace buffer of the last call on ctx into dst (device memory,
 * caller-owned, `bytes` long) on `stream`.  which: 0 activation codes [T,H]
 * int8, 1 token scales [T] fp32, 2 router logits [T,E] fp64, 3 SwiGLU outputs h
 * [T,S,F] fp32, 4 requantised h codes [T,S,F] int8, 5 their scales [T,S] fp32,
 * 6 expert outputs Y [T,S,H] fp32, 7 (MXFP4 layers) SwiGLU outputs h as bf16
 * [T,S,F]; S = k + n_shared slots per token (slot k is the shared expert).
 * E_INVAL if bytes exceeds the buffer or the buffer does not exist. */
moe_status moe_debug_read(moe_ctx *ctx, int32_t which, void *dst, size_t bytes,
                          void *stream);
/* Raw int4 x int8 projection of one packed weight matrix of a blob
 * (part 0 gate, 1 up, 2 down) on int8 rows q_in [T,K] with scales s_in [T]:
 * y [T,N] fp32 = fp32(fp64(exact group sums x scales) * s_in).  Uses the same
 * kernels as the FFN path selected by moe_ctx_set_path. */
moe_status moe_debug_project(moe_ctx *ctx, const void *blob, int32_t part,
                             const int8_t *q_in, const float *s_in, int32_t T,
                             float *y, void *stream);
/* Measurement helper: reads `bytes` of device memory at src (16-byte aligned,
 * a nonzero multiple of 65536) with the 16-byte non-temporal loads the decode
 * kernels use for expert weights, 64 KiB per block; sink [bytes/65536]
 * (device, caller-owned) receives the XOR of the 32-bit words of each 64 KiB
 * block.  Enqueued on `stream`; E_INVAL on a bad argument, nothing enqueued. */
moe_status moe_debug_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif
