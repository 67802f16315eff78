// api.cpp -- C ABI of the quantised MoE layer: argument validation, context
// and workspace, and the order of kernel launches for each call.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "host_common.h"

using namespace moe;

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
// a fixed buffer: reporting an error allocates nothing
static thread_local char g_last_error[512];

namespace moe {
moe_status fail(moe_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

moe_status hip_fail(hipError_t e, const char *what)
{
    return fail(MOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

moe_status validate_desc(const moe_layer_desc *d)
{
    if (!d)
        return fail(MOE_E_INVAL, "desc is NULL");
    if (d->hidden <= 0 || d->hidden % 256)
        return fail(MOE_E_INVAL, "hidden=%d must be a positive multiple of 256", d->hidden);
    if (d->ffn <= 0 || d->ffn % 256)
        return fail(MOE_E_INVAL, "ffn=%d must be a positive multiple of 256", d->ffn);
    if (d->n_experts < 1 || d->n_experts > 1024)
        return fail(MOE_E_INVAL, "n_experts=%d must be in [1,1024]", d->n_experts);
    if (d->top_k < 1 || d->top_k > 32 || d->top_k > d->n_experts)
        return fail(MOE_E_INVAL, "top_k=%d must be in [1, min(n_experts,32)]", d->top_k);
    if (d->n_shared != 0 && d->n_shared != 1)
        return fail(MOE_E_INVAL, "n_shared=%d must be 0 or 1", d->n_shared);
    if (d->wfmt == MOE_WFMT_INT4) {
        if (d->group != 32 && d->group != 64)
            return fail(MOE_E_INVAL, "group=%d must be 32 or 64 for int4", d->group);
    } else if (d->wfmt == MOE_WFMT_MXFP4) {
        if (d->group != 32)
            return fail(MOE_E_INVAL, "group=%d must be 32 for mxfp4", d->group);
    } else {
        return fail(MOE_E_INVAL, "unknown weight format %d", d->wfmt);
    }
    if (!(d->routed_scale == d->routed_scale) || d->routed_scale < 0.0f ||
        d->routed_scale > 1.0e30f)
        return fail(MOE_E_INVAL, "routed_scale must be finite and >= 0");
    if (d->out_dtype != MOE_DT_F32 && d->out_dtype != MOE_DT_BF16)
        return fail(MOE_E_INVAL, "unknown out_dtype %d", d->out_dtype);
    return MOE_OK;
}
}  // namespace moe

extern "C" const char *moe_last_error(void)
{
    return g_last_error;
}

// ---------------------------------------------------------------------------
// context
// ---------------------------------------------------------------------------

static moe_status ws_alloc(moe_ctx *c, void **p, size_t bytes)
{
    void *q = nullptr;
    if (bytes == 0)
        bytes = 16;
    hipError_t e = hipMalloc(&q, bytes);
    if (e != hipSuccess)
        return fail(MOE_E_NOMEM, "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    c->allocs.push_back(q);
    *p = q;
    return MOE_OK;
}

static void ctx_free(moe_ctx *c)
{
    if (!c)
        return;
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(c->device);
    for (void *p : c->allocs)
        (void)hipFree(p);
    for (hipEvent_t ev : c->prof_ev)
        if (ev)
            (void)hipEventDestroy(ev);
    (void)hipSetDevice(prev);
    delete c;
}

namespace moe {
moe_status check_device(int device)
{
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n <= 0)
        return fail(MOE_E_UNSUPPORTED, "no HIP device available");
    if (device < 0 || device >= n)
        return fail(MOE_E_INVAL, "device %d out of range [0,%d)", device, n);
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDeviceProperties");
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(MOE_E_UNSUPPORTED, "device %d is %s; this library runs on gfx950 only",
                    device, prop.gcnArchName);
    return MOE_OK;
}
}  // namespace moe

extern "C" moe_status moe_ctx_create(int32_t device, const moe_layer_desc *desc,
                                     int32_t max_tokens, moe_ctx **out)
{
    if (!out)
        return fail(MOE_E_INVAL, "out is NULL");
    *out = nullptr;
    moe_status st = validate_desc(desc);
    if (st)
        return st;
    if (max_tokens < 1 || max_tokens > (1 << 20))
        return fail(MOE_E_INVAL, "max_tokens=%d must be in [1, 2^20]", max_tokens);
    st = check_device(device);
    if (st)
        return st;
    hipError_t e = hipSetDevice(device);
    if (e != hipSuccess)
        return hip_fail(e, "hipSetDevice");
    moe_ctx *c = new moe_ctx();
    c->device = device;
    c->d = *desc;
    c->max_tokens = max_tokens;
    c->L = blob_layout(desc->hidden, desc->ffn, desc->group, desc->wfmt);
    c->S = desc->top_k + desc->n_shared;
    st = ws_plan(c, [c](void **p, size_t bytes, int) { return ws_alloc(c, p, bytes); });
    if (st) {
        ctx_free(c);
        return st;
    }
    const size_t T = (size_t)max_tokens, H = desc->hidden, E = desc->n_experts;
    std::vector<int32_t> ident(T);
    for (size_t i = 0; i < T; ++i)
        ident[i] = (int32_t)i;
    const int32_t zero = 0, one = 1;
    if ((e = hipMemcpy(c->ident, ident.data(), T * 4, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(c->zero1, &zero, 4, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(c->one1, &one, 4, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemset(c->done, 0, 16)) != hipSuccess ||
        (e = hipMemset(c->ctr_gu, 0, (E + 1) * 4)) != hipSuccess ||
        (e = hipMemset(c->ctr_dn, 0, (H / 32) * 4)) != hipSuccess ||
        (e = hipMemset(c->n_tiles, 0, 16)) != hipSuccess) {
        ctx_free(c);
        return hip_fail(e, "workspace init");
    }
    *out = c;
    return MOE_OK;
}

extern "C" void moe_ctx_destroy(moe_ctx *ctx)
{
    ctx_free(ctx);
}

extern "C" moe_status moe_ctx_set_path(moe_ctx *ctx, int32_t path)
{
    if (!ctx)
        return fail(MOE_E_INVAL, "ctx is NULL");
    if (path != MOE_PATH_AUTO && path != MOE_PATH_GEMV && path != MOE_PATH_MFMA &&
        path != MOE_PATH_MX_BF16)
        return fail(MOE_E_INVAL, "unknown path %d", path);
    if (path == MOE_PATH_MFMA && ctx->d.wfmt != MOE_WFMT_INT4)
        return fail(MOE_E_UNSUPPORTED, "the int8 MFMA path covers int4 weights");
    if (path == MOE_PATH_MX_BF16 && ctx->d.wfmt != MOE_WFMT_MXFP4)
        return fail(MOE_E_UNSUPPORTED, "the bf16 MX path covers MXFP4 weights");
    ctx->path = path;
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// hot calls
// ---------------------------------------------------------------------------
static moe_status check_call(moe_ctx *ctx, const void *x, int32_t T, const moe_layer_weights *w)
{
    if (!ctx)
        return fail(MOE_E_INVAL, "ctx is NULL");
    if (T < 0 || T > ctx->max_tokens)
        return fail(MOE_E_INVAL, "T=%d out of range [0,%d]", T, ctx->max_tokens);
    if (T > 0 && !x)
        return fail(MOE_E_INVAL, "x is NULL");
    if (!w)
        return fail(MOE_E_INVAL, "weights is NULL");
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
namespace moe {
ProfSlot &prof_slot()
{
    static thread_local ProfSlot slot;
    return slot;
}

static hipEvent_t prof_event(moe_ctx *c, int k, int64_t i, int which)
{
    return c->prof_ev[((size_t)k * moe_ctx::PROF_RING + (size_t)(i % moe_ctx::PROF_RING)) * 2 + which];
}

// waits for every recorded launch of kind k and adds up its duration
static hipError_t prof_drain(moe_ctx *c, int k)
{
    for (; c->prof_tail[k] < c->prof_head[k]; ++c->prof_tail[k]) {
        const int64_t i = c->prof_tail[k];
        hipError_t e = hipEventSynchronize(prof_event(c, k, i, 1));
        float ms = 0.0f;
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, prof_event(c, k, i, 0), prof_event(c, k, i, 1));
        if (e != hipSuccess) {
            c->prof_tail[k] = c->prof_head[k];
            return e;
        }
        c->prof_ms[k] += ms;
        c->prof_cnt[k] += 1;
    }
    return hipSuccess;
}

void prof_begin(moe_ctx *c, int k, hipStream_t st)
{
    if (!c->prof_on)
        return;
    if (c->prof_head[k] - c->prof_tail[k] >= moe_ctx::PROF_RING) {
        const hipError_t e = prof_drain(c, k);
        if (e != hipSuccess && c->prof_err == hipSuccess)
            c->prof_err = e;
    }
    (void)st;
    const int64_t i = c->prof_head[k];
    ProfSlot &p = prof_slot();
    p.start = prof_event(c, k, i, 0);
    p.stop = prof_event(c, k, i, 1);
    p.used = false;
}

// counts the launch if launch() stamped it (a launcher that found nothing to
// do enqueues no kernel and is not counted)
void prof_end(moe_ctx *c, int k, hipStream_t st)
{
    (void)st;
    if (!c->prof_on)
        return;
    ProfSlot &p = prof_slot();
    if (p.used)
        c->prof_head[k] += 1;
    p = ProfSlot{};
}

moe_status prof_collect(moe_ctx *c)
{
    if (c->prof_err != hipSuccess) {
        const hipError_t e = c->prof_err;
        c->prof_err = hipSuccess;
        return hip_fail(e, "profiling events");
    }
    return MOE_OK;
}
}  // namespace moe

extern "C" moe_status moe_ctx_profile(moe_ctx *ctx, int32_t on)
{
    if (!ctx)
        return fail(MOE_E_INVAL, "ctx is NULL");
    if (on && ctx->prof_ev.empty()) {
        ctx->prof_ev.assign((size_t)2 * MOE_PROF_N * moe_ctx::PROF_RING, nullptr);
        for (hipEvent_t &ev : ctx->prof_ev) {
            hipError_t e = hipEventCreate(&ev);
            if (e != hipSuccess)
                return hip_fail(e, "hipEventCreate");
        }
    }
    ctx->prof_on = on != 0;
    return MOE_OK;
}

extern "C" moe_status moe_ctx_profile_read(moe_ctx *ctx, double *ms, int64_t *counts)
{
    if (!ctx || !ms || !counts)
        return fail(MOE_E_INVAL, "NULL argument");
    hipError_t err = hipSuccess;
    for (int k = 0; k < MOE_PROF_N; ++k) {
        const hipError_t e = prof_drain(ctx, k);
        if (e != hipSuccess && err == hipSuccess)
            err = e;
    }
    for (int k = 0; k < MOE_PROF_N; ++k) {
        ms[k] = ctx->prof_ms[k];
        counts[k] = ctx->prof_cnt[k];
        ctx->prof_ms[k] = 0.0;
        ctx->prof_cnt[k] = 0;
    }
    return err != hipSuccess ? hip_fail(err, "profiling events") : MOE_OK;
}

// Runs `expr` (a launcher returning hipError_t) bracketed by timing events.
#define LAUNCH(kind, what, expr)                 \
    do {                                         \
        prof_begin(c, (kind), st);               \
        hipError_t e_ = (expr);                  \
        if (e_ != hipSuccess)                    \
            return hip_fail(e_, what);           \
        prof_end(c, (kind), st);                 \
    } while (0)

// One token on the GEMV path (where the one-token kernels do not apply):
// routing, quantisation and lists in one launch, requant and combine fused
// into the projections.  From two tokens on, separate launches (router GEMV,
// top-k, quantisation, permutation, projections, requant, combine) measured
// 7-32 % faster at 2-16 tokens than this fused form: its single-block top-k
// runs the tokens one after another and its cross-block tails wait on
// device-scope counters.
static bool small_path(const moe_ctx *c, int T)
{
    // the fused down kernel requantises SwiGLU rows of up to 4096 values
    // (the fused kernels keep a token's router slice and a SwiGLU row in registers)
    // (and at most 16 ranks: the fused routing launch keeps 16 candidates)
    return T == 1 && c->d.wfmt == MOE_WFMT_INT4 && c->d.ffn <= 4096 &&
           c->d.hidden <= 8192 && c->d.top_k <= 16 && !use_mfma(c, T);
}

// Whether all expert blobs of a layer fit the last-level cache (the 256 MiB
// Infinity Cache of an MI355X): then the few-token projections read them with
// plain loads and they stay cached from one call to the next.
static bool experts_fit_llc(const moe_layer_desc &d, const BlobLayout &L)
{
    constexpr double kLastLevelCacheBytes = 256.0 * 1024 * 1024;
    return (double)(d.n_experts + d.n_shared) * (double)L.total <= kLastLevelCacheBytes;
}

// One token: expert FFN straight from the top-k output (kernels_bs1.hip).
static bool bs1_path(const moe_ctx *c, int T)
{
    return T == 1 && small_path(c, T) &&
           bs1_supported(c->d.hidden, c->d.ffn, c->d.top_k, c->d.n_shared);
}

static Bs1Args make_bs1(const moe_ctx *c, const moe_layer_weights *w,
                        const void *const *expert_ptrs, const int32_t *idx, const float *gw,
                        void *out, bool sel_ready)
{
    const moe_layer_desc &d = c->d;
    Bs1Args b{};
    b.ex.ptrs = expert_ptrs;
    b.ex.shared = w->shared;
    b.ex.E = d.n_experts;
    b.sel = sel_ready ? c->sel : nullptr;
    b.idx = idx;
    b.w = gw;
    b.k = d.top_k;
    b.n_shared = d.n_shared;
    b.xq = c->xq;
    b.sa = c->sa;
    b.H = d.hidden;
    b.F = d.ffn;
    b.group_shift = (d.group == 64) ? 1 : 0;
    b.gu_w = c->L.gu_w;
    b.gu_s = c->L.gu_s;
    b.gu_tile_w = c->L.gu_tile_w;
    b.gu_tile_s = c->L.gu_tile_s;
    b.dn_w = c->L.dn_w;
    b.dn_s = c->L.dn_s;
    b.dn_tile_w = c->L.dn_tile_w;
    b.dn_tile_s = c->L.dn_tile_s;
    b.h = c->h;
    b.qh = c->qh;
    b.sh = c->sh;
    b.Y = c->Y;
    b.out = out;
    b.out_dtype = d.out_dtype;
    return b;
}

static RouteSmallArgs route_small_args(moe_ctx *c, const void *x, int T, const moe_layer_weights *w,
                                       int32_t *idx, float *gw, int flags)
{
    const moe_layer_desc &d = c->d;
    RouteSmallArgs r{};
    r.x = static_cast<const uint16_t *>(x);
    r.T = T;
    r.H = d.hidden;
    r.Wr = w ? w->router_w : nullptr;
    r.bias = w ? w->router_bias : nullptr;
    r.E = d.n_experts;
    r.k = d.top_k;
    r.r = d.routed_scale;
    r.logits = c->logits;
    r.idx = idx;
    r.w = gw;
    r.flags = flags;
    r.xq = c->xq;
    r.sa = c->sa;
    r.cnt = c->cnt;
    r.list = c->list;
    r.list_stride = c->max_tokens;
    r.active = c->active;
    r.n_active = c->n_active;
    r.n_shared = d.n_shared;
    r.done = c->done;
    r.ptrs = w ? w->expert_ptrs : nullptr;
    r.sel = c->sel;
    return r;
}

// Router + top-k.  On the one-token GEMV path `extra` (RS_QUANT | RS_LISTS)
// folds the token quantisation and the routing lists into the same launch;
// otherwise RS_QUANT has the top-k launch quantise the tokens (hidden <= 8192).
static moe_status router_enqueue(moe_ctx *c, const void *x, int32_t T, const moe_layer_weights *w,
                                 int32_t *idx, float *gw, hipStream_t st, int extra = 0)
{
    if (!w->router_w || !w->router_bias)
        return fail(MOE_E_INVAL, "router weights are NULL");
    const moe_layer_desc &d = c->d;
    if (small_path(c, T)) {
        LAUNCH(MOE_PROF_ROUTER, "routing launch",
               launch_route_small(route_small_args(c, x, T, w, idx, gw, RS_ROUTER | extra), st));
        return MOE_OK;
    }
    LAUNCH(MOE_PROF_ROUTER, "router logits launch",
           launch_router_logits(static_cast<const uint16_t *>(x), T, d.hidden, w->router_w,
                                d.n_experts, c->logits, st));
    const bool q = (extra & RS_QUANT) != 0;
    LAUNCH(MOE_PROF_TOPK, "top-k launch",
           launch_topk(c->logits, w->router_bias, T, d.n_experts, d.top_k, d.routed_scale, idx,
                       gw, st, q ? static_cast<const uint16_t *>(x) : nullptr, d.hidden,
                       q ? c->xq : nullptr, q ? c->sa : nullptr,
                       router_ksplit(T, d.hidden, d.n_experts)));
    return MOE_OK;
}

// One token, E <= 256: router logits, scores and the token codes in one
// launch, then the top-k (with the shared expert's gate/up beside it).
static moe_status router_bs1_enqueue(moe_ctx *c, const void *x, const moe_layer_weights *w,
                                     int32_t *idx, float *gw, bool sel, hipStream_t st)
{
    if (!w->router_w || !w->router_bias)
        return fail(MOE_E_INVAL, "router weights are NULL");
    if (c->d.n_shared && !w->shared)
        return fail(MOE_E_INVAL, "shared expert blob is NULL");
    const RouteSmallArgs ra = route_small_args(c, x, 1, w, idx, gw, RS_QUANT);
    LAUNCH(MOE_PROF_ROUTER, "router launch", launch_router_bs1(ra, st));
    const Bs1Args b = make_bs1(c, w, nullptr, idx, gw, nullptr, false);
    LAUNCH(MOE_PROF_TOPK, "top-k launch",
           launch_topk_bs1(c->logits, w->router_bias, c->d.n_experts, c->d.routed_scale,
                           sel ? w->expert_ptrs : nullptr,
                           idx, gw, c->sel, b, st));
    return MOE_OK;
}

extern "C" moe_status moe_router_topk(moe_ctx *ctx, const void *x, int32_t T,
                                      const moe_layer_weights *w, int32_t *idx, float *gate_w,
                                      void *stream)
{
    moe_status s = check_call(ctx, x, T, w);
    if (s)
        return s;
    if (T == 0)
        return MOE_OK;
    if (!idx || !gate_w)
        return fail(MOE_E_INVAL, "idx/gate_w is NULL");
    ctx->last_T = T;
    s = router_enqueue(ctx, x, T, w, idx, gate_w, static_cast<hipStream_t>(stream));
    if (s)
        return s;
    return prof_collect(ctx);
}

static int mg_for(int T)
{
    int mg = 1;
    while (mg < T && mg < 8)
        mg <<= 1;
    return mg;
}

// prepped: the router launch already quantised x (and built the lists, or
// with sel_ready selected the blobs of the ranks; with shared_done it also ran
// the shared expert's gate/up).
static moe_status ffn_enqueue(moe_ctx *c, const void *x, int32_t T, const moe_layer_weights *w,
                              const void *const *expert_ptrs, const int32_t *idx,
                              const float *gw, void *out, hipStream_t st, bool prepped = false,
                              bool sel_ready = false, bool shared_done = false)
{
    const moe_layer_desc &d = c->d;
    const int H = d.hidden, F = d.ffn, E = d.n_experts, k = d.top_k;
    if (d.n_shared && !w->shared)
        return fail(MOE_E_INVAL, "shared expert blob is NULL");
    if (!expert_ptrs)
        return fail(MOE_E_INVAL, "expert_ptrs is NULL");
    if (d.wfmt == MOE_WFMT_MXFP4)
        return mx_ffn_enqueue(c, x, T, w, expert_ptrs, idx, gw, out, st);
    if (bs1_path(c, T)) {
        if (!prepped) {
            RouteSmallArgs ra = route_small_args(c, x, T, nullptr, const_cast<int32_t *>(idx),
                                                 const_cast<float *>(gw), RS_QUANT | RS_SEL);
            ra.ptrs = expert_ptrs;
            LAUNCH(MOE_PROF_QUANT, "quant launch", launch_route_small(ra, st));
            sel_ready = true;
        }
        const Bs1Args b = make_bs1(c, w, expert_ptrs, idx, gw, out, sel_ready);
        LAUNCH(MOE_PROF_GATEUP, "gate/up launch",
               launch_gateup_bs1(b, shared_done ? k : k + d.n_shared, st));
        LAUNCH(MOE_PROF_DOWN, "down launch", launch_down_bs1(b, st));
        return MOE_OK;
    }
    const bool small = small_path(c, T);
    if (small && !prepped) {
        LAUNCH(MOE_PROF_QUANT, "quant/lists launch",
               launch_route_small(route_small_args(c, x, T, nullptr, const_cast<int32_t *>(idx),
                                                   const_cast<float *>(gw), RS_QUANT | RS_LISTS),
                                  st));
    } else if (!small) {
        if (!prepped)
            LAUNCH(MOE_PROF_QUANT, "quant launch",
                   launch_quant_tokens(static_cast<const uint16_t *>(x), T, H, c->xq, c->sa, st));
        LAUNCH(MOE_PROF_PERMUTE, "permute launch",
               launch_permute(idx, T, k, E, d.n_shared, c->cnt, c->list, c->max_tokens, c->active,
                              c->n_active, c->done, st));
    }
    TailArgs tail{};
    tail.qh = c->qh;
    tail.sh = c->sh;
    tail.F = F;
    tail.idx = idx;
    tail.w = gw;
    tail.T = T;
    tail.k = k;
    tail.E = E;
    tail.n_shared = d.n_shared;
    tail.H = H;
    tail.out_dtype = d.out_dtype;
    tail.out = out;
    const int max_active = (T * k < E ? T * k : E) + d.n_shared;
    const int mg = mg_for(T);

    ProjArgs a{};
    a.ex.ptrs = expert_ptrs;
    a.ex.shared = w->shared;
    a.ex.E = E;
    a.cached = experts_fit_llc(d, c->L) ? 1 : 0;
    a.rt.active = c->active;
    a.rt.n_active = c->n_active;
    a.rt.cnt = c->cnt;
    a.rt.list = c->list;
    a.rt.list_stride = c->max_tokens;
    a.rt.S = c->S;
    a.group_shift = (d.group == 64) ? 1 : 0;

    const bool mfma = use_mfma(c, T);
    // gate/up + SwiGLU -> h [T*S, F]
    a.q = c->xq;
    a.s = c->sa;
    a.in_by_token = 1;
    a.K = H;
    a.w_off = c->L.gu_w;
    a.s_off = c->L.gu_s;
    a.tile_w = c->L.gu_tile_w;
    a.tile_s = c->L.gu_tile_s;
    if (mfma) {
        LAUNCH(MOE_PROF_TILES, "tile list launch", launch_mfma_tiles(c, T, st));
        LAUNCH(MOE_PROF_GATEUP, "gate/up launch", launch_gateup_mfma(a, c, T, F, c->h, F, st));
    } else {
        tail.ctr = c->ctr_gu;
        LAUNCH(MOE_PROF_GATEUP, "gate/up launch",
               launch_gateup_gemv(a, max_active, F, mg, c->h, F, small ? &tail : nullptr, st));
    }
    if (!small)
        LAUNCH(MOE_PROF_REQUANT, "requant launch",
               launch_requant(c->h, T * c->S, F, c->qh, c->sh, st));
    // down -> Y [T*S, H]
    a.q = c->qh;
    a.s = c->sh;
    a.in_by_token = 0;
    a.K = F;
    a.w_off = c->L.dn_w;
    a.s_off = c->L.dn_s;
    a.tile_w = c->L.dn_tile_w;
    a.tile_s = c->L.dn_tile_s;
    a.tile_base = 0;
    a.pair_stride = 2;
    a.j_stride = 1;
    a.out = c->Y;
    a.ldo = H;
    tail.ctr = c->ctr_dn;
    if (mfma)
        LAUNCH(MOE_PROF_DOWN, "down launch", launch_proj_mfma(a, c, T, H, st));
    else
        LAUNCH(MOE_PROF_DOWN, "down launch",
               launch_proj_gemv(a, max_active, H / 32, mg, small ? &tail : nullptr, st));
    if (!small)
        LAUNCH(MOE_PROF_COMBINE, "combine launch",
               launch_combine(c->Y, idx, gw, T, k, E, d.n_shared, H, out, d.out_dtype, st));
    return MOE_OK;
}

extern "C" moe_status moe_expert_ffn(moe_ctx *ctx, const void *x, int32_t T,
                                     const moe_layer_weights *w, const int32_t *idx,
                                     const float *gate_w, void *out, void *stream)
{
    moe_status s = check_call(ctx, x, T, w);
    if (s)
        return s;
    if (T == 0)
        return MOE_OK;
    if (!idx || !gate_w || !out)
        return fail(MOE_E_INVAL, "idx/gate_w/out is NULL");
    ctx->last_T = T;
    s = ffn_enqueue(ctx, x, T, w, w->expert_ptrs, idx, gate_w, out,
                    static_cast<hipStream_t>(stream));
    if (s)
        return s;
    return prof_collect(ctx);
}

extern "C" moe_status moe_layer_forward(moe_ctx *ctx, const void *x, int32_t T,
                                        const moe_layer_weights *w, moe_cache *cache,
                                        int32_t layer, int32_t *idx_out, float *gate_w_out,
                                        void *out, void *stream)
{
    moe_status s = check_call(ctx, x, T, w);
    if (s)
        return s;
    return layer_forward_enqueue(ctx, x, T, w, cache, layer, idx_out, gate_w_out, out,
                                 static_cast<hipStream_t>(stream));
}

moe_status moe::layer_forward_enqueue(moe_ctx *ctx, const void *x, int32_t T,
                                      const moe_layer_weights *w, moe_cache *cache,
                                      int32_t layer, int32_t *idx_out, float *gate_w_out,
                                      void *out, hipStream_t st)
{
    moe_status s = MOE_OK;
    if (T == 0)
        return MOE_OK;
    if (!out)
        return fail(MOE_E_INVAL, "out is NULL");
    if (cache) {
        s = cache_check_for_layer(cache, ctx->d, layer, T);
        if (s)
            return s;
    }
    if (!w->router_w || !w->router_bias)
        return fail(MOE_E_INVAL, "router weights are NULL");
    if (ctx->d.n_shared && !w->shared)
        return fail(MOE_E_INVAL, "shared expert blob is NULL");
    if (!cache && !w->expert_ptrs)
        return fail(MOE_E_INVAL, "expert_ptrs is NULL");
    int32_t *idx = idx_out ? idx_out : ctx->idx;
    float *gw = gate_w_out ? gate_w_out : ctx->gw;
    ctx->last_T = T;
    // one token: quantisation (and, on the GEMV fallback, the routing lists)
    // ride on the router launch.  One token with E <= 256: the router is two
    // launches, the second also runs the shared expert's gate/up and, without
    // the cache, picks the ranks' blobs.
    const bool fused = small_path(ctx, T) && ctx->d.wfmt == MOE_WFMT_INT4;
    const bool bs1 = bs1_path(ctx, T);
    const bool two = bs1 && ctx->d.n_experts <= 256;
    const bool sel = two && !cache && w->expert_ptrs;
    // more tokens: the top-k launch quantises them
    const bool rq = !bs1 && !fused && ctx->d.wfmt == MOE_WFMT_INT4 && ctx->d.hidden <= 8192;
    if (two)
        s = router_bs1_enqueue(ctx, x, w, idx, gw, sel, st);
    else
        s = router_enqueue(ctx, x, T, w, idx, gw, st,
                           (bs1 || rq) ? RS_QUANT : fused ? (RS_QUANT | RS_LISTS) : 0);
    if (s)
        return s;
    const void *const *ptrs = w->expert_ptrs;
    if (cache) {
        // the caller may prefetch the next layer after this call, then calls
        // moe_cache_release
        s = cache_demand_for_layer(cache, ctx->d, layer, idx, T, st, &ptrs);
        if (s)
            return s;
    }
    s = ffn_enqueue(ctx, x, T, w, ptrs, idx, gw, out, st, fused || rq, sel, two && ctx->d.n_shared);
    if (s)
        return s;
    return prof_collect(ctx);
}

// ---------------------------------------------------------------------------
// inspection
// ---------------------------------------------------------------------------
extern "C" moe_status moe_debug_read(moe_ctx *ctx, int32_t which, void *dst, size_t bytes,
                                     void *stream)
{
    if (!ctx || !dst)
        return fail(MOE_E_INVAL, "ctx/dst is NULL");
    const size_t T = ctx->max_tokens, H = ctx->d.hidden, F = ctx->d.ffn, S = ctx->S;
    const void *src = nullptr;
    size_t cap = 0;
    switch (which) {
    case 0: src = ctx->xq; cap = T * H; break;
    case 1: src = ctx->sa; cap = T * 4; break;
    case 2: src = ctx->logits; cap = T * ctx->d.n_experts * 8; break;
    case 3: src = ctx->h; cap = T * S * F * 4; break;
    case 4: src = ctx->qh; cap = T * S * F; break;
    case 5: src = ctx->sh; cap = T * S * 4; break;
    case 6: src = ctx->Y; cap = T * S * H * 4; break;
    case 7: src = ctx->hb; cap = ctx->hb ? T * S * F * 2 : 0; break;
    default: return fail(MOE_E_INVAL, "unknown buffer %d", which);
    }
    if (bytes > cap)
        return fail(MOE_E_INVAL, "bytes=%zu exceeds buffer size %zu", bytes, cap);
    hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "hipMemcpyAsync");
    return MOE_OK;
}

extern "C" moe_status moe_debug_project(moe_ctx *ctx, const void *blob, int32_t part,
                                        const int8_t *q_in, const float *s_in, int32_t T,
                                        float *y, void *stream)
{
    if (!ctx || !blob || !q_in || !s_in || !y)
        return fail(MOE_E_INVAL, "NULL argument");
    if (ctx->d.wfmt != MOE_WFMT_INT4)
        return fail(MOE_E_UNSUPPORTED, "raw projection covers int4 blobs");
    if (part < 0 || part > 2)
        return fail(MOE_E_INVAL, "part=%d must be 0 (gate), 1 (up) or 2 (down)", part);
    if (T < 0 || T > ctx->max_tokens)
        return fail(MOE_E_INVAL, "T=%d out of range", T);
    if (T == 0)
        return MOE_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const moe_layer_desc &d = ctx->d;
    const int K = (part == 2) ? d.ffn : d.hidden;
    const int N = (part == 2) ? d.hidden : d.ffn;
    hipError_t e;
    ProjArgs a{};
    a.ex.ptrs = nullptr;
    a.ex.shared = blob;                // expert id 0 == E: the blob itself
    a.ex.E = 0;
    a.rt.active = ctx->zero1;
    a.rt.n_active = ctx->one1;
    a.rt.cnt = ctx->dbg_cnt;           // T rows, written below
    a.rt.list = ctx->ident;
    a.rt.list_stride = 0;
    a.rt.S = 1;
    a.q = q_in;
    a.s = s_in;
    a.in_by_token = 1;
    a.K = K;
    a.group_shift = (d.group == 64) ? 1 : 0;
    if (part == 2) {
        a.w_off = ctx->L.dn_w;
        a.s_off = ctx->L.dn_s;
        a.tile_w = ctx->L.dn_tile_w;
        a.tile_s = ctx->L.dn_tile_s;
        a.tile_base = 0;
        a.pair_stride = 2;
        a.j_stride = 1;
    } else {
        a.w_off = ctx->L.gu_w;
        a.s_off = ctx->L.gu_s;
        a.tile_w = ctx->L.gu_tile_w;
        a.tile_s = ctx->L.gu_tile_s;
        a.tile_base = part;            // gate tiles are even, up tiles odd
        a.pair_stride = 4;
        a.j_stride = 2;
    }
    a.out = y;
    a.ldo = N;
    if ((e = launch_set_i32(ctx->dbg_cnt, T, st)) != hipSuccess)
        return hip_fail(e, "count launch");
    if (use_mfma(ctx, T)) {
        if ((e = launch_mfma_tiles_single(ctx, T, st)) != hipSuccess)
            return hip_fail(e, "tile list launch");
        if ((e = launch_proj_mfma(a, ctx, T, N, st)) != hipSuccess)
            return hip_fail(e, "projection launch");
        return MOE_OK;
    }
    if ((e = launch_proj_gemv(a, 1, N / 32, mg_for(T), nullptr, st)) != hipSuccess)
        return hip_fail(e, "projection launch");
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// pinned host memory
// ---------------------------------------------------------------------------
extern "C" moe_status moe_host_alloc_pinned(size_t bytes, void **out)
{
    if (!out || bytes == 0)
        return fail(MOE_E_INVAL, "bad arguments");
    hipError_t e = hipHostMalloc(out, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
        *out = nullptr;
        return fail(MOE_E_NOMEM, "hipHostMalloc(%zu): %s", bytes, hipGetErrorString(e));
    }
    return MOE_OK;
}

extern "C" moe_status moe_host_free_pinned(void *p)
{
    if (!p)
        return MOE_OK;
    hipError_t e = hipHostFree(p);
    if (e != hipSuccess)
        return hip_fail(e, "hipHostFree");
    return MOE_OK;
}
