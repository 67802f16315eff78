// host_common.h -- host-side state shared by the C ABI implementation files.
#pragma once

#include <hip/hip_runtime.h>

#include <vector>

#include "moe_internal.h"

// Context: descriptor, kernel path and the workspace of one layer shape.
struct moe_ctx {
    int device = 0;
    moe_layer_desc d{};
    int max_tokens = 0;
    int path = MOE_PATH_AUTO;
    moe::BlobLayout L{};
    int S = 0;                     // slots per token (top_k + n_shared)
    std::vector<void *> allocs;
    // token quantisation
    int8_t *xq = nullptr;
    float *sa = nullptr;
    // router
    double *logits = nullptr;
    int32_t *idx = nullptr;
    float *gw = nullptr;
    // routing lists
    int32_t *cnt = nullptr, *list = nullptr, *active = nullptr, *n_active = nullptr;
    uint32_t *done = nullptr;
    uint32_t *ctr_gu = nullptr, *ctr_dn = nullptr;   // fused-tail counters
    // expert FFN intermediates, one row per slot
    float *h = nullptr;
    int8_t *qh = nullptr;
    float *sh = nullptr;
    float *Y = nullptr;
    const void **sel = nullptr;   // one-token path: blob of each rank
    // MFMA path: tile work list
    int32_t *tiles = nullptr, *n_tiles = nullptr;
    int max_tiles = 0;
    // MXFP4 path: bf16 activations of h; activation rows split into E4M3
    // hi/lo parts [rows][K] and their E8M0 scales [rows][K/32]
    uint16_t *hb = nullptr;
    uint8_t *mx_hi = nullptr, *mx_lo = nullptr, *mx_ehi = nullptr, *mx_elo = nullptr;
    // small device constants for single-blob projections
    int32_t *zero1 = nullptr, *one1 = nullptr, *dbg_cnt = nullptr, *ident = nullptr;
    int last_T = 0;
    // kernel timing: per kind a ring of PROF_RING (start, stop) event pairs;
    // launches [prof_tail, prof_head) are recorded and not yet added up
    static constexpr int PROF_RING = 256;
    bool prof_on = false;
    std::vector<hipEvent_t> prof_ev;   // [MOE_PROF_N][PROF_RING][2]
    int64_t prof_head[MOE_PROF_N] = {}, prof_tail[MOE_PROF_N] = {};
    hipError_t prof_err = hipSuccess;
    double prof_ms[MOE_PROF_N] = {};
    int64_t prof_cnt[MOE_PROF_N] = {};
};

namespace moe {

// Workspace buffers of a context.  ws_plan() calls f(&member, bytes, kind)
// once per buffer for c->d, c->max_tokens and c->S (kind WS_COUNTER: must be
// zero before the first call, and every kernel that uses it leaves it at zero
// again; WS_DEBUG: used by moe_debug_project only, set up at creation).  It
// stops at the first non-OK status f returns.
enum { WS_DATA = 0, WS_COUNTER = 1, WS_DEBUG = 2 };
size_t mfma_max_tiles(int T, int E, int n_shared, int S);
size_t mx_max_tiles(int T, int E, int n_shared, int S);

template <class Fn>
moe_status ws_plan(moe_ctx *c, Fn &&f)
{
    const moe_layer_desc &d = c->d;
    const size_t T = (size_t)c->max_tokens, H = d.hidden, F = d.ffn, E = d.n_experts;
    const size_t k = d.top_k, S = c->S;
    c->max_tiles = (int)(d.wfmt == MOE_WFMT_MXFP4
                             ? mx_max_tiles((int)T, (int)E, d.n_shared, (int)S)
                             : mfma_max_tiles((int)T, (int)E, d.n_shared, (int)S));
    moe_status st = MOE_OK;
#define WS(member, count, kind)                                                     \
    do {                                                                            \
        if ((st = f(reinterpret_cast<void **>(&c->member),                          \
                    (size_t)(count) * sizeof(*c->member), (kind))) != MOE_OK)       \
            return st;                                                              \
    } while (0)
    WS(done, 4, WS_COUNTER);
    WS(ctr_gu, E + 1, WS_COUNTER);
    WS(ctr_dn, H / 32, WS_COUNTER);
    WS(xq, T * H, WS_DATA);
    WS(sa, T, WS_DATA);
    WS(logits, 2 * T * E, WS_DATA);        // two K parts for few tokens
    WS(idx, T * k, WS_DATA);
    WS(gw, T * k, WS_DATA);
    WS(cnt, E + 1, WS_DATA);
    WS(list, (E + 1) * T, WS_DATA);
    WS(active, E + 1, WS_DATA);
    WS(n_active, 1, WS_DATA);
    WS(h, T * S * F, WS_DATA);
    WS(qh, T * S * F, WS_DATA);
    WS(sh, T * S, WS_DATA);
    WS(Y, T * S * H, WS_DATA);
    WS(sel, k, WS_DATA);
    WS(tiles, (size_t)c->max_tiles * 2, WS_DATA);
    WS(n_tiles, 4, WS_DATA);
    if (d.wfmt == MOE_WFMT_MXFP4) {
        // split buffers sized for the larger of the two uses (tokens x H, slots x F)
        const size_t split = (T * H > T * S * F) ? T * H : T * S * F;
        WS(hb, T * S * F, WS_DATA);
        WS(mx_hi, split, WS_DATA);
        WS(mx_lo, split, WS_DATA);
        WS(mx_ehi, split / 32, WS_DATA);
        WS(mx_elo, split / 32, WS_DATA);
    }
    WS(ident, T, WS_DEBUG);
    WS(zero1, 1, WS_DEBUG);
    WS(one1, 1, WS_DEBUG);
    WS(dbg_cnt, 1, WS_DEBUG);
#undef WS
    return st;
}

// The hot part of moe_layer_forward on a prepared context (arguments already
// checked by check_call): router, optional cache staging, expert FFNs.
moe_status layer_forward_enqueue(moe_ctx *ctx, const void *x, int32_t T,
                                 const moe_layer_weights *w, moe_cache *cache, int32_t layer,
                                 int32_t *idx_out, float *gate_w_out, void *out,
                                 hipStream_t st);

moe_status fail(moe_status st, const char *fmt, ...);
moe_status hip_fail(hipError_t e, const char *what);
moe_status validate_desc(const moe_layer_desc *d);
moe_status check_device(int device);

// Kernel timing helpers: prof_begin/prof_end bracket one launch of kind `k`
// with the next event pair of that kind's ring; nothing waits for them until
// the ring is full or the caller reads the totals (moe_ctx_profile_read), so
// profiled calls run back to back as unprofiled ones do.  prof_collect
// reports an error met while draining a full ring.
void prof_begin(moe_ctx *c, int k, hipStream_t st);
void prof_end(moe_ctx *c, int k, hipStream_t st);
moe_status prof_collect(moe_ctx *c);

// kernel path selection
bool use_mfma(const moe_ctx *c, int T);

// MFMA grouped GEMM path (kernels_gemm.hip)
hipError_t launch_mfma_tiles(moe_ctx *c, int T, hipStream_t st);
hipError_t launch_mfma_tiles_single(moe_ctx *c, int T, hipStream_t st);
// (expert, first row) tiles of mt rows from the routing counts
hipError_t launch_row_tiles(moe_ctx *c, int mt, hipStream_t st);
hipError_t launch_gateup_mfma(const ProjArgs &a, const moe_ctx *c, int T, int F, float *h, int ldh,
                              hipStream_t st);
hipError_t launch_proj_mfma(const ProjArgs &a, const moe_ctx *c, int T, int n_rows,
                            hipStream_t st);

// MXFP4 path (kernels_mx.hip)
moe_status mx_ffn_enqueue(moe_ctx *c, const void *x, int T, const moe_layer_weights *w,
                          const void *const *expert_ptrs, const int32_t *idx, const float *gw,
                          void *out, hipStream_t st);

// small helpers (kernels_router.hip)
hipError_t launch_set_i32(int32_t *p, int32_t v, hipStream_t st);

// cache (cache.cpp): the checks of a moe_layer_forward call with a cache
// (backend, layer in range, shapes, id buffer), run before anything is enqueued
moe_status cache_check_for_layer(const moe_cache *cache, const moe_layer_desc &d, int layer,
                                 int T);
// DEMAND stage of the routed experts of `layer` for the
// T*k device ids in idx; returns the device pointer table for the layer.
moe_status cache_demand_for_layer(moe_cache *cache, const moe_layer_desc &d, int layer,
                                  const int32_t *idx_dev, int T, hipStream_t compute,
                                  const void *const **table);

}  // namespace moe
