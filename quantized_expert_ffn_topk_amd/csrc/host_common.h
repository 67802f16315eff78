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
    double *cs = nullptr;         // one-token path: biased scores and scores [2E]
    // MFMA path: tile work list
    int32_t *tiles = nullptr, *n_tiles = nullptr;
    int max_tiles = 0;
    // MXFP4 path: bf16 activations of h
    uint16_t *hb = nullptr;
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
size_t mfma_max_tiles(int T, int E, int n_shared);

// MXFP4 path (kernels_mx.hip)
size_t mx_max_tiles(int T, int E, int n_shared, int S);
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
