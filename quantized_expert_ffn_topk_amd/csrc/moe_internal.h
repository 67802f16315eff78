// moe_internal.h -- private declarations shared by the host runtime and the
// gfx950 kernels of the quantised MoE layer.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// Blob layout (this library's own format).
//
// An expert blob holds two weight sections, each split into tiles of 16 output
// rows.  A tile stores, for every chunk of 32 inputs kc and every row r of the
// tile, 16 bytes: [tile][kc][r][16 B].  So one 64-lane load of 16 B per lane
// covers 4 consecutive chunks of all 16 rows as 1 KiB of contiguous memory.
//   INT4 : byte j of a chunk holds input kc*32+j in its low nibble and input
//          kc*32+16+j in its high nibble, as 4-bit two's complement.  Masking
//          a nibble into the top of its byte gives the signed byte 16*q, so
//          byte dot products need no offset correction.
//   MXFP4: byte j holds input kc*32+2j (low nibble) and kc*32+2j+1 (high
//          nibble) as E2M1 codes.
// Scales follow each section's weights as [tile][group][r]: fp16 bits per
// group of `group` inputs (INT4) or one E8M0 byte per chunk (MXFP4).
//   gate/up section: 2F rows as F/8 tiles; tile 2b = gate rows [16b,16b+16),
//                    tile 2b+1 = up rows [16b,16b+16); K = H.
//   down section   : H rows as H/16 tiles; K = F.
// ---------------------------------------------------------------------------
struct BlobLayout {
    size_t gu_w, gu_s, dn_w, dn_s, total;
    size_t gu_tile_w, gu_tile_s, dn_tile_w, dn_tile_s;   // bytes per tile
};

inline BlobLayout blob_layout(int H, int F, int group, int wfmt)
{
    BlobLayout L;
    L.gu_tile_w = (size_t)H * 8;          // 16 rows * H/2 bytes
    L.dn_tile_w = (size_t)F * 8;
    if (wfmt == MOE_WFMT_MXFP4) {
        L.gu_tile_s = (size_t)(H / 32) * 16;
        L.dn_tile_s = (size_t)(F / 32) * 16;
    } else {
        L.gu_tile_s = (size_t)(H / group) * 16 * 2;
        L.dn_tile_s = (size_t)(F / group) * 16 * 2;
    }
    size_t gu_tiles = (size_t)F / 8, dn_tiles = (size_t)H / 16;
    L.gu_w = 0;
    L.gu_s = L.gu_w + gu_tiles * L.gu_tile_w;
    L.dn_w = L.gu_s + gu_tiles * L.gu_tile_s;
    L.dn_s = L.dn_w + dn_tiles * L.dn_tile_w;
    L.total = L.dn_s + dn_tiles * L.dn_tile_s;
    return L;
}

// ---------------------------------------------------------------------------
// Kernel argument blocks.
// ---------------------------------------------------------------------------
// Which experts run and on which rows ("slots").  A slot is token t, rank i:
// s = t*S + i with S = top_k + n_shared; rank top_k is the shared expert.
struct Routing {
    const int32_t *active;     // [n_experts + n_shared] expert ids with rows (E = shared)
    const int32_t *n_active;   // device scalar
    const int32_t *cnt;        // [E+1] rows per expert
    const int32_t *list;       // [E+1][list_stride] slots, token order
    int list_stride;
    int S;                     // slots per token
};

struct Experts {
    const void *const *ptrs;   // [E] device blob pointers
    const void *shared;        // blob of expert id E
    int E;
};

struct ProjArgs {
    Experts ex;
    Routing rt;
    // activation rows (int8 codes, fp32 scale)
    const int8_t *q;
    const float *s;
    int in_by_token;           // 1: input row = slot / S, 0: input row = slot
    int K;
    int group_shift;           // log2(group / 32)
    // weights: section offsets and tile selection
    size_t w_off, s_off, tile_w, tile_s;
    int tile_base, pair_stride, j_stride;
    // output rows: out[slot * ldo + 32*pair + 16*j + r]
    float *out;
    int ldo;
    // 1: the layer's expert blobs fit the last-level cache, so the GEMV reads
    // them with plain loads and they stay there between calls; 0: they are
    // streamed with the non-temporal hint
    int cached;
};

// Fused tails of the one-token GEMV path: requantisation of the SwiGLU rows
// (gate/up) and the combine (down); ctr is a zeroed device counter array.
struct TailArgs {
    int8_t *qh;
    float *sh;
    int F;
    const int32_t *idx;
    const float *w;
    int T, k, E, n_shared, H, out_dtype;
    void *out;
    uint32_t *ctr;
};

// One-token expert FFN (kernels_bs1.hip): slot i < k is rank i of the token,
// slot k the shared expert.
struct Bs1Args {
    Experts ex;
    const void *const *sel;    // [k] blob of each rank (NULL: out of range), or
                               // NULL to look the blobs up through idx and ex.ptrs
    const int32_t *idx;        // [k] expert of each rank
    const float *w;            // [k] gate weights
    int k, n_shared;
    const int8_t *xq;          // [H] token codes
    const float *sa;           // token scale
    int H, F, group_shift;
    size_t gu_w, gu_s, gu_tile_w, gu_tile_s, dn_w, dn_s, dn_tile_w, dn_tile_s;
    float *h;                  // [S][F] SwiGLU rows
    int8_t *qh;                // [S][F] their codes and scales (written by output block 0)
    float *sh;
    float *Y;                  // [S][H] per-slot projections
    void *out;
    int out_dtype;
};

// Few-token routing in one launch (kernels_router.hip).
enum { RS_ROUTER = 1, RS_QUANT = 2, RS_LISTS = 4, RS_SEL = 8 };
constexpr int RS_MAXT = 16;

struct RouteSmallArgs {
    const uint16_t *x;
    int T, H;
    const float *Wr, *bias;
    int E, k;
    float r;
    double *logits;
    int32_t *idx;
    float *w;
    int flags;
    int8_t *xq;
    float *sa;
    int32_t *cnt, *list;
    int list_stride;
    int32_t *active, *n_active;
    int n_shared;
    uint32_t *done;
    // RS_SEL (one token, without the router): sel[i] = ptrs[idx[i]] for the k
    // ranks (NULL for an id out of range), so the expert kernels find their
    // blobs with one load instead of two dependent ones
    const void *const *ptrs;
    const void **sel;
};

// ---------------------------------------------------------------------------
// Kernel timing.  While a profiled launch is enqueued, prof_slot() holds its
// start/stop events and launch() takes the kernel's own begin and end
// timestamps from its dispatch (hipExtLaunchKernelGGL), so the measured time
// is the kernel's, not that of the stream markers around it.
// ---------------------------------------------------------------------------
struct ProfSlot {
    hipEvent_t start = nullptr, stop = nullptr;
    bool used = false;
};
ProfSlot &prof_slot();

template <typename K, typename... Args>
inline void launch(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, Args... args)
{
    ProfSlot &p = prof_slot();
    if (p.start) {
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, p.start, p.stop, 0, args...);
        p.used = true;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, args...);
    }
}

// ---------------------------------------------------------------------------
// Launchers (kernels_*.hip).  All enqueue on `st` and return hipGetLastError.
// ---------------------------------------------------------------------------
hipError_t launch_quant_tokens(const uint16_t *x, int T, int H, int8_t *q, float *s,
                               hipStream_t st);
// K parts of the router logits for T tokens (1 or 2; with 2 the logits
// buffer holds 2*T*E partials until the top-k launch sums them).
int router_ksplit(int T, int H, int E);
hipError_t launch_router_logits(const uint16_t *x, int T, int H, const float *Wr, int E,
                                double *logits, hipStream_t st);
// With xq/sa set, the launch also quantises the T token rows of x (H <= 8192)
// into xq/sa as launch_quant_tokens does.
hipError_t launch_topk(double *logits, const float *bias, int T, int E, int k, float r,
                       int32_t *idx, float *w, hipStream_t st, const uint16_t *x = nullptr,
                       int H = 0, int8_t *xq = nullptr, float *sa = nullptr, int kparts = 1);
hipError_t launch_permute(const int32_t *idx, int T, int k, int E, int n_shared,
                          int32_t *cnt, int32_t *list, int list_stride, int32_t *active,
                          int32_t *n_active, uint32_t *done_counter, hipStream_t st);
hipError_t launch_gateup_gemv(const ProjArgs &a, int max_active, int F, int mg,
                              float *h, int ldh, const TailArgs *tail, hipStream_t st);
hipError_t launch_proj_gemv(const ProjArgs &a, int max_active, int n_pairs, int mg,
                            const TailArgs *tail, hipStream_t st);
hipError_t launch_route_small(const RouteSmallArgs &a, hipStream_t st);
hipError_t launch_requant(const float *h, int rows, int F, int8_t *q, float *s,
                          hipStream_t st);
hipError_t launch_combine(const float *Y, const int32_t *idx, const float *w, int T,
                          int k, int E, int n_shared, int H, void *out, int out_dtype,
                          hipStream_t st);
bool bs1_supported(int H, int F, int k, int n_shared);
hipError_t launch_gateup_bs1(const Bs1Args &a, int slots, hipStream_t st);
hipError_t launch_router_bs1(const RouteSmallArgs &a, hipStream_t st);
hipError_t launch_topk_bs1(const double *logits, const float *bias, int E, float r,
                           const void *const *ptrs,
                           int32_t *idx_out, float *w_out, const void **sel, const Bs1Args &a,
                           hipStream_t st);
hipError_t launch_down_bs1(const Bs1Args &a, hipStream_t st);
// table[set_idx] = ptr and, when clear_idx >= 0, table[clear_idx] = NULL
// (one thread; the pointers travel as kernel arguments).
hipError_t launch_table_update(const void **table, int set_idx, const void *ptr, int clear_idx,
                               hipStream_t st);

}  // namespace moe
