// kernels_bs1.hip -- expert FFN for one token (batch-1 decode) on gfx950.
//
// With one token every routed expert and the shared expert has exactly one
// row, so slot i is rank i (i = top_k: shared expert) and the kernels read
// the expert of a slot straight from the top-k output: no routing lists.
//
// Both kernels stream the expert weights once.  A wave owns a 16-row tile of
// an expert (blob layout [tile][kc][r][16 B]); lane l owns row l&15 and the
// chunks kc = 4j + (l>>4), so the 64 lanes of one 16-byte load read 1 KiB of
// contiguous blob.  Each int32 group dot (v_dot4_i32_i8 on nibbles masked
// into the top of their bytes, see kernels_gemv.hip) is scaled in fp64 and
// summed; those sums are exact, so the split over lanes does not change the
// result.  Integer-dot scheme: Colibri guide, table "Points techniques cles".
//
//   gateup_bs1_kernel : block (slot, b) = the gate tile 2b and the up tile
//                       2b+1 over all of K = hidden, K split over 2 or 4
//                       waves per tile; SwiGLU of the 16 rows.
//   down_bs1_kernel   : block = 16 or 32 output rows, one wave per slot.  Each
//                       wave requantises its slot's SwiGLU row (same rule as
//                       the token quantisation) into LDS, projects the 16-row
//                       tiles, and the block then combines
//                       the slots of its outputs: shared expert first, then
//                       rank order, in fp64, rounded once.  No cross-block
//                       hand-off inside a kernel.
//   down_bs1h_kernel  : the same over half tiles (8 output rows), F = 2048:
//                       NH half tiles per block so that the grid covers the
//                       chip's compute units evenly (H/(8 NH) blocks).
//   topk_bs1h_kernel  : the top-k launch with the shared expert's gate/up
//                       over half tile pairs (8 gate + 8 up rows per block),
//                       twice as many blocks as tile pairs.
#include "device_common.h"
#include "host_common.h"
#include "topk_common.h"

namespace moe {

// 16 bytes read as a global-memory load (a generic one becomes a flat load,
// which also counts against the LDS wait counter).
typedef unsigned int gu32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 gload16(const uint4 *p)
{
    const gu32x4 v = *(const __attribute__((address_space(1))) gu32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// One batch of U 16-byte weight loads and their fp16 scales.
template <int U>
__device__ __forceinline__ void bs1_load(const uint4 *__restrict__ wp,
                                         const uint16_t *__restrict__ sp, int sstride, int j0,
                                         uint4 (&wv)[U], uint16_t (&sv)[U])
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        wv[u] = load_stream16(wp + (size_t)64 * (j0 + u));
        sv[u] = load_stream2(sp + (size_t)sstride * (j0 + u));
    }
}

// Adds the exact group sums of one batch: chunk kc = 4(j0+u) + c4 of the
// lane's row against the activation codes in LDS.
template <int U>
__device__ __forceinline__ double bs1_dot(const uint4 (&wv)[U], const uint16_t (&sv)[U], int j0,
                                          int c4, const int8_t *__restrict__ lq, double p)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = 4 * (j0 + u) + c4;
        const int4 *qa = reinterpret_cast<const int4 *>(lq + c * 32);
        const int4 a0 = qa[0], a1 = qa[1];
        const uint32_t wd[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
        int acc = 0;
        acc = sdot4((int)((wd[0] << 4) & 0xf0f0f0f0u), a0.x, acc);
        acc = sdot4((int)((wd[1] << 4) & 0xf0f0f0f0u), a0.y, acc);
        acc = sdot4((int)((wd[2] << 4) & 0xf0f0f0f0u), a0.z, acc);
        acc = sdot4((int)((wd[3] << 4) & 0xf0f0f0f0u), a0.w, acc);
        acc = sdot4((int)(wd[0] & 0xf0f0f0f0u), a1.x, acc);
        acc = sdot4((int)(wd[1] & 0xf0f0f0f0u), a1.y, acc);
        acc = sdot4((int)(wd[2] & 0xf0f0f0f0u), a1.z, acc);
        acc = sdot4((int)(wd[3] & 0xf0f0f0f0u), a1.w, acc);
        // 16 x the group dot; S/16 is exact
        p = fma((double)acc, (double)f16_to_f32(sv[u]) * 0.0625, p);
    }
    return p;
}

// Blob of slot ai, or NULL when the slot's expert id is out of range (such a
// slot contributes nothing, as in the combine).  With the router's blob
// selection this is one load; otherwise the id, then the pointer table.
__device__ __forceinline__ const uint8_t *bs1_slot_blob(const Bs1Args &a, int ai)
{
    if (ai >= a.k)
        return reinterpret_cast<const uint8_t *>(a.ex.shared);
    if (a.sel)
        return reinterpret_cast<const uint8_t *>(a.sel[ai]);
    const int e = a.idx[ai];
    return (e >= 0 && e < a.ex.E) ? reinterpret_cast<const uint8_t *>(a.ex.ptrs[e]) : nullptr;
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU: h[slot, 16b + r] = fp32(G/(1+exp(-G)) * U) with
// G, U = exact sum * token scale (fp64).
// ---------------------------------------------------------------------------
// NP tile pairs per block of 128*NP*KS threads: pair p = b0 + p' has its gate
// tile 2b and up tile 2b+1, each split over KS waves by K (wave w: pair w /
// (2 KS), tile half (w / KS) % 2, K segment w % KS).  The KS partial sums of a
// row are exact, so adding them in any order gives the exact sum.
template <int U, int NP, int KS>
__device__ __forceinline__ void gateup_pairs(const Bs1Args &a, int ai, int b0, unsigned char *smem)
{
    constexpr int NT = 128 * NP * KS;
    constexpr int XS = (512 + NT - 1) / NT;          // H <= 8192: 512 x 16 B of codes
    __shared__ double sp[NP][2][KS][16];
    // the token codes are fetched while the blob pointer is looked up
    const uint4 *xsrc = reinterpret_cast<const uint4 *>(a.xq);
    const int nx = a.H >> 4;
    uint4 xs[XS];
#pragma unroll
    for (int i = 0; i < XS; ++i)                     // clamped: every load in bounds
        xs[i] = xsrc[min((int)threadIdx.x + NT * i, nx - 1)];
    const uint8_t *blob = bs1_slot_blob(a, ai);
    if (!blob)
        return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int seg = wave % KS, half = (wave / KS) & 1, pair = wave / (2 * KS), b = b0 + pair;
    const int r = lane & 15, c4 = lane >> 4, gs = a.group_shift;
    const int tile = 2 * b + half;
    const uint4 *wp = reinterpret_cast<const uint4 *>(blob + a.gu_w + (size_t)tile * a.gu_tile_w) + lane;
    const uint16_t *sp_ = reinterpret_cast<const uint16_t *>(blob + a.gu_s + (size_t)tile * a.gu_tile_s) +
                          (((c4 >> gs) << 4) + r);
    const int sstride = 64 >> gs;
    const int nseg = (a.H >> 7) / KS, j_begin = seg * nseg, j_end = j_begin + nseg;

    uint4 wv[U];
    uint16_t sv[U];
    bs1_load<U>(wp, sp_, sstride, j_begin, wv, sv);
    {
        uint4 *dst = reinterpret_cast<uint4 *>(smem);
#pragma unroll
        for (int i = 0; i < XS; ++i)
            if ((int)threadIdx.x + NT * i < nx)
                dst[threadIdx.x + NT * i] = xs[i];
    }
    __syncthreads();
    const int8_t *lq = reinterpret_cast<const int8_t *>(smem);
    double p = bs1_dot<U>(wv, sv, j_begin, c4, lq, 0.0);
    for (int j0 = j_begin + U; j0 < j_end; j0 += U) {
        bs1_load<U>(wp, sp_, sstride, j0, wv, sv);
        p = bs1_dot<U>(wv, sv, j0, c4, lq, p);
    }
    p += xor_lane_d<16>(p);
    p += xor_lane_d<32>(p);
    if (lane < 16)
        sp[pair][half][seg][lane] = p;
    __syncthreads();
    if (half == 0 && seg == 0 && lane < 16) {
        double g = 0.0, u = 0.0;
#pragma unroll
        for (int q = 0; q < KS; ++q) {
            g += sp[pair][0][q][lane];
            u += sp[pair][1][q][lane];
        }
        const double sa = (double)a.sa[0];
        const double G = g * sa;
        const double Uv = u * sa;
        const double silu = G / (1.0 + exp(-G));
        a.h[(size_t)ai * a.F + 16 * b + lane] = (float)(silu * Uv);
    }
}

// Block (slot, b): the tile pair b of the slot's expert, K split over KS waves.
template <int U, int KS>
__global__ __launch_bounds__(128 * KS) void gateup_bs1_kernel(Bs1Args a)
{
    extern __shared__ __align__(16) unsigned char smem[];   // H activation codes
    gateup_pairs<U, 1, KS>(a, blockIdx.x, blockIdx.y, smem);
}

// Sigmoid score s and biased score c (NaN -> -inf) of expert e from its fp64
// logit, as the many-token top-k computes them.
__device__ __forceinline__ double bs1_scores(const double *__restrict__ logits,
                                             const float *__restrict__ bias, int e, double &s)
{
    s = 1.0 / (1.0 + exp(-logits[e]));
    const double cv = s + (double)bias[e];
    return (cv != cv) ? -INFINITY : cv;
}

// ---------------------------------------------------------------------------
// Second launch of the one-token router (after router_bs1_kernel): block 0
// turns the logits into scores s and biased scores c (one expert per
// thread), selects the top k, writes ids, weights and the ranks' blobs.  The other blocks run the shared
// expert's gate/up meanwhile (it needs no routing): block 1 + q takes the tile
// pair q with K split over 2 waves per tile, so the routed gate/up launch that
// follows is k slots wide.
// ---------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(256) void topk_bs1_kernel(const double *__restrict__ logits,
                                                       const float *__restrict__ bias, int E,
                                                       float r, const void *const *ptrs,
                                                       int32_t *idx_out, float *w_out,
                                                       const void **sel, Bs1Args a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    if (blockIdx.x > 0) {
        gateup_pairs<U, 1, 2>(a, a.k, blockIdx.x - 1, smem);
        return;
    }
    __shared__ double s_s[256], cand_c[64], sel_s[16];
    __shared__ int cand_i[64], s_idx[16];
    __shared__ const void *s_ptr[256];
    const int tid = threadIdx.x;
    double c = -INFINITY;
    int ci = INT_MAX;
    if (tid < E) {
        // the blob pointer's load goes out with the score's loads and is
        // stored after them, so the two share one round trip
        const void *pt = ptrs ? ptrs[tid] : nullptr;
        double sv;
        c = bs1_scores(logits, bias, tid, sv);
        s_s[tid] = sv;
        ci = tid;
        if (ptrs)
            s_ptr[tid] = pt;
    }
    topk_select_256(c, ci, s_s, a.k, r, idx_out, w_out, s_idx, cand_c, cand_i, sel_s);
    if (ptrs && tid < a.k)
        sel[tid] = s_ptr[s_idx[tid]];
}

// Gate/up + SwiGLU of half a tile pair (8 gate rows and the matching 8 up
// rows) for slot ai: block of 8 waves, wave w takes the gate (w < 4) or up
// tile, K segment w % 4.  Lane l owns row l&7 and chunks kc = 8j + (l>>3) of
// the segment, NL = H/1024 loads per lane.
template <int NL>
__device__ __forceinline__ void gateup_half(const Bs1Args &a, int ai, int q, unsigned char *smem)
{
    __shared__ double sp[2][4][8];
    const uint4 *xsrc = reinterpret_cast<const uint4 *>(a.xq);
    const int nx = a.H >> 4;                         // <= 512
    const uint4 xs = xsrc[min((int)threadIdx.x, nx - 1)];
    const uint8_t *blob = bs1_slot_blob(a, ai);
    if (!blob)
        return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gu = wave >> 2, seg = wave & 3, pp = q >> 1, hf = q & 1;
    const int r = lane & 7, c8 = lane >> 3, gs = a.group_shift;
    const int tile = 2 * pp + gu;
    const int kc0 = seg * NL * 8;
    const uint4 *wp = reinterpret_cast<const uint4 *>(blob + a.gu_w + (size_t)tile * a.gu_tile_w) +
                      kc0 * 16 + 8 * hf + r + 16 * c8;
    const uint16_t *sp_ = reinterpret_cast<const uint16_t *>(blob + a.gu_s + (size_t)tile * a.gu_tile_s) +
                          ((kc0 >> gs) << 4) + ((c8 >> gs) << 4) + 8 * hf + r;
    uint4 wv[NL];
    uint16_t sv[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        wv[j] = gload16(wp + 128 * j);
        sv[j] = load_stream2(sp_ + (size_t)(128 >> gs) * j);
    }
    if ((int)threadIdx.x < nx)
        reinterpret_cast<uint4 *>(smem)[threadIdx.x] = xs;
    __syncthreads();
    const int8_t *lq = reinterpret_cast<const int8_t *>(smem);
    double p = 0.0;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int c = kc0 + 8 * j + c8;
        const int4 *qa = reinterpret_cast<const int4 *>(lq + c * 32);
        const int4 a0 = qa[0], a1 = qa[1];
        const uint32_t wd[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
        int acc = 0;
        acc = sdot4((int)((wd[0] << 4) & 0xf0f0f0f0u), a0.x, acc);
        acc = sdot4((int)((wd[1] << 4) & 0xf0f0f0f0u), a0.y, acc);
        acc = sdot4((int)((wd[2] << 4) & 0xf0f0f0f0u), a0.z, acc);
        acc = sdot4((int)((wd[3] << 4) & 0xf0f0f0f0u), a0.w, acc);
        acc = sdot4((int)(wd[0] & 0xf0f0f0f0u), a1.x, acc);
        acc = sdot4((int)(wd[1] & 0xf0f0f0f0u), a1.y, acc);
        acc = sdot4((int)(wd[2] & 0xf0f0f0f0u), a1.z, acc);
        acc = sdot4((int)(wd[3] & 0xf0f0f0f0u), a1.w, acc);
        p = fma((double)acc, (double)f16_to_f32(sv[j]) * 0.0625, p);
    }
    p += xor_lane_d<8>(p);
    p += xor_lane_d<16>(p);
    p += xor_lane_d<32>(p);
    if (lane < 8)
        sp[gu][seg][lane] = p;
    __syncthreads();
    if (wave == 0 && lane < 8) {
        double g = 0.0, u = 0.0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            g += sp[0][t][lane];
            u += sp[1][t][lane];
        }
        const double sa = (double)a.sa[0];
        const double G = g * sa;
        const double Uv = u * sa;
        const double silu = G / (1.0 + exp(-G));
        a.h[(size_t)ai * a.F + 16 * pp + 8 * hf + lane] = (float)(silu * Uv);
    }
}

template <int NL>
__global__ __launch_bounds__(512) void topk_bs1h_kernel(const double *__restrict__ logits,
                                                        const float *__restrict__ bias, int E,
                                                        float r, const void *const *ptrs,
                                                        int32_t *idx_out, float *w_out,
                                                        const void **sel, Bs1Args a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    if (blockIdx.x > 0) {
        gateup_half<NL>(a, a.k, blockIdx.x - 1, smem);
        return;
    }
    __shared__ double s_s[256], cand_c[64], sel_s[16];
    __shared__ int cand_i[64], s_idx[16];
    __shared__ const void *s_ptr[256];
    const int tid = threadIdx.x;
    if (tid >= 256) {
        // the selection runs on waves 0-3; the others pass its three barriers
        __syncthreads();
        __syncthreads();
        __syncthreads();
        return;
    }
    double c = -INFINITY;
    int ci = INT_MAX;
    if (tid < E) {
        // the blob pointer's load goes out with the score's loads and is
        // stored after them, so the two share one round trip
        const void *pt = ptrs ? ptrs[tid] : nullptr;
        double sv;
        c = bs1_scores(logits, bias, tid, sv);
        s_s[tid] = sv;
        ci = tid;
        if (ptrs)
            s_ptr[tid] = pt;
    }
    topk_select_256(c, ci, s_s, a.k, r, idx_out, w_out, s_idx, cand_c, cand_i, sel_s);
    if (ptrs && tid < a.k)
        sel[tid] = s_ptr[s_idx[tid]];
}

// ---------------------------------------------------------------------------
// Down projection + combine for the TPW 16-row tiles TPW*p, ... of every
// slot (output rows [16*TPW*p, 16*TPW*(p+1))).  F <= 2048.  Each wave codes its slot's
// SwiGLU row with the token quantisation rule (amax over the row, inv =
// 127/amax, s = amax/127, q = rint(h*inv) clamped to [-127, 127]) into LDS,
// then streams both tiles with two batches of U loads in flight.
// ---------------------------------------------------------------------------
template <int U>
__device__ __forceinline__ void bs1_load2(const uint4 *wp, const uint16_t *sp, size_t wstep,
                                          size_t sstep, int sstride, int j, int nj,
                                          uint4 (&wv)[U], uint16_t (&sv)[U])
{
    if (j < nj)
        bs1_load<U>(wp, sp, sstride, j, wv, sv);
    else
        bs1_load<U>(wp + wstep, sp + sstep, sstride, j - nj, wv, sv);
}

template <int U, int NW, bool DB, int TPW>
__global__ __launch_bounds__(64 * NW) void down_bs1_kernel(Bs1Args a)
{
    extern __shared__ __align__(16) unsigned char smem[];   // S rows of F codes
    __shared__ float sY[16][16 * TPW];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, c4 = lane >> 4, gs = a.group_shift;
    const int ai = wave, pr = blockIdx.x;
    const int F = a.F, nj = F >> 7;
    int8_t *lq = reinterpret_cast<int8_t *>(smem) + (size_t)ai * F;

    uint4 wa[U], wb[U];
    uint16_t sa[U], sb[U];
    const uint4 *wp = nullptr;
    const uint16_t *sp = nullptr;
    size_t wstep = 0, sstep = 0;
    const int sstride = 64 >> gs;
    float sc = 0.0f;
    // the SwiGLU row first: it depends on nothing and comes from L2, ahead of
    // the weights in the wave's load queue
    const float4 *hr = reinterpret_cast<const float4 *>(a.h + (size_t)ai * F);
    const int nv = F >> 8;                           // float4 per lane, <= 8
    float4 hv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < nv)
            hv[i] = hr[lane + 64 * i];
    const uint8_t *blob = bs1_slot_blob(a, ai);
    if (blob) {
        wp = reinterpret_cast<const uint4 *>(blob + a.dn_w + (size_t)(TPW * pr) * a.dn_tile_w) + lane;
        sp = reinterpret_cast<const uint16_t *>(blob + a.dn_s + (size_t)(TPW * pr) * a.dn_tile_s) +
             (((c4 >> gs) << 4) + r);
        wstep = a.dn_tile_w >> 4;
        sstep = a.dn_tile_s >> 1;
        bs1_load<U>(wp, sp, sstride, 0, wa, sa);
        if (DB && U < TPW * nj)
            bs1_load2<U>(wp, sp, wstep, sstep, sstride, U, nj, wb, sb);

        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nv)
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(hv[i].x), fabsf(hv[i].y)),
                                         fmaxf(fabsf(hv[i].z), fabsf(hv[i].w))));
        amax = wave_max(amax);
        float inv = 0.0f;
        if (amax > 0.0f) {
            inv = 127.0f / amax;
            sc = amax / 127.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < nv) {
                const float vv[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
                uint32_t packed = 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float q = fminf(fmaxf(rintf(vv[j] * inv), -127.0f), 127.0f);
                    packed |= ((uint32_t)(int)q & 0xffu) << (8 * j);
                }
                const int o = 4 * (lane + 64 * i);
                *reinterpret_cast<uint32_t *>(lq + o) = packed;
                if (pr == 0)
                    *reinterpret_cast<uint32_t *>(a.qh + (size_t)ai * F + o) = packed;
            }
        }
        if (pr == 0 && lane == 0)
            a.sh[ai] = sc;
        // only this wave reads its codes: wait for its LDS writes
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
    }
    if (blob) {
        // batches j0 = 0, U, 2U, ... over the wave's tiles (U divides nj, so no
        // batch straddles two tiles)
        const int nb = TPW * nj;
        double p = 0.0, p0 = 0.0;                  // p: the tile being summed
        if (DB) {
            // two batches in flight: compute one while the next loads
            for (int j0 = 0; j0 < nb; j0 += 2 * U) {
                if (j0 == nj) {
                    p0 = p;
                    p = 0.0;
                }
                p = bs1_dot<U>(wa, sa, j0 < nj ? j0 : j0 - nj, c4, lq, p);
                if (j0 + 2 * U < nb)
                    bs1_load2<U>(wp, sp, wstep, sstep, sstride, j0 + 2 * U, nj, wa, sa);
                const int j1 = j0 + U;
                if (j1 >= nb)
                    break;
                if (j1 == nj) {
                    p0 = p;
                    p = 0.0;
                }
                p = bs1_dot<U>(wb, sb, j1 < nj ? j1 : j1 - nj, c4, lq, p);
                if (j0 + 3 * U < nb)
                    bs1_load2<U>(wp, sp, wstep, sstep, sstride, j0 + 3 * U, nj, wb, sb);
            }
        } else {
            for (int j0 = 0; j0 < nb; j0 += U) {
                if (j0 == nj) {
                    p0 = p;
                    p = 0.0;
                }
                if (j0)
                    bs1_load2<U>(wp, sp, wstep, sstep, sstride, j0, nj, wa, sa);
                p = bs1_dot<U>(wa, sa, j0 < nj ? j0 : j0 - nj, c4, lq, p);
            }
        }
        double p1 = p;
        if (TPW == 1)
            p0 = p;
        p0 += xor_lane_d<16>(p0);
        p0 += xor_lane_d<32>(p0);
        if (TPW == 2) {
            p1 += xor_lane_d<16>(p1);
            p1 += xor_lane_d<32>(p1);
        }
        if (lane < 16) {
            float *yg = a.Y + (size_t)ai * a.H + 16 * TPW * pr;
            const float y0 = (float)(p0 * (double)sc);
            sY[ai][r] = y0;
            yg[r] = y0;
            if (TPW == 2) {
                const float y1 = (float)(p1 * (double)sc);
                sY[ai][16 + r] = y1;
                yg[16 + r] = y1;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < 16 * TPW) {
        double o = a.n_shared ? (double)sY[a.k][threadIdx.x] : 0.0;
        for (int i = 0; i < a.k; ++i) {
            const int ex = a.idx[i];
            if (ex >= 0 && ex < a.ex.E)
                o = fma((double)a.w[i], (double)sY[i][threadIdx.x], o);
        }
        const float f = (float)o;
        const size_t n = (size_t)16 * TPW * pr + threadIdx.x;
        if (a.out_dtype == MOE_DT_BF16)
            reinterpret_cast<uint16_t *>(a.out)[n] = f32_to_bf16(f);
        else
            reinterpret_cast<float *>(a.out)[n] = f;
    }
}

// Down projection + combine over half tiles (8 output rows): block pr takes
// the NH half tiles NH*pr, ..., NH*pr + NH - 1 of every slot (output rows
// [8*NH*pr, 8*NH*(pr+1))), one wave per slot.  Lane l owns row l&7 of the
// half tile and chunks kc = 8j + (l>>3), j < 8 (F = 2048): one 16-byte load
// per lane reads 8 chunks x 128 B of the blob.  A half tile is one batch of
// 8 loads; two batches are in flight.
template <int NH>
__device__ __forceinline__ void dnh_load(const uint8_t *blob, const Bs1Args &a, int hidx, int r,
                                         int c8, uint4 (&wv)[8], uint16_t (&sv)[8])
{
    const int t = hidx >> 1, hf = hidx & 1, gs = a.group_shift;
    const uint4 *wp = reinterpret_cast<const uint4 *>(blob + a.dn_w + (size_t)t * a.dn_tile_w) +
                      8 * hf + r + 16 * c8;
    const uint16_t *sp = reinterpret_cast<const uint16_t *>(blob + a.dn_s + (size_t)t * a.dn_tile_s) +
                         ((c8 >> gs) << 4) + 8 * hf + r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        wv[j] = load_stream16(wp + 128 * j);
        sv[j] = load_stream2(sp + (size_t)(128 >> gs) * j);
    }
}

__device__ __forceinline__ double dnh_dot(const uint4 (&wv)[8], const uint16_t (&sv)[8], int c8,
                                          const int8_t *__restrict__ lq)
{
    double p = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int c = 8 * j + c8;
        const int4 *qa = reinterpret_cast<const int4 *>(lq + c * 32);
        const int4 a0 = qa[0], a1 = qa[1];
        const uint32_t wd[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
        int acc = 0;
        acc = sdot4((int)((wd[0] << 4) & 0xf0f0f0f0u), a0.x, acc);
        acc = sdot4((int)((wd[1] << 4) & 0xf0f0f0f0u), a0.y, acc);
        acc = sdot4((int)((wd[2] << 4) & 0xf0f0f0f0u), a0.z, acc);
        acc = sdot4((int)((wd[3] << 4) & 0xf0f0f0f0u), a0.w, acc);
        acc = sdot4((int)(wd[0] & 0xf0f0f0f0u), a1.x, acc);
        acc = sdot4((int)(wd[1] & 0xf0f0f0f0u), a1.y, acc);
        acc = sdot4((int)(wd[2] & 0xf0f0f0f0u), a1.z, acc);
        acc = sdot4((int)(wd[3] & 0xf0f0f0f0u), a1.w, acc);
        p = fma((double)acc, (double)f16_to_f32(sv[j]) * 0.0625, p);
    }
    return p;
}

// The shared expert's part of the block for SQ: wave q (0-3) of the four
// after the k routed waves takes inputs [512q, 512q+512) of every half tile
// (loads j = 2q, 2q+1 of the 8), codes only that quarter of the SwiGLU row
// (amax still over the whole row) and leaves the quarter's exact sums in sP;
// the four are added in the combine (exact, so the order does not matter).
template <int NH>
__device__ __forceinline__ void down_shared_quarter(const Bs1Args &a, const uint8_t *blob, int q,
                                                    int pr, int lane, const float4 (&hv)[8],
                                                    int8_t *lq, double (*sP)[8 * NH],
                                                    float *s_sc)
{
    const int r = lane & 7, c8 = lane >> 3, gs = a.group_shift, ai = a.k;
    const int F = 2048;
    uint4 wv[NH][2];
    uint16_t sv[NH][2];
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        const int hidx = NH * pr + i, t = hidx >> 1, hf = hidx & 1;
        const uint4 *wp = reinterpret_cast<const uint4 *>(blob + a.dn_w + (size_t)t * a.dn_tile_w) +
                          8 * hf + r + 16 * c8;
        const uint16_t *sp = reinterpret_cast<const uint16_t *>(blob + a.dn_s + (size_t)t * a.dn_tile_s) +
                             ((c8 >> gs) << 4) + 8 * hf + r;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * q + jj;
            // plain loads: every step reads the shared expert again, so it
            // may stay in the last-level cache (0.3 us per step faster than
            // the non-temporal hint in an A/B run)
            wv[i][jj] = gload16(wp + 128 * j);
            sv[i][jj] = load_stream2(sp + (size_t)(128 >> gs) * j);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(hv[i].x), fabsf(hv[i].y)),
                                 fmaxf(fabsf(hv[i].z), fabsf(hv[i].w))));
    amax = wave_max(amax);
    float inv = 0.0f, sc = 0.0f;
    if (amax > 0.0f) {
        inv = 127.0f / amax;
        sc = amax / 127.0f;
    }
    // float4 i of the lane holds inputs 256 i + 4 lane ...: the quarter is i = 2q, 2q+1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if ((i >> 1) != q)
            continue;
        const float vv[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
        uint32_t packed = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float qv = fminf(fmaxf(rintf(vv[j] * inv), -127.0f), 127.0f);
            packed |= ((uint32_t)(int)qv & 0xffu) << (8 * j);
        }
        const int o = 4 * (lane + 64 * i);
        *reinterpret_cast<uint32_t *>(lq + o) = packed;
        if (pr == 0)
            *reinterpret_cast<uint32_t *>(a.qh + (size_t)ai * F + o) = packed;
    }
    if (lane == 0 && q == 0) {
        *s_sc = sc;
        if (pr == 0)
            a.sh[ai] = sc;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0): this wave's codes
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        double p = 0.0;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int c = 8 * (2 * q + jj) + c8;
            const int4 *qa = reinterpret_cast<const int4 *>(lq + c * 32);
            const int4 a0 = qa[0], a1 = qa[1];
            const uint32_t wd[4] = {wv[i][jj].x, wv[i][jj].y, wv[i][jj].z, wv[i][jj].w};
            int acc = 0;
            acc = sdot4((int)((wd[0] << 4) & 0xf0f0f0f0u), a0.x, acc);
            acc = sdot4((int)((wd[1] << 4) & 0xf0f0f0f0u), a0.y, acc);
            acc = sdot4((int)((wd[2] << 4) & 0xf0f0f0f0u), a0.z, acc);
            acc = sdot4((int)((wd[3] << 4) & 0xf0f0f0f0u), a0.w, acc);
            acc = sdot4((int)(wd[0] & 0xf0f0f0f0u), a1.x, acc);
            acc = sdot4((int)(wd[1] & 0xf0f0f0f0u), a1.y, acc);
            acc = sdot4((int)(wd[2] & 0xf0f0f0f0u), a1.z, acc);
            acc = sdot4((int)(wd[3] & 0xf0f0f0f0u), a1.w, acc);
            p = fma((double)acc, (double)f16_to_f32(sv[i][jj]) * 0.0625, p);
        }
        p += xor_lane_d<8>(p);
        p += xor_lane_d<16>(p);
        p += xor_lane_d<32>(p);
        if (lane < 8)
            sP[q][8 * i + r] = p;
    }
}

// SQ: k routed waves, then the shared expert over four K-quarter waves (k + 4
// waves: for k = 8 every SIMD holds two routed waves and one quarter wave,
// where one wave per slot puts three full waves on one SIMD).
template <int NH, bool SQ>
__global__ __launch_bounds__(64 * 12) void down_bs1h_kernel(Bs1Args a)
{
    extern __shared__ __align__(16) unsigned char smem[];   // S rows of F codes
    __shared__ float sY[9][8 * NH];
    __shared__ double sP[SQ ? 4 : 1][8 * NH];
    __shared__ float s_sc;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 7, c8 = lane >> 3;
    const bool shq = SQ && wave >= a.k;
    const int ai = shq ? a.k : wave, pr = blockIdx.x;
    const int F = 2048;
    int8_t *lq = reinterpret_cast<int8_t *>(smem) + (size_t)ai * F;

    float sc = 0.0f;
    // the combine's ids and weights: loaded here (every thread, so that no
    // wave waits for them before its own loads) and written to LDS before the
    // block's barrier
    __shared__ float s_w[16];
    __shared__ int s_e[16];
    const int cw = threadIdx.x < a.k ? threadIdx.x : 0;
    const int e_cw = a.idx[cw];
    const float w_cw = a.w[cw];
    const float4 *hr = reinterpret_cast<const float4 *>(a.h + (size_t)ai * F);
    float4 hv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        hv[i] = hr[lane + 64 * i];
    const uint8_t *blob = bs1_slot_blob(a, ai);
    if (shq)
        down_shared_quarter<NH>(a, blob, wave - a.k, pr, lane, hv, lq, sP, &s_sc);
    else if (blob) {
        uint4 wa[8], wb[8];
        uint16_t sa[8], sb[8];
        dnh_load<NH>(blob, a, NH * pr, r, c8, wa, sa);
        if (NH > 1)
            dnh_load<NH>(blob, a, NH * pr + 1, r, c8, wb, sb);

        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(hv[i].x), fabsf(hv[i].y)),
                                     fmaxf(fabsf(hv[i].z), fabsf(hv[i].w))));
        amax = wave_max(amax);
        float inv = 0.0f;
        if (amax > 0.0f) {
            inv = 127.0f / amax;
            sc = amax / 127.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float vv[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
            uint32_t packed = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float q = fminf(fmaxf(rintf(vv[j] * inv), -127.0f), 127.0f);
                packed |= ((uint32_t)(int)q & 0xffu) << (8 * j);
            }
            const int o = 4 * (lane + 64 * i);
            *reinterpret_cast<uint32_t *>(lq + o) = packed;
            if (pr == 0)
                *reinterpret_cast<uint32_t *>(a.qh + (size_t)ai * F + o) = packed;
        }
        if (pr == 0 && lane == 0)
            a.sh[ai] = sc;
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();

        double ps[NH];
#pragma unroll
        for (int i = 0; i < NH; i += 2) {
            ps[i] = dnh_dot(wa, sa, c8, lq);
            if (i + 2 < NH)
                dnh_load<NH>(blob, a, NH * pr + i + 2, r, c8, wa, sa);
            if (i + 1 < NH) {
                ps[i + 1] = dnh_dot(wb, sb, c8, lq);
                if (i + 3 < NH)
                    dnh_load<NH>(blob, a, NH * pr + i + 3, r, c8, wb, sb);
            }
        }
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            double p = ps[i];
            p += xor_lane_d<8>(p);
            p += xor_lane_d<16>(p);
            p += xor_lane_d<32>(p);
            if (lane < 8) {
                const float y = (float)(p * (double)sc);
                sY[ai][8 * i + r] = y;
                a.Y[(size_t)ai * a.H + 8 * NH * pr + 8 * i + r] = y;
            }
        }
    }
    if (threadIdx.x < a.k) {
        s_e[threadIdx.x] = e_cw;
        s_w[threadIdx.x] = w_cw;
    }
    __syncthreads();
    if (threadIdx.x < 8 * NH) {
        double o = 0.0;
        if (SQ) {
            // the quarter sums are exact, so is their sum: the shared row's y
            // is that of one wave over the whole row
            const double p = ((sP[0][threadIdx.x] + sP[1][threadIdx.x]) + sP[2][threadIdx.x]) +
                             sP[3][threadIdx.x];
            const float y = (float)(p * (double)s_sc);
            a.Y[(size_t)a.k * a.H + 8 * NH * pr + threadIdx.x] = y;
            o = (double)y;
        } else if (a.n_shared) {
            o = (double)sY[a.k][threadIdx.x];
        }
        for (int i = 0; i < a.k; ++i) {
            const int ex = s_e[i];
            if (ex >= 0 && ex < a.ex.E)
                o = fma((double)s_w[i], (double)sY[i][threadIdx.x], o);
        }
        const float f = (float)o;
        const size_t n = (size_t)8 * NH * pr + threadIdx.x;
        if (a.out_dtype == MOE_DT_BF16)
            reinterpret_cast<uint16_t *>(a.out)[n] = f32_to_bf16(f);
        else
            reinterpret_cast<float *>(a.out)[n] = f;
    }
}

// Loads per lane per batch: the largest of umax, ..., 4, 2 dividing nj = K/128
// (K is a multiple of 256, so nj is even).
static int bs1_u(int nj, int umax)
{
    static const int cand[] = {16, 12, 8, 6, 4, 2};
    for (int u : cand)
        if (u <= umax && nj % u == 0)
            return u;
    return 1;
}

bool bs1_supported(int H, int F, int k, int n_shared)
{
    return F <= 2048 && H <= 8192 && k + n_shared <= 16;
}

// slots: how many slots from 0 the launch covers (k when the shared expert
// already ran in the top-k launch, k + n_shared otherwise).
template <int KS>
static void gateup_bs1_u(const Bs1Args &a, dim3 grid, size_t lds, hipStream_t st)
{
    // where the wave's loads divide by 6, batches of 6 (hidden 6144: two per
    // wave): 0.3 us per decode step faster in an A/B run than the whole
    // 12-load segment in one batch, and than batches of 4; otherwise the
    // largest batch up to 16
    const int nj = (a.H >> 7) / KS;
    switch (bs1_u(nj, nj % 6 == 0 ? 6 : 16)) {
    case 6: launch(gateup_bs1_kernel<6, KS>, grid, 128 * KS, lds, st, a); break;
    case 16: launch(gateup_bs1_kernel<16, KS>, grid, 128 * KS, lds, st, a); break;
    case 12: launch(gateup_bs1_kernel<12, KS>, grid, 128 * KS, lds, st, a); break;
    case 8: launch(gateup_bs1_kernel<8, KS>, grid, 128 * KS, lds, st, a); break;
    case 4: launch(gateup_bs1_kernel<4, KS>, grid, 128 * KS, lds, st, a); break;
    case 2: launch(gateup_bs1_kernel<2, KS>, grid, 128 * KS, lds, st, a); break;
    default: launch(gateup_bs1_kernel<1, KS>, grid, 128 * KS, lds, st, a); break;
    }
}

// slots: how many slots from 0 the launch covers (k when the shared expert
// already ran in the top-k launch, k + n_shared otherwise).
hipError_t launch_gateup_bs1(const Bs1Args &a, int slots, hipStream_t st)
{
    const dim3 grid(slots, a.F / 16);
    const size_t lds = (size_t)a.H;
    // K split over 4 waves per tile (12 KB of weights per wave) when the
    // H/128 chunk batches divide by 4, else over 2 (H is a multiple of 256)
    if ((a.H >> 7) % 4 == 0)
        gateup_bs1_u<4>(a, grid, lds, st);
    else
        gateup_bs1_u<2>(a, grid, lds, st);
    return hipGetLastError();
}

hipError_t launch_topk_bs1(const double *logits, const float *bias, int E, float r,
                           const void *const *ptrs,
                           int32_t *idx_out, float *w_out, const void **sel, const Bs1Args &a,
                           hipStream_t st)
{
    const size_t lds = (size_t)a.H;
    // shared gate/up over half tile pairs when H/1024 loads per lane fit
    if (a.n_shared && a.H % 1024 == 0) {
        const int blocks = 1 + a.F / 8;
        switch (a.H >> 10) {
        case 2: launch(topk_bs1h_kernel<2>, blocks, 512, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); return hipGetLastError();
        case 4: launch(topk_bs1h_kernel<4>, blocks, 512, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); return hipGetLastError();
        case 6: launch(topk_bs1h_kernel<6>, blocks, 512, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); return hipGetLastError();
        case 8: launch(topk_bs1h_kernel<8>, blocks, 512, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); return hipGetLastError();
        default: break;
        }
    }
    const int blocks = 1 + (a.n_shared ? a.F / 16 : 0);
    switch (bs1_u((a.H >> 7) / 2, 16)) {
    case 16: launch(topk_bs1_kernel<16>, blocks, 256, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); break;
    case 12: launch(topk_bs1_kernel<12>, blocks, 256, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); break;
    case 8: launch(topk_bs1_kernel<8>, blocks, 256, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); break;
    case 6: launch(topk_bs1_kernel<6>, blocks, 256, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); break;
    case 4: launch(topk_bs1_kernel<4>, blocks, 256, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); break;
    case 2: launch(topk_bs1_kernel<2>, blocks, 256, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); break;
    default: launch(topk_bs1_kernel<1>, blocks, 256, lds, st, logits, bias, E, r, ptrs, idx_out, w_out, sel, a); break;
    }
    return hipGetLastError();
}

#ifndef MOE_BS1_DOWN_TPW
#define MOE_BS1_DOWN_TPW 2
#endif
#ifndef MOE_BS1_DOWN_U
#define MOE_BS1_DOWN_U 2
#endif

hipError_t launch_down_bs1(const Bs1Args &a, hipStream_t st)
{
    constexpr int TPW = MOE_BS1_DOWN_TPW;
    const int S = a.k + a.n_shared;
    const dim3 grid(a.H / (16 * TPW));
    const size_t lds = (size_t)S * a.F;
    // half tiles for F = 2048 and up to 9 slots: NH = H/2048 half tiles per
    // block (H/(8 NH) blocks, 256 for H = 6144), else one; H = 8192 takes two
    // over 512 blocks (four would hold more load registers than fit: spills)
    if (S <= 9 && a.F == 2048) {
        int nh = (a.H % 2048 == 0) ? a.H / 2048 : 1;
        if (nh > 3)
            nh = (nh % 2 == 0) ? 2 : 1;
        const dim3 g(a.H / (8 * nh));
        // the shared expert over four K-quarter waves when it exists and the
        // block stays within 12 waves
        if (a.n_shared && a.k <= 8) {
            const int nt = 64 * (a.k + 4);
            switch (nh) {
            case 1: launch(down_bs1h_kernel<1, true>, g, nt, lds, st, a); return hipGetLastError();
            case 2: launch(down_bs1h_kernel<2, true>, g, nt, lds, st, a); return hipGetLastError();
            case 3: launch(down_bs1h_kernel<3, true>, g, nt, lds, st, a); return hipGetLastError();
            default: break;
            }
        }
        switch (nh) {
        case 1: launch(down_bs1h_kernel<1, false>, g, 64 * S, lds, st, a); return hipGetLastError();
        case 2: launch(down_bs1h_kernel<2, false>, g, 64 * S, lds, st, a); return hipGetLastError();
        case 3: launch(down_bs1h_kernel<3, false>, g, 64 * S, lds, st, a); return hipGetLastError();
        default: break;
        }
    }
    // two batches of 2 loads in flight per wave next to the SwiGLU row: for up
    // to 9 slots the block may use 3 waves per SIMD, for up to 16 slots 4
    if (S <= 9)
        launch(down_bs1_kernel<MOE_BS1_DOWN_U, 9, true, TPW>, grid, 64 * S, lds, st, a);
    else
        launch(down_bs1_kernel<2, 16, true, TPW>, grid, 64 * S, lds, st, a);
    return hipGetLastError();
}

}  // namespace moe
