// topk_common.h -- selection of the k best experts of one token on gfx950:
// the order is the DeepSeek-V3 one (larger biased score first, lower expert
// index on ties; "Guide Complet de Colibri", table "Points techniques cles",
// router row).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

#include <climits>
#include <cstdint>

namespace moe {

// True when (ca, ia) comes before (cb, ib) in the selection order: larger
// biased score first, the lower expert index on ties.
__device__ __forceinline__ bool sel_before(double ca, int ia, double cb, int ib)
{
    return ca > cb || (ca == cb && ia < ib);
}

// One compare-exchange step of the bitonic network over the 64 lanes of a
// wave: lane pairs at distance STRIDE inside sequences of SIZE lanes.
template <int SIZE, int STRIDE>
__device__ __forceinline__ void sort_step(double &c, int &ci)
{
    const int lane = threadIdx.x & 63;
    const double oc = xor_lane_d<STRIDE>(c);
    const int oi = xor_lane<STRIDE>(ci);
    const bool lower = (lane & STRIDE) == 0;
    const bool up = (lane & SIZE) == 0 || SIZE == 64;
    const bool other_first = sel_before(oc, oi, c, ci);
    if ((lower == up) ? other_first : !other_first) {
        c = oc;
        ci = oi;
    }
}

// Bitonic sort of one (c, i) pair per lane across the 64 lanes of a wave, so
// that lane 0 holds the first in the selection order, lane 1 the second ...
__device__ __forceinline__ void wave_sort_sel(double &c, int &ci)
{
    sort_step<2, 1>(c, ci);
    sort_step<4, 2>(c, ci);
    sort_step<4, 1>(c, ci);
    sort_step<8, 4>(c, ci);
    sort_step<8, 2>(c, ci);
    sort_step<8, 1>(c, ci);
    sort_step<16, 8>(c, ci);
    sort_step<16, 4>(c, ci);
    sort_step<16, 2>(c, ci);
    sort_step<16, 1>(c, ci);
    sort_step<32, 16>(c, ci);
    sort_step<32, 8>(c, ci);
    sort_step<32, 4>(c, ci);
    sort_step<32, 2>(c, ci);
    sort_step<32, 1>(c, ci);
    sort_step<64, 32>(c, ci);
    sort_step<64, 16>(c, ci);
    sort_step<64, 8>(c, ci);
    sort_step<64, 4>(c, ci);
    sort_step<64, 2>(c, ci);
    sort_step<64, 1>(c, ci);
}

// Merge of sorted runs of R lanes (R = 16 or 32, each in the selection order)
// into one sorted wave: the caller loads the odd runs reversed, so that every
// pair of runs forms a bitonic sequence, and the half-cleaner stages from
// 2R lanes up to 64 finish the sort (11 steps for R = 16, 6 for R = 32,
// against 21 for a full sort).
template <int R>
__device__ __forceinline__ void wave_merge_sel(double &c, int &ci)
{
    static_assert(R == 16 || R == 32, "runs of 16 or 32 lanes");
    if constexpr (R == 16) {
        sort_step<32, 16>(c, ci);
        sort_step<32, 8>(c, ci);
        sort_step<32, 4>(c, ci);
        sort_step<32, 2>(c, ci);
        sort_step<32, 1>(c, ci);
    }
    sort_step<64, 32>(c, ci);
    sort_step<64, 16>(c, ci);
    sort_step<64, 8>(c, ci);
    sort_step<64, 4>(c, ci);
    sort_step<64, 2>(c, ci);
    sort_step<64, 1>(c, ci);
}

// Index to load lane l's candidate from, for runs of R sorted entries laid
// out one after another: the odd runs reversed (see wave_merge_sel).
template <int R>
__device__ __forceinline__ int merge_src(int l)
{
    const int run = l / R, pos = l % R;
    return (run & 1) ? run * R + (R - 1 - pos) : l;
}

// Top-k of one token for E <= 64*NW (NW = 4, 8 or 16 waves), k <= KEEP (16 or
// 32).  Thread e < E holds the biased score c of expert e (NaN already mapped
// to -inf) and has put its sigmoid score in s_s[e]; other threads hold (-inf,
// INT_MAX).  Each wave sorts its 64 candidates and keeps the first KEEP; while
// more than 64 remain, waves sort them again 64 at a time and keep KEEP of
// each 64; wave 0 sorts the last at most 64.  Every group of 64 keeps all of
// its members that belong to the global top k (k <= KEEP), and the order is
// total, so the grouping does not change the result.  Writes the ranks' ids
// (s_idx too) and weights w_i = s_i / sum(s) * r, the sum taken in rank order
// in fp64.  cand_c/cand_i hold KEEP*NW entries, s_idx and sel_s KEEP.
template <int NW, int KEEP>
__device__ __forceinline__ void topk_select_waves(double c, int ci, const double *s_s, int k,
                                                  float r, int32_t *__restrict__ idx_out,
                                                  float *__restrict__ w_out, int32_t *s_idx,
                                                  double *cand_c, int *cand_i, double *sel_s)
{
    static_assert(KEEP == 16 || KEEP == 32, "a wave keeps 16 or 32 candidates");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    wave_sort_sel(c, ci);                            // s_s is read after the next barrier
    if (lane < KEEP) {
        cand_c[wave * KEEP + lane] = c;
        cand_i[wave * KEEP + lane] = ci;
    }
    __syncthreads();
    // candidates left: KEEP*NW, then KEEP per 64 of them per round; every 64
    // of them are 64/KEEP sorted runs, merged rather than sorted again
#pragma unroll
    for (int n = KEEP * NW; n > 64; n = n / 64 * KEEP) {
        const int nw = n / 64;
        double cc = -INFINITY;
        int cci = INT_MAX;
        if (wave < nw) {
            const int src = 64 * wave + merge_src<KEEP>(lane);
            cc = cand_c[src];
            cci = cand_i[src];
            wave_merge_sel<KEEP>(cc, cci);
        }
        __syncthreads();
        if (wave < nw && lane < KEEP) {
            cand_c[KEEP * wave + lane] = cc;
            cand_i[KEEP * wave + lane] = cci;
        }
        __syncthreads();
    }
    constexpr int NL = [] {
        int n = KEEP * NW;
        while (n > 64)
            n = n / 64 * KEEP;
        return n;
    }();                                             // at most 64 candidates left
    if (wave == 0) {
        // NL = KEEP * (number of runs): sorted runs of KEEP, padded past NL
        // with entries that sort last
        const int src = merge_src<KEEP>(lane);
        c = lane < NL ? cand_c[src] : -INFINITY;
        ci = lane < NL ? cand_i[src] : INT_MAX;
        wave_merge_sel<KEEP>(c, ci);
        if (lane < k) {
            s_idx[lane] = ci;
            sel_s[lane] = s_s[ci];
        }
    }
    __syncthreads();
    if (tid < k) {
        double den = 0.0;
        for (int i = 0; i < k; ++i)
            den += sel_s[i];
        const double wi = (den > 0.0) ? (sel_s[tid] / den) * (double)r : 0.0;
        idx_out[tid] = s_idx[tid];
        w_out[tid] = (float)wi;
    }
    __syncthreads();
}

// E <= 256 on 256 threads (three barriers).
__device__ __forceinline__ void topk_select_256(double c, int ci, const double *s_s, int k,
                                                float r, int32_t *__restrict__ idx_out,
                                                float *__restrict__ w_out, int32_t *s_idx,
                                                double *cand_c, int *cand_i, double *sel_s)
{
    topk_select_waves<4, 16>(c, ci, s_s, k, r, idx_out, w_out, s_idx, cand_c, cand_i, sel_s);
}

}  // namespace moe
