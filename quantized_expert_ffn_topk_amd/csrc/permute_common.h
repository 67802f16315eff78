// Single-block bodies of the few-token routing permutation and of the row
// tile list, shared by their own kernels and by the fused few-token
// preparation launch of the MXFP4 path.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace moe {

// The routing permutation for at most 256 entries (decode at a few tokens), in
// one block: the entries go to LDS once, thread e collects the slots of expert
// e in token order (four entries per LDS read), and the experts with rows
// are compacted in expert order.  At 2-8 tokens ≈4-5 µs against ≈8 µs for the
// block-per-expert form (its 257 blocks each scan every entry); at 16 tokens
// both take ≈8 µs.
__device__ __forceinline__ void permute_small_block(const int32_t *__restrict__ idx, int T,
                                                    int k, int E, int n_shared,
                                                    int32_t *__restrict__ cnt,
                                                    int32_t *__restrict__ list,
                                                    int list_stride,
                                                    int32_t *__restrict__ active,
                                                    int32_t *__restrict__ n_active)
{
    __shared__ __align__(16) int s_idx[256];
    __shared__ int s_wc[16];
    const int N = T * k, S = k + n_shared, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int N4 = (N + 3) & ~3;                   // padded with -1 (no expert)
    if (tid < N4)
        s_idx[tid] = tid < N ? idx[tid] : -1;
    __syncthreads();
    const int nE = E + n_shared;
    int base = 0;
    for (int e0 = 0; e0 < nE; e0 += 1024) {
        const int e = e0 + tid;
        int c = 0;
        if (e < E) {
            int32_t *mine = list + (size_t)e * list_stride;
            for (int j4 = 0; j4 < N4; j4 += 4) {
                const int4 v = *reinterpret_cast<const int4 *>(s_idx + j4);
                const int vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (vv[q] == e) {
                        // ids repeated within a token (not allowed by the API)
                        // could give an expert more rows than its list holds:
                        // extra rows are dropped
                        if (c < list_stride) {
                            const int j = j4 + q, t = j / k, i = j - t * k;
                            mine[c] = t * S + i;
                        }
                        ++c;
                    }
                }
            }
        } else if (e < nE) {                       // the shared expert: every token
            int32_t *mine = list + (size_t)e * list_stride;
            for (int t = 0; t < T; ++t)
                mine[t] = t * S + k;
            c = T;
        }
        if (e < nE)
            cnt[e] = c < list_stride ? c : list_stride;
        const bool has = e < nE && c > 0;
        const uint64_t bal = __ballot(has);
        if (lane == 0)
            s_wc[wave] = __popcll(bal);
        __syncthreads();
        int off = base, tot = 0;
        for (int v = 0; v < 16; ++v) {
            off += (v < wave) ? s_wc[v] : 0;
            tot += s_wc[v];
        }
        if (has)
            active[off + __popcll(bal & ((1ull << lane) - 1ull))] = e;
        __syncthreads();
        base += tot;
    }
    if (tid == 0)
        *n_active = base;
}

// The same permutation, ballot form: one block of 16 waves; the entries go to LDS once; wave w takes experts w,
// w + 16, ..., and finds an expert's entries 64 at a time with one ballot
// (lanes = consecutive entries, so the rows land in token order at the
// popcount of the lanes below); then one wave compacts the experts with rows
// in expert order.  Each wave runs ceil(nE/16) * ceil(N/64) ballot steps,
// where the thread-per-expert form runs N/4 LDS reads per thread: with few
// experts and many entries this form wins (64 experts, 128 entries: 4.2-4.7
// against 12.6-13.4 us), with many experts and few entries the other.
__device__ __forceinline__ void permute_small_ballot_block(const int32_t *__restrict__ idx, int T,
                                                           int k, int E, int n_shared,
                                                           int32_t *__restrict__ cnt,
                                                           int32_t *__restrict__ list,
                                                           int list_stride,
                                                           int32_t *__restrict__ active,
                                                           int32_t *__restrict__ n_active)
{
    __shared__ int s_idx[256];
    __shared__ int s_cnt[1024 + 1];
    const int N = T * k, S = k + n_shared, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    if (tid < 256)
        s_idx[tid] = tid < N ? idx[tid] : -1;
    __syncthreads();
    const int nE = E + n_shared;
    for (int e = wave; e < nE; e += 16) {
        int32_t *mine = list + (size_t)e * list_stride;
        int c = 0;
        if (e < E) {
            for (int j0 = 0; j0 < N; j0 += 64) {
                const int j = j0 + lane;
                const bool hit = j < N && s_idx[j] == e;
                const uint64_t bal = __ballot(hit);
                if (hit) {
                    // ids repeated within a token (not allowed by the API)
                    // could give an expert more rows than its list holds:
                    // extra rows are dropped
                    const int pos = c + __popcll(bal & below);
                    if (pos < list_stride) {
                        const int t = j / k, i = j - t * k;
                        mine[pos] = t * S + i;
                    }
                }
                c += __popcll(bal);
            }
        } else {                                   // the shared expert: every token
            for (int t = lane; t < T; t += 64)
                mine[t] = t * S + k;
            c = T;
        }
        if (lane == 0) {
            cnt[e] = c < list_stride ? c : list_stride;
            s_cnt[e] = c;
        }
    }
    __syncthreads();
    if (wave == 0) {
        int na = 0;
        for (int e0 = 0; e0 < nE; e0 += 64) {
            const int e = e0 + lane;
            const bool has = e < nE && s_cnt[e] > 0;
            const uint64_t bal = __ballot(has);
            if (has)
                active[na + __popcll(bal & below)] = e;
            na += __popcll(bal);
        }
        if (lane == 0)
            *n_active = na;
    }
}

// ---------------------------------------------------------------------------
// Tile list: for experts 0..n_exp-1 in order, ceil(cnt/mt) tiles (e, m0).
// One block of 1024 threads; n_exp <= 2048.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void row_tiles_block(const int32_t *__restrict__ cnt,
                                                int n_exp, int mt,
                                                int2 *__restrict__ tiles,
                                                int32_t *__restrict__ n_tiles)
{
    __shared__ int sc[1024];
    const int t = threadIdx.x;
    const int e0 = 2 * t, e1 = 2 * t + 1;
    const int c0 = e0 < n_exp ? (cnt[e0] + mt - 1) / mt : 0;
    const int c1 = e1 < n_exp ? (cnt[e1] + mt - 1) / mt : 0;
    sc[t] = c0 + c1;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int v = (t >= off) ? sc[t - off] : 0;
        __syncthreads();
        sc[t] += v;
        __syncthreads();
    }
    int base = sc[t] - c0 - c1;
    for (int j = 0; j < c0; ++j)
        tiles[base + j] = make_int2(e0, j * mt);
    for (int j = 0; j < c1; ++j)
        tiles[base + c0 + j] = make_int2(e1, j * mt);
    if (t == 1023)
        *n_tiles = sc[1023];
}

}  // namespace moe
