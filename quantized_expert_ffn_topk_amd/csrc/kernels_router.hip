// kernels_router.hip -- activation quantisation, sigmoid router, top-k and the
// token->expert permutation for gfx950.
//
// Router: DeepSeek-V3 style ("Guide Complet de Colibri", table "Points
// techniques cles", router row): sigmoid scores, a bias that only steers the
// selection, the k best experts per token, weights normalised over the
// selected experts and multiplied by the routed scale.  Logits and scores are
// computed in fp64 so that the choice does not depend on summation order.
#include "device_common.h"
#include "moe_internal.h"
#include "topk_common.h"
#include "permute_common.h"

#include <climits>

namespace moe {

// ---------------------------------------------------------------------------
// Per-token int8 quantisation: amax over the row, inv = 127/amax and
// s = amax/127 in fp32 (correctly rounded), q = clamp(rint(x*inv), -127, 127).
// One 256-thread block per token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_tokens_kernel(const uint16_t *__restrict__ x, int H,
                                                           int8_t *__restrict__ q,
                                                           float *__restrict__ s)
{
    __shared__ float red[4];
    const int t = blockIdx.x;
    const uint16_t *xr = x + (size_t)t * H;
    float amax = 0.0f;
    for (int i = threadIdx.x * 8; i < H; i += 2048) {
        uint4 v = *reinterpret_cast<const uint4 *>(xr + i);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            amax = fmaxf(amax, fabsf(bf16_to_f32(w[j] & 0xffffu)));
            amax = fmaxf(amax, fabsf(bf16_to_f32(w[j] >> 16)));
        }
    }
    amax = block_max_256(amax, red);
    float inv = 0.0f, sc = 0.0f;
    if (amax > 0.0f) {
        inv = 127.0f / amax;
        sc = amax / 127.0f;
    }
    int8_t *qr = q + (size_t)t * H;
    for (int i = threadIdx.x * 8; i < H; i += 2048) {
        uint4 v = *reinterpret_cast<const uint4 *>(xr + i);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float xv = bf16_to_f32((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu));
            float r = rintf(xv * inv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            int qi = (int)r;
            packed[j >> 2] |= ((uint32_t)qi & 0xffu) << (8 * (j & 3));
        }
        *reinterpret_cast<uint2 *>(qr + i) = make_uint2(packed[0], packed[1]);
    }
    if (threadIdx.x == 0)
        s[t] = sc;
}

hipError_t launch_quant_tokens(const uint16_t *x, int T, int H, int8_t *q, float *s,
                               hipStream_t st)
{
    if (T <= 0)
        return hipSuccess;
    launch(quant_tokens_kernel, T, 256, 0, st, x, H, q, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router logits l[t,e] = sum_k x[t,k]*Wr[e,k] in fp64 (bf16 x fp32 products
// are exact in fp64).
// 2-16 tokens: one block per expert and TB tokens; its four waves split the
// router row into four K slices, each slice's loads in flight together (one
// batch of U 256-input steps for H = 6144), and the slices' sums are added in
// slice order.  Many tokens: the fp64 MFMA below.
// ---------------------------------------------------------------------------
template <int TB>
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t *__restrict__ x, int T,
                                                          int H, const float *__restrict__ Wr,
                                                          int E, double *__restrict__ logits)
{
    constexpr int U = 6;                         // 256-input steps whose loads fly together
    __shared__ double part[4][TB];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * TB;
    const float *w = Wr + (size_t)e * H;
    const uint16_t *xr[TB];
#pragma unroll
    for (int m = 0; m < TB; ++m)                 // rows past T repeat row T-1 (not stored)
        xr[m] = x + (size_t)min(t0 + m, T - 1) * H;
    double acc[TB];
#pragma unroll
    for (int m = 0; m < TB; ++m)
        acc[m] = 0.0;
    const int nk = H / 256;                      // H is a multiple of 256
    const int k_lo = wave * nk / 4, k_hi = (wave + 1) * nk / 4;   // this wave's steps
    for (int k0 = k_lo; k0 < k_hi; k0 += U) {
        float4 wv[U];
        uint2 xv[U][TB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = 256 * min(k0 + u, k_hi - 1) + lane * 4;   // clamped: in the slice
            wv[u] = *reinterpret_cast<const float4 *>(w + k);
#pragma unroll
            for (int m = 0; m < TB; ++m)
                xv[u][m] = *reinterpret_cast<const uint2 *>(xr[m] + k);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (k0 + u < k_hi) {
#pragma unroll
                for (int m = 0; m < TB; ++m) {
                    acc[m] = fma((double)bf16_to_f32(xv[u][m].x & 0xffffu), (double)wv[u].x, acc[m]);
                    acc[m] = fma((double)bf16_to_f32(xv[u][m].x >> 16), (double)wv[u].y, acc[m]);
                    acc[m] = fma((double)bf16_to_f32(xv[u][m].y & 0xffffu), (double)wv[u].z, acc[m]);
                    acc[m] = fma((double)bf16_to_f32(xv[u][m].y >> 16), (double)wv[u].w, acc[m]);
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < TB; ++m) {
        const double v = wave_sum_d(acc[m]);
        if (lane == 0)
            part[wave][m] = v;
    }
    __syncthreads();
    if (threadIdx.x < TB && t0 + (int)threadIdx.x < T) {
        const int m = threadIdx.x;
        logits[(size_t)(t0 + m) * E + e] = ((part[0][m] + part[1][m]) + part[2][m]) + part[3][m];
    }
}

// Many tokens on the fp64 MFMA (v_mfma_f64_16x16x4_f64; checked on the
// device: lane l supplies A[l%16][l/16] and B[l/16][l%16], result register i
// of lane l is D[l/16 + 4i][l%16]).  A wave computes MT tiles of 16 tokens
// against one tile of 16 experts over a K slice; the block's KS waves take KS
// consecutive slices and their partial sums are added in slice order.  Every
// product of a bf16 input and an fp32 weight is exact in fp64.  For each 32
// inputs, lane group g = l/16 loads inputs 8g..8g+7 of its token row and its
// router row, and MFMA j takes element j of them: the 32 products are summed
// in an order fixed by the kernel.
template <int MT, int KS>
__global__ __launch_bounds__(64 * KS) void router_mfma_kernel(const uint16_t *__restrict__ x,
                                                              int T, int H,
                                                              const float *__restrict__ Wr,
                                                              int E, double *__restrict__ logits)
{
    typedef double f64x4 __attribute__((ext_vector_type(4)));
    __shared__ double part[KS > 1 ? KS : 1][MT][4][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16 * MT;
    // gridDim.z K parts on separate blocks, part z written to logits + z*T*E
    const int KL = H / (KS * gridDim.z), kb = blockIdx.z * (H / gridDim.z) + wave * KL;
    logits += (size_t)blockIdx.z * T * E;
    const float *wrow = Wr + (size_t)min(e0 + r, E - 1) * H + kb + 8 * g;   // clamped rows
    const uint16_t *xrow[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        xrow[m] = x + (size_t)min(t0 + 16 * m + r, T - 1) * H + kb + 8 * g;
    f64x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        acc[m] = f64x4{0.0, 0.0, 0.0, 0.0};
    // the loads of step k + 32 are issued before step k is summed (the last
    // step reloads itself, so every load is unconditional and in bounds)
    float4 w0n = *reinterpret_cast<const float4 *>(wrow);
    float4 w1n = *reinterpret_cast<const float4 *>(wrow + 4);
    uint4 xvn[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        xvn[m] = *reinterpret_cast<const uint4 *>(xrow[m]);
    for (int k = 0; k < KL; k += 32) {
        const float4 w0 = w0n, w1 = w1n;
        uint4 xv[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m)
            xv[m] = xvn[m];
        const int kn = min(k + 32, KL - 32);
        w0n = *reinterpret_cast<const float4 *>(wrow + kn);
        w1n = *reinterpret_cast<const float4 *>(wrow + kn + 4);
#pragma unroll
        for (int m = 0; m < MT; ++m)
            xvn[m] = *reinterpret_cast<const uint4 *>(xrow[m] + kn);
        const float wf[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const double b = (double)wf[j];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint32_t d = (j >> 1) == 0 ? xv[m].x : (j >> 1) == 1 ? xv[m].y
                                 : (j >> 1) == 2 ? xv[m].z : xv[m].w;
                const double a = (double)bf16_to_f32((j & 1) ? (d >> 16) : (d & 0xffffu));
                acc[m] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[m], 0, 0, 0);
            }
        }
    }
    if (KS > 1) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part[wave][m][i][lane] = acc[m][i];
        __syncthreads();
        if (wave != 0)
            return;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                double v = part[0][m][i][lane];
#pragma unroll
                for (int q = 1; q < KS; ++q)
                    v += part[q][m][i][lane];
                acc[m][i] = v;
            }
    }
    const int e = e0 + r;
    if (e >= E)
        return;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 16 * m + g + 4 * i;
            if (t < T)
                logits[(size_t)t * E + e] = acc[m][i];
        }
}

// Few 16-token tiles (fewer than 128 blocks): the two K halves go to separate
// blocks, so twice as many CUs run the fp64 MFMA; the top-k launch adds the
// two partial logits in order.  Needs whole 32-input steps per wave.
int router_ksplit(int T, int H, int E)
{
    if (T <= 16 || T >= 1024)
        return 1;
    const int ne = (E + 15) / 16, H32 = H / 32;
    const long tiles = (long)ne * ((T + 15) / 16);
    if (tiles >= 128)
        return 1;
    const int ks = (H32 % 16) ? 8 : 16;
    return (H32 % (2 * ks) == 0) ? 2 : 1;
}

hipError_t launch_router_logits(const uint16_t *x, int T, int H, const float *Wr, int E,
                                double *logits, hipStream_t st)
{
    if (T <= 0)
        return hipSuccess;
    if (T <= 16) {
        dim3 grid(E, (T + 3) / 4);
        launch(router_gemv_kernel<4>, grid, 256, 0, st, x, T, H, Wr, E, logits);
        return hipGetLastError();
    }
    // enough waves to fill the chip: 64-token tiles with 4 K slices for many
    // tokens (4 waves per SIMD; 1 or 2 slices ran 1.5x slower, 8 slices or
    // 32-token tiles 1.1-1.2x slower at 4096 tokens), 16-token tiles with up
    // to 16 slices for few (H/32 is a multiple of 8, so 1, 2, 4 and 8 slices
    // of whole 32-input steps always exist)
    const int ne = (E + 15) / 16, H32 = H / 32;
    if (T >= 1024) {
        dim3 grid(ne, (T + 63) / 64);
        launch(router_mfma_kernel<4, 4>, grid, 256, 0, st, x, T, H, Wr, E, logits);
    } else {
        dim3 grid(ne, (T + 15) / 16, router_ksplit(T, H, E));
        const long tiles = (long)grid.x * grid.y;
        if (tiles >= 512 || H32 % 16)
            launch(router_mfma_kernel<1, 8>, grid, 512, 0, st, x, T, H, Wr, E, logits);
        else
            launch(router_mfma_kernel<1, 16>, grid, 1024, 0, st, x, T, H, Wr, E, logits);
    }
    return hipGetLastError();
}

// Top-k of token t = blockIdx.x for E <= 64*NW: thread e scores expert e, then
// the bitonic selection of the one-token path (lowest index first on ties).
// With xq set the block also quantises token t (the rule of
// quant_tokens_kernel), its row loads issued before the selection.
template <int NW, int KEEP>
__global__ __launch_bounds__(64 * NW) void topk_block_kernel(double *__restrict__ logits,
                                                             const float *__restrict__ bias, int E,
                                                             int k, float r, int32_t *__restrict__ idx,
                                                             float *__restrict__ w,
                                                             const uint16_t *__restrict__ x, int H,
                                                             int8_t *__restrict__ xq,
                                                             float *__restrict__ sa, int kparts)
{
    constexpr int NT = 64 * NW;
    constexpr int XL = 8192 / (8 * NT);          // 16-byte pieces per thread, H <= 8192
    __shared__ double s_s[64 * NW], cand_c[KEEP * NW], sel_s[KEEP];
    __shared__ int cand_i[KEEP * NW], s_idx[KEEP];
    __shared__ float s_am[NW];
    const int t = blockIdx.x, tid = threadIdx.x;
    uint4 xv[XL];
    if (xq) {
        const uint4 *xr = reinterpret_cast<const uint4 *>(x + (size_t)t * H);
#pragma unroll
        for (int i = 0; i < XL; ++i)               // clamped: every load in bounds
            xv[i] = xr[min(tid + NT * i, H / 8 - 1)];
    }
    double c = -INFINITY;
    int ci = INT_MAX;
    if (tid < E) {
        double l = logits[(size_t)t * E + tid];
        if (kparts == 2) {                       // two K halves: summed in order, kept
            l = l + logits[(size_t)gridDim.x * E + (size_t)t * E + tid];
            logits[(size_t)t * E + tid] = l;
        }
        const double sv = 1.0 / (1.0 + exp(-l));
        const double cv = sv + (double)bias[tid];
        s_s[tid] = sv;
        c = (cv != cv) ? -INFINITY : cv;
        ci = tid;
    }
    topk_select_waves<NW, KEEP>(c, ci, s_s, k, r, idx + (size_t)t * k, w + (size_t)t * k, s_idx,
                                cand_c, cand_i, sel_s);
    if (!xq)
        return;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        if (8 * (tid + NT * i) < H) {
            const uint32_t wd[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(wd[j] & 0xffffu)), fabsf(bf16_to_f32(wd[j] >> 16))));
        }
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0)
        s_am[tid >> 6] = amax;
    __syncthreads();
    amax = s_am[0];
#pragma unroll
    for (int v = 1; v < NW; ++v)
        amax = fmaxf(amax, s_am[v]);
    float inv = 0.0f, sc = 0.0f;
    if (amax > 0.0f) {
        inv = 127.0f / amax;
        sc = amax / 127.0f;
    }
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        const int p = tid + NT * i;
        if (8 * p < H) {
            const uint32_t wd[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xf = bf16_to_f32((j & 1) ? (wd[j >> 1] >> 16) : (wd[j >> 1] & 0xffffu));
                const float q = fminf(fmaxf(rintf(xf * inv), -127.0f), 127.0f);
                packed[j >> 2] |= ((uint32_t)(int)q & 0xffu) << (8 * (j & 3));
            }
            *reinterpret_cast<uint2 *>(xq + (size_t)t * H + 8 * p) = make_uint2(packed[0], packed[1]);
        }
    }
    if (tid == 0)
        sa[t] = sc;
}

template <int KEEP>
static void launch_topk_keep(double *logits, const float *bias, int T, int E, int k, float r,
                             int32_t *idx, float *w, hipStream_t st, const uint16_t *x, int H,
                             int8_t *xq, float *sa, int kparts)
{
    if (E <= 256)
        launch(topk_block_kernel<4, KEEP>, T, 256, 0, st, logits, bias, E, k, r, idx, w, x, H, xq,
               sa, kparts);
    else if (E <= 512)
        launch(topk_block_kernel<8, KEEP>, T, 512, 0, st, logits, bias, E, k, r, idx, w, x, H, xq,
               sa, kparts);
    else
        launch(topk_block_kernel<16, KEEP>, T, 1024, 0, st, logits, bias, E, k, r, idx, w, x, H, xq,
               sa, kparts);
}

hipError_t launch_topk(double *logits, const float *bias, int T, int E, int k, float r,
                       int32_t *idx, float *w, hipStream_t st, const uint16_t *x, int H,
                       int8_t *xq, float *sa, int kparts)
{
    if (T <= 0)
        return hipSuccess;
    // E <= 1024 and k <= 32 (checked at context creation)
    if (k <= 16)
        launch_topk_keep<16>(logits, bias, T, E, k, r, idx, w, st, x, H, xq, sa, kparts);
    else
        launch_topk_keep<32>(logits, bias, T, E, k, r, idx, w, st, x, H, xq, sa, kparts);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token -> expert permutation.  Block e (e < E) collects, in token order, the
// slots t*S+i with idx[t,i] == e; block E (shared expert, when present) takes
// every token at slot t*S+k.  The last block to finish lists the experts that
// received rows, in expert order.
// Ordered compaction without a barrier per step: wave w owns a contiguous
// quarter of the T*k entries; a first pass counts its matches (wave ballots),
// one barrier turns the four counts into offsets, and a second pass writes
// the matches at their ranks.  Each pass reads batches of 8 entries per lane
// with the next batch's loads in flight.
// ---------------------------------------------------------------------------
constexpr int PERM_U = 8;

// count (WRITE = false) or write (WRITE = true) the matches of e in
// idx[j_begin, j_end); `base` is the wave's first output rank
template <bool WRITE>
__device__ __forceinline__ int permute_pass(const int32_t *__restrict__ idx, int j_begin, int j_end,
                                            int e, int k, int S, int32_t *__restrict__ mine,
                                            int list_stride, int base)
{
    const int lane = threadIdx.x & 63;
    const int last = max(j_end - 1, 0);
    int run = base;
    int nxt[PERM_U];
#pragma unroll
    for (int u = 0; u < PERM_U; ++u)
        nxt[u] = idx[min(j_begin + 64 * u + lane, last)];
    for (int j0 = j_begin; j0 < j_end; j0 += 64 * PERM_U) {
        int cur[PERM_U];
#pragma unroll
        for (int u = 0; u < PERM_U; ++u) {
            cur[u] = nxt[u];
            nxt[u] = idx[min(j0 + 64 * (PERM_U + u) + lane, last)];
        }
#pragma unroll
        for (int u = 0; u < PERM_U; ++u) {
            const int j = j0 + 64 * u + lane;
            const bool m = (j < j_end) && (cur[u] == e);
            const uint64_t bal = __ballot(m);
            if (WRITE && m) {
                const int pos = run + __popcll(bal & ((1ull << lane) - 1ull));
                // ids repeated within a token (not allowed by the API) could
                // give an expert more rows than its list holds: extra rows
                // are dropped
                if (pos < list_stride) {
                    const int t = j / k, i = j - t * k;
                    mine[pos] = t * S + i;
                }
            }
            run += __popcll(bal);
        }
    }
    return run - base;
}

__global__ __launch_bounds__(256) void permute_kernel(const int32_t *__restrict__ idx, int T,
                                                      int k, int E, int n_shared,
                                                      int32_t *__restrict__ cnt,
                                                      int32_t *__restrict__ list,
                                                      int list_stride,
                                                      int32_t *__restrict__ active,
                                                      int32_t *__restrict__ n_active,
                                                      uint32_t *__restrict__ done)
{
    __shared__ int wcnt[4];
    __shared__ int last;
    const int e = blockIdx.x;
    const int S = k + n_shared;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int total = 0;
    int32_t *mine = list + (size_t)e * list_stride;
    if (e < E) {
        const int N = T * k;
        const int Q = (((N + 3) / 4) + 63) & ~63;
        const int jb = min(wave * Q, N), je = min(jb + Q, N);
        const int c = permute_pass<false>(idx, jb, je, e, k, S, mine, list_stride, 0);
        if (lane == 0)
            wcnt[wave] = c;
        __syncthreads();
        int off = 0;
        for (int v = 0; v < wave; ++v)
            off += wcnt[v];
        total = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
        permute_pass<true>(idx, jb, je, e, k, S, mine, list_stride, off);
    } else {
        for (int t = threadIdx.x; t < T; t += 256)
            mine[t] = t * S + k;
        total = T;
    }
    if (threadIdx.x == 0)
        store_dev(cnt + e, total < list_stride ? total : list_stride);
    if (!block_arrives_last(done, gridDim.x, &last) || wave != 0)
        return;
    const int nE = gridDim.x;
    int na = 0;
    for (int e0 = 0; e0 < nE; e0 += 64) {
        int ee = e0 + lane;
        int c = (ee < nE) ? load_dev(cnt + ee) : 0;
        uint64_t bal = __ballot(c > 0);
        if (c > 0)
            active[na + __popcll(bal & ((1ull << lane) - 1ull))] = ee;
        na += __popcll(bal);
    }
    if (lane == 0) {
        *n_active = na;
        *done = 0u;
    }
}

// The permutation for at most 256 entries in one block, one thread per
// expert (permute_small_block).
__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t *__restrict__ idx, int T,
                                                             int k, int E, int n_shared,
                                                             int32_t *__restrict__ cnt,
                                                             int32_t *__restrict__ list,
                                                             int list_stride,
                                                             int32_t *__restrict__ active,
                                                             int32_t *__restrict__ n_active)
{
    permute_small_block(idx, T, k, E, n_shared, cnt, list, list_stride, active, n_active);
}

// The same in one block, one ballot per expert and 64 entries
// (permute_small_ballot_block).
__global__ __launch_bounds__(1024) void permute_small_ballot_kernel(const int32_t *__restrict__ idx, int T,
                                                                    int k, int E, int n_shared,
                                                                    int32_t *__restrict__ cnt,
                                                                    int32_t *__restrict__ list,
                                                                    int list_stride,
                                                                    int32_t *__restrict__ active,
                                                                    int32_t *__restrict__ n_active)
{
    permute_small_ballot_block(idx, T, k, E, n_shared, cnt, list, list_stride, active, n_active);
}

hipError_t launch_permute(const int32_t *idx, int T, int k, int E, int n_shared, int32_t *cnt,
                          int32_t *list, int list_stride, int32_t *active, int32_t *n_active,
                          uint32_t *done_counter, hipStream_t st)
{
    if (T * k <= 256) {
        const int N = T * k, nE = E + n_shared;
        if (((nE + 15) / 16) * ((N + 63) / 64) < N / 4)
            launch(permute_small_ballot_kernel, 1, 1024, 0, st, idx, T, k, E, n_shared, cnt, list,
                   list_stride, active, n_active);
        else
            launch(permute_small_kernel, 1, 1024, 0, st, idx, T, k, E, n_shared, cnt, list,
                   list_stride, active, n_active);
        return hipGetLastError();
    }
    launch(permute_kernel, E + n_shared, 256, 0, st, idx, T, k, E, n_shared, cnt, list, list_stride,
                                                  active, n_active, done_counter);
    return hipGetLastError();
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------
// Small helpers.
// ---------------------------------------------------------------------------
__global__ void set_i32_kernel(int32_t *p, int32_t v)
{
    *p = v;
}

hipError_t launch_set_i32(int32_t *p, int32_t v, hipStream_t st)
{
    launch(set_i32_kernel, 1, 1, 0, st, p, v);
    return hipGetLastError();
}

__global__ void table_update_kernel(const void **table, int set_idx, const void *ptr,
                                    int clear_idx)
{
    if (clear_idx >= 0)
        table[clear_idx] = nullptr;
    table[set_idx] = ptr;
}

hipError_t launch_table_update(const void **table, int set_idx, const void *ptr, int clear_idx,
                               hipStream_t st)
{
    launch(table_update_kernel, 1, 1, 0, st, table, set_idx, ptr, clear_idx);
    return hipGetLastError();
}

}  // namespace moe

namespace moe {

// ---------------------------------------------------------------------------
// Few-token routing in one launch (decode).  With RS_ROUTER, block e computes
// the fp64 logits of expert e for all T tokens (each thread a fixed slice of
// H, then a fixed-order block reduction); the last block to finish then runs
// the per-token top-k.  Every block has read all of x, so with RS_QUANT the
// blocks also share the token quantisation (each codes a slice once the block
// is past the hand-off); without the router a single block quantises.  The
// last (or single) block then builds the routing lists (RS_LISTS): per expert
// its slots in token order, the shared expert's slots, and the list of experts
// with rows.
// ---------------------------------------------------------------------------
// Top-k of one token by ranks: every thread takes experts e = tid + 256j and
// counts the experts that precede e in the order (c desc, index asc); experts
// with rank < k are the selection, in rank order.  s_c/s_s: LDS scratch of E
// doubles each; sel_s: k doubles.
__device__ __forceinline__ void topk_rank_block(const double *__restrict__ lg,
                                                const float *__restrict__ bias, int E, int k,
                                                float r, int32_t *__restrict__ idx_out,
                                                float *__restrict__ w_out, int32_t *s_idx,
                                                double *s_c, double *s_s, double *sel_s)
{
    for (int e = threadIdx.x; e < E; e += 256) {
        const double sv = 1.0 / (1.0 + exp(-load_dev(lg + e)));
        const double cv = sv + (double)bias[e];
        s_s[e] = sv;
        s_c[e] = (cv != cv) ? -INFINITY : cv;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        const double ce = s_c[e];
        int rank = 0;
#pragma unroll 16
        for (int f = 0; f < E; ++f) {
            const double cf = s_c[f];
            rank += (cf > ce || (cf == ce && f < e)) ? 1 : 0;
        }
        if (rank < k) {
            s_idx[rank] = e;
            sel_s[rank] = s_s[e];
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double den = 0.0;
        for (int i = 0; i < k; ++i)
            den += sel_s[i];
        for (int i = 0; i < k; ++i) {
            const double wi = (den > 0.0) ? (sel_s[i] / den) * (double)r : 0.0;
            idx_out[i] = s_idx[i];
            w_out[i] = (float)wi;
        }
    }
    __syncthreads();
}

// Top-k of one token for E <= 256 from the fp64 logits written by the other
// blocks (load_dev): sigmoid scores, biased scores, then topk_select_256.
__device__ __forceinline__ void topk_sort_block(const double *__restrict__ lg,
                                                const float *__restrict__ bias, int E, int k,
                                                float r, int32_t *__restrict__ idx_out,
                                                float *__restrict__ w_out, int32_t *s_idx,
                                                double *s_s, double *cand_c, int *cand_i,
                                                double *sel_s)
{
    const int tid = threadIdx.x;
    double c = -INFINITY;
    int ci = INT_MAX;
    if (tid < E) {
        const double sv = 1.0 / (1.0 + exp(-load_dev(lg + tid)));
        const double cv = sv + (double)bias[tid];
        s_s[tid] = sv;
        c = (cv != cv) ? -INFINITY : cv;
        ci = tid;
    }
    topk_select_256(c, ci, s_s, k, r, idx_out, w_out, s_idx, cand_c, cand_i, sel_s);
}

// This block's share of the per-token quantisation (same rule as
// quant_tokens_kernel) once every block of the router has the amax of each
// token: block b codes the 4-element groups g = tid + 256i of the row with
// g % gridDim.x == b.  xv holds token 0's groups when T == 1.
__device__ __forceinline__ void quant_share(const RouteSmallArgs &a, const uint2 (&xv)[8],
                                            const float (*samax)[RS_MAXT])
{
    const int tid = threadIdx.x, nb = gridDim.x, b = blockIdx.x;
    for (int m = 0; m < a.T; ++m) {
        const float amax = fmaxf(fmaxf(samax[0][m], samax[1][m]), fmaxf(samax[2][m], samax[3][m]));
        float inv = 0.0f, sc = 0.0f;
        if (amax > 0.0f) {
            inv = 127.0f / amax;
            sc = amax / 127.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int g = tid + 256 * i;
            if (4 * g < a.H && g % nb == b) {
                const uint2 v = (a.T == 1) ? xv[i]
                                           : *reinterpret_cast<const uint2 *>(a.x + (size_t)m * a.H + 4 * g);
                const float f[4] = {bf16_to_f32(v.x & 0xffffu), bf16_to_f32(v.x >> 16),
                                    bf16_to_f32(v.y & 0xffffu), bf16_to_f32(v.y >> 16)};
                uint32_t packed = 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float q = fminf(fmaxf(rintf(f[j] * inv), -127.0f), 127.0f);
                    packed |= ((uint32_t)(int)q & 0xffu) << (8 * j);
                }
                *reinterpret_cast<uint32_t *>(a.xq + (size_t)m * a.H + 4 * g) = packed;
            }
        }
        if (b == 0 && tid == 0)
            a.sa[m] = sc;
    }
}

__global__ __launch_bounds__(256) void route_small_kernel(RouteSmallArgs a)
{
    __shared__ double sred[4][RS_MAXT];
    __shared__ float samax[4][RS_MAXT];
    __shared__ int32_t s_idx[RS_MAXT * 16];
    __shared__ double cand_c[64];
    __shared__ int cand_i[64];
    __shared__ double s_c[1024], s_s[1024], sel_s[16];
    __shared__ uint32_t s_bits[33];
    __shared__ float red[4];
    __shared__ int s_last;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int T = a.T;
    const bool spread_quant = (a.flags & RS_ROUTER) && (a.flags & RS_QUANT);
    uint2 xq_v[8];                       // this block's share of token 0 (T == 1)
    if (a.flags & RS_ROUTER) {
        const int e = blockIdx.x;
        // all of this thread's router-row loads first (H <= 8192), then the
        // FMAs; lanes past H read the row's first inputs and zero them after
        // the loads (a load under the branch let the compiler convert each
        // value as it arrived, one round trip at a time)
        constexpr int NI = 8;
        float4 wv[NI];
        const float *wr = a.Wr + (size_t)e * a.H;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int k0 = tid * 4 + 1024 * i;
            wv[i] = *reinterpret_cast<const float4 *>(wr + ((k0 < a.H) ? k0 : 0));
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if (tid * 4 + 1024 * i >= a.H)
                wv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int m = 0; m < T; ++m) {
            uint2 xv[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int k0 = tid * 4 + 1024 * i;
                xv[i] = *reinterpret_cast<const uint2 *>(a.x + (size_t)m * a.H + ((k0 < a.H) ? k0 : 0));
            }
#pragma unroll
            for (int i = 0; i < NI; ++i)
                if (tid * 4 + 1024 * i >= a.H)
                    xv[i] = make_uint2(0u, 0u);
            double acc = 0.0;
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const float x0 = bf16_to_f32(xv[i].x & 0xffffu), x1 = bf16_to_f32(xv[i].x >> 16);
                const float x2 = bf16_to_f32(xv[i].y & 0xffffu), x3 = bf16_to_f32(xv[i].y >> 16);
                acc = fma((double)x0, (double)wv[i].x, acc);
                acc = fma((double)x1, (double)wv[i].y, acc);
                acc = fma((double)x2, (double)wv[i].z, acc);
                acc = fma((double)x3, (double)wv[i].w, acc);
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3))));
            }
            if (m == 0) {
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    xq_v[i] = xv[i];
            }
            const double v = wave_sum_d(acc);
            const float am = wave_max(amax);
            if (lane == 0) {
                sred[wave][m] = v;
                samax[wave][m] = am;
            }
        }
        __syncthreads();
        if (tid < T)
            store_dev(a.logits + (size_t)tid * a.E + e,
                      (sred[0][tid] + sred[1][tid]) + (sred[2][tid] + sred[3][tid]));
        const bool last = block_arrives_last(a.done, gridDim.x, &s_last);
        if (!last) {
            // every block saw all of x: the blocks share its quantisation
            if (spread_quant)
                quant_share(a, xq_v, samax);
            return;
        }
    }
    // ---- the last (or only) block ----
    if ((a.flags & RS_SEL) && !(a.flags & RS_ROUTER) && tid < a.k) {
        const int e = a.idx[tid];
        a.sel[tid] = (e >= 0 && e < a.E) ? a.ptrs[e] : nullptr;
    }
    if ((a.flags & RS_QUANT) && !(a.flags & RS_ROUTER)) {
        for (int m = 0; m < T; ++m) {
            const uint16_t *xr = a.x + (size_t)m * a.H;
            float amax = 0.0f;
            for (int i = tid * 8; i < a.H; i += 2048) {
                const uint4 v = *reinterpret_cast<const uint4 *>(xr + i);
                const uint32_t ww[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    amax = fmaxf(amax, fabsf(bf16_to_f32(ww[j] & 0xffffu)));
                    amax = fmaxf(amax, fabsf(bf16_to_f32(ww[j] >> 16)));
                }
            }
            amax = block_max_256(amax, red);
            float inv = 0.0f, sc = 0.0f;
            if (amax > 0.0f) {
                inv = 127.0f / amax;
                sc = amax / 127.0f;
            }
            int8_t *qr = a.xq + (size_t)m * a.H;
            for (int i = tid * 8; i < a.H; i += 2048) {
                const uint4 v = *reinterpret_cast<const uint4 *>(xr + i);
                const uint32_t ww[4] = {v.x, v.y, v.z, v.w};
                uint32_t packed[2] = {0u, 0u};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float xv = bf16_to_f32((j & 1) ? (ww[j >> 1] >> 16) : (ww[j >> 1] & 0xffffu));
                    const float rr = fminf(fmaxf(rintf(xv * inv), -127.0f), 127.0f);
                    packed[j >> 2] |= ((uint32_t)(int)rr & 0xffu) << (8 * (j & 3));
                }
                *reinterpret_cast<uint2 *>(qr + i) = make_uint2(packed[0], packed[1]);
            }
            if (tid == 0)
                a.sa[m] = sc;
        }
    }
    if (a.flags & RS_ROUTER) {
        for (int m = 0; m < T; ++m) {
            if (a.E <= 256)
                topk_sort_block(a.logits + (size_t)m * a.E, a.bias, a.E, a.k, a.r,
                                a.idx + (size_t)m * a.k, a.w + (size_t)m * a.k, s_idx + m * a.k,
                                s_s, cand_c, cand_i, sel_s);
            else
                topk_rank_block(a.logits + (size_t)m * a.E, a.bias, a.E, a.k, a.r,
                                a.idx + (size_t)m * a.k, a.w + (size_t)m * a.k, s_idx + m * a.k,
                                s_c, s_s, sel_s);
        }
        if (spread_quant)
            quant_share(a, xq_v, samax);
        if (tid == 0)
            *a.done = 0u;
    } else if (a.flags & RS_LISTS) {
        for (int j = tid; j < T * a.k; j += 256)
            s_idx[j] = a.idx[j];
        __syncthreads();
    }
    if (!(a.flags & RS_LISTS))
        return;
    const int S = a.k + a.n_shared;
    const int nE = a.E + a.n_shared;
    for (int e = tid; e < nE; e += 256)
        a.cnt[e] = 0;
    if (tid < 33)
        s_bits[tid] = 0u;
    __syncthreads();
    const int N = T * a.k;
    for (int j = tid; j < N; j += 256) {
        const int e = s_idx[j];
        if (e < 0 || e >= a.E)
            continue;
        int pos = 0;
        bool last = true;
        for (int jj = 0; jj < N; ++jj) {
            if (s_idx[jj] == e) {
                if (jj < j)
                    ++pos;
                else if (jj > j)
                    last = false;
            }
        }
        if (pos < a.list_stride)
            a.list[(size_t)e * a.list_stride + pos] = (j / a.k) * S + (j % a.k);
        if (last)
            a.cnt[e] = pos + 1 < a.list_stride ? pos + 1 : a.list_stride;
        atomicOr(&s_bits[e >> 5], 1u << (e & 31));
    }
    if (a.n_shared) {
        for (int m = tid; m < T; m += 256)
            a.list[(size_t)a.E * a.list_stride + m] = m * S + a.k;
        if (tid == 0) {
            a.cnt[a.E] = T;
            atomicOr(&s_bits[a.E >> 5], 1u << (a.E & 31));
        }
    }
    __syncthreads();
    if (wave == 0) {
        const uint32_t bits = lane < 33 ? s_bits[lane] : 0u;
        const int nb = __popc(bits);
        int pre = nb;                            // inclusive prefix over lanes
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(pre, o, 64);
            if (lane >= o)
                pre += v;
        }
        int pos = pre - nb;
        for (int b = 0; b < 32; ++b)
            if ((bits >> b) & 1u)
                a.active[pos++] = lane * 32 + b;
        if (lane == 63)
            *a.n_active = pre;
    }
}

// ---------------------------------------------------------------------------
// One token, first of the two router launches (E <= 256, H <= 8192): block e
// computes the fp64 logit of expert e (same slices and reduction order as
// route_small_kernel) and codes its share of the token (quant_share).  The
// top-k launch turns the logits into scores, all experts at once (the fp64
// sigmoid in one thread per block here would delay this launch's end).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_bs1_kernel(RouteSmallArgs a)
{
    __shared__ double sred[4];
    __shared__ float samax[4][RS_MAXT];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int e = blockIdx.x;
    constexpr int NI = 8;
    float4 wv[NI];
    uint2 xv[NI];
    const float *wr = a.Wr + (size_t)e * a.H;
    // every load is issued before any is used: lanes past H read the row's
    // first inputs and zero them afterwards (a load under the branch let the
    // compiler convert each value as it arrived, one round trip at a time)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int k0 = tid * 4 + 1024 * i;
        const int kc = (k0 < a.H) ? k0 : 0;
        wv[i] = *reinterpret_cast<const float4 *>(wr + kc);
        xv[i] = *reinterpret_cast<const uint2 *>(a.x + kc);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (tid * 4 + 1024 * i >= a.H) {
            wv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            xv[i] = make_uint2(0u, 0u);
        }
    }
    double acc = 0.0;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const float x0 = bf16_to_f32(xv[i].x & 0xffffu), x1 = bf16_to_f32(xv[i].x >> 16);
        const float x2 = bf16_to_f32(xv[i].y & 0xffffu), x3 = bf16_to_f32(xv[i].y >> 16);
        acc = fma((double)x0, (double)wv[i].x, acc);
        acc = fma((double)x1, (double)wv[i].y, acc);
        acc = fma((double)x2, (double)wv[i].z, acc);
        acc = fma((double)x3, (double)wv[i].w, acc);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3))));
    }
    const double v = wave_sum_d(acc);
    const float am = wave_max(amax);
    if (lane == 0) {
        sred[wave] = v;
        samax[wave][0] = am;
    }
    __syncthreads();
    if (tid == 0)
        a.logits[e] = (sred[0] + sred[1]) + (sred[2] + sred[3]);
    if (a.flags & RS_QUANT)
        quant_share(a, xv, samax);
}

hipError_t launch_router_bs1(const RouteSmallArgs &a, hipStream_t st)
{
    launch(router_bs1_kernel, a.E, 256, 0, st, a);
    return hipGetLastError();
}

hipError_t launch_route_small(const RouteSmallArgs &a, hipStream_t st)
{
    const int grid = (a.flags & RS_ROUTER) ? a.E : 1;
    launch(route_small_kernel, grid, 256, 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
