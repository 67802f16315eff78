// kernels_gemv.hip -- int4 x int8 expert projections for few rows per expert
// (decode), SwiGLU, requantisation and the combine, for gfx950.
//
// The integer-dot scheme is the one the Colibri guide describes (table
// "Points techniques cles", integer dot-product row): byte products summed
// exactly in integers.  A weight nibble (4-bit two's complement) masked into the
// top of its byte is the signed byte 16*q, so v_dot4_i32_i8 on those bytes and
// the int8 activations gives 16 x the exact group dot; the factor 16 is folded
// into the fp64 scale (S/16 is exact).
// Each int32 group sum times its fp16 scale is exact in fp64 and so is their
// sum (the packer bounds the scale spread of a row), so the fp64 result does
// not depend on how lanes and waves split the reduction.
//
// Work split: a block (4 waves) owns a pair of 16-row weight tiles of one
// expert; wave w reads tile w>>1, half w&1 of the K chunks.  Lane l owns row
// l&15 and every 4th chunk from l>>4, so one 16-byte load per lane reads 1 KiB
// of contiguous blob (4 chunks x 16 rows).  A wave's first U loads are issued
// before the activation rows are staged in LDS, so the weight stream starts at
// once.
//
// Fused tails (one token where the one-token kernels do not apply): the last
// block to finish an expert's gate/up requantises that expert's SwiGLU rows;
// the last block to finish an output tile of the down projection combines the
// experts for that tile.  "Last" is decided with a device-scope counter that
// the last block resets.  From two tokens on, requant and combine run as
// launches of their own (faster there).
#include "device_common.h"
#include "host_common.h"

namespace moe {

// One batch of U weight loads and their scales; CACHED: plain loads (the
// layer's experts fit the last-level cache and stay there between calls: the
// 16-token tiny layer 188 k -> 195 k tokens/s), else the non-temporal hint
// (the GLM-shaped layer's experts do not fit: plain loads 8-11 % slower).  A
// template parameter, not a runtime flag: both load forms in one kernel
// raised its registers (gate/up 179 VGPRs) and cost a third of the speed.
template <int U, bool CACHED>
__device__ __forceinline__ void load_batch(const uint8_t *__restrict__ wt,
                                           const uint16_t *__restrict__ st, int cb, int it0,
                                           int niter, int c4, int r, int gshift,
                                           uint4 (&wv)[U], uint32_t (&sv)[U])
{
    typedef unsigned int g4 __attribute__((ext_vector_type(4)));
    if constexpr (CACHED) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (it0 + u < niter) {
                const int c = cb + (it0 + u) * 4 + c4;
                const g4 v = *(const __attribute__((address_space(1))) g4 *)(wt + ((size_t)c * 16 + r) * 16);
                wv[u] = make_uint4(v.x, v.y, v.z, v.w);
                sv[u] = *(const __attribute__((address_space(1))) uint16_t *)(st + (size_t)(c >> gshift) * 16 + r);
            }
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (it0 + u < niter) {
            const int c = cb + (it0 + u) * 4 + c4;
            wv[u] = load_stream16(wt + ((size_t)c * 16 + r) * 16);
            sv[u] = load_stream2(st + (size_t)(c >> gshift) * 16 + r);
        }
    }
}

template <int MG, int U>
__device__ __forceinline__ void compute_batch(const uint4 (&wv)[U], const uint32_t (&sv)[U], int cb,
                                              int it0, int niter, int c4, int mc,
                                              const int8_t *__restrict__ lq, int K, double (&p)[MG])
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (it0 + u < niter) {
            const int c = cb + (it0 + u) * 4 + c4;
            const double sd = (double)f16_to_f32((uint16_t)sv[u]) * 0.0625;
            const uint32_t wd[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
            int lo[4], hi[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                lo[d] = (int)((wd[d] << 4) & 0xf0f0f0f0u);
                hi[d] = (int)(wd[d] & 0xf0f0f0f0u);
            }
#pragma unroll
            for (int m = 0; m < MG; ++m) {
                if (m < mc) {
                    const int4 *qa = reinterpret_cast<const int4 *>(lq + m * K + c * 32);
                    const int4 a0 = qa[0], a1 = qa[1];
                    int acc = 0;
                    acc = sdot4(lo[0], a0.x, acc);
                    acc = sdot4(lo[1], a0.y, acc);
                    acc = sdot4(lo[2], a0.z, acc);
                    acc = sdot4(lo[3], a0.w, acc);
                    acc = sdot4(hi[0], a1.x, acc);
                    acc = sdot4(hi[1], a1.y, acc);
                    acc = sdot4(hi[2], a1.z, acc);
                    acc = sdot4(hi[3], a1.w, acc);
                    p[m] = fma((double)acc, sd, p[m]);
                }
            }
        }
    }
}

// Requantises one row of F <= 4096 floats written by other blocks of this
// kernel (store_dev): all of the thread's loads are issued before any is used.
__device__ __forceinline__ void requant_row_dev(const float *__restrict__ hr, int F,
                                                int8_t *__restrict__ qr, float *__restrict__ s_out,
                                                float *red)
{
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int i = threadIdx.x * 4 + 1024 * (j >> 2) + (j & 3);
        v[j] = (i < F) ? load_dev(hr + i) : 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        amax = fmaxf(amax, fabsf(v[j]));
    amax = block_max_256(amax, red);
    float inv = 0.0f, sc = 0.0f;
    if (amax > 0.0f) {
        inv = 127.0f / amax;
        sc = amax / 127.0f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = threadIdx.x * 4 + 1024 * j;
        if (i < F) {
            uint32_t packed = 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float rr = fminf(fmaxf(rintf(v[4 * j + b] * inv), -127.0f), 127.0f);
                packed |= ((uint32_t)(int)rr & 0xffu) << (8 * b);
            }
            *reinterpret_cast<uint32_t *>(qr + i) = packed;
        }
    }
    if (threadIdx.x == 0)
        *s_out = sc;
}

// Stages up to MG activation rows of the expert's list into LDS: the pass's
// slots first (one load per row, all rows at once), then the rows' codes,
// copied global -> LDS by the load unit (global_load_lds_dwordx4: a wave moves
// 1 KiB, lane l's 16 bytes to LDS byte 16 l of the wave's destination) with
// every copy of the pass in flight at once, and the rows' token scales beside
// them: two round trips for the pass, where one row at a time took two per
// row.  Rows whose length is not a multiple of 1 KiB take plain copies.  The
// caller's next barrier publishes lq, lsa and lslot.
template <int MG>
__device__ __forceinline__ void stage_rows(const ProjArgs &a, const int32_t *lst, int base,
                                           int mc, int8_t *lq, float *lsa, int *lslot)
{
    const int K = a.K;
    const int tid = threadIdx.x;
    if (tid < mc)
        lslot[tid] = lst[base + tid];
    __syncthreads();
    float sc = 0.0f;
    if (tid < mc) {
        const int slot = lslot[tid];
        sc = a.s[a.in_by_token ? slot / a.rt.S : slot];
    }
    if ((K & 1023) == 0) {
        const int gpr = K >> 10;                     // 1 KiB pieces per row
        const int wave = tid >> 6, lane = tid & 63;
        int m = 0, g = wave;
        while (m < mc && g >= gpr) {
            g -= gpr;
            ++m;
        }
        for (; m < mc;) {
            const int slot = lslot[m];
            const int row = a.in_by_token ? slot / a.rt.S : slot;
            const int8_t *src = a.q + (size_t)row * K + 1024 * g + 16 * lane;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)src,
                (__attribute__((address_space(3))) void *)(lq + (size_t)m * K + 1024 * g), 16, 0, 0);
            g += 4;
            while (m < mc && g >= gpr) {
                g -= gpr;
                ++m;
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);          // vmcnt(0): the copies have landed
    } else {
        for (int m = 0; m < mc; ++m) {
            const int slot = lslot[m];
            const int row = a.in_by_token ? slot / a.rt.S : slot;
            const uint4 *src = reinterpret_cast<const uint4 *>(a.q + (size_t)row * K);
            uint4 *dst = reinterpret_cast<uint4 *>(lq + m * K);
            for (int i = tid; i < (K >> 4); i += 256)
                dst[i] = src[i];
        }
    }
    if (tid < mc)
        lsa[tid] = sc;
}

// Exact partial sums of tile pair (wt0, wt1) for all passes of MG rows; calls
// epi(base, mc, part, lsa, lslot) after each pass (part[wave][m][r] in LDS).
template <int MG, int U, bool CACHED, class Epi>
__device__ __forceinline__ void gemv_tile_pair(const ProjArgs &a, const uint8_t *wt0,
                                               const uint8_t *wt1, const uint16_t *st0,
                                               const uint16_t *st1, const int32_t *lst, int n,
                                               unsigned char *smem, Epi epi)
{
    const int K = a.K, KC = K >> 5;
    int8_t *lq = reinterpret_cast<int8_t *>(smem);
    double *part = reinterpret_cast<double *>(smem + MG * K);
    float *lsa = reinterpret_cast<float *>(part + 4 * MG * 16);
    int *lslot = reinterpret_cast<int *>(lsa + MG);

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = wave >> 1, half = wave & 1;
    const uint8_t *wt = j ? wt1 : wt0;
    const uint16_t *st = j ? st1 : st0;
    const int r = lane & 15, c4 = lane >> 4;
    const int nk = KC >> 1;
    const int cb = half * nk;
    const int niter = nk >> 2;

    uint4 wv[U];
    uint32_t sv[U];           // 16-bit scales, one per register: packing two per
                              // register made each load wait for the one before
    load_batch<U, CACHED>(wt, st, cb, 0, niter, c4, r, a.group_shift, wv, sv);   // before staging
    for (int base = 0; base < n; base += MG) {
        const int mc = min(MG, n - base);
        stage_rows<MG>(a, lst, base, mc, lq, lsa, lslot);
        __syncthreads();
        double p[MG];
#pragma unroll
        for (int m = 0; m < MG; ++m)
            p[m] = 0.0;
        for (int it0 = 0; it0 < niter; it0 += U) {
            if (base > 0 || it0 > 0)
                load_batch<U, CACHED>(wt, st, cb, it0, niter, c4, r, a.group_shift, wv, sv);
            compute_batch<MG, U>(wv, sv, cb, it0, niter, c4, mc, lq, K, p);
        }
#pragma unroll
        for (int m = 0; m < MG; ++m) {
            p[m] += xor_lane_d<16>(p[m]);
            p[m] += xor_lane_d<32>(p[m]);
        }
        if (c4 == 0) {
#pragma unroll
            for (int m = 0; m < MG; ++m)
                part[(wave * MG + m) * 16 + r] = p[m];
        }
        __syncthreads();
        epi(base, mc, part, lsa, lslot);
        __syncthreads();
    }
}

// Requantises one row of F floats into int8 with the token-quantisation rule
// (DEV: the row was written by other blocks of this kernel with store_dev).
template <bool DEV>
__device__ __forceinline__ float4 load4(const float *p)
{
    if (DEV)
        return make_float4(load_dev(p), load_dev(p + 1), load_dev(p + 2), load_dev(p + 3));
    return *reinterpret_cast<const float4 *>(p);
}

template <bool DEV>
__device__ __forceinline__ void requant_row(const float *__restrict__ hr, int F,
                                            int8_t *__restrict__ qr, float *__restrict__ s_out,
                                            float *red)
{
    float amax = 0.0f;
    for (int i = threadIdx.x * 4; i < F; i += 1024) {
        const float4 v = load4<DEV>(hr + i);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = block_max_256(amax, red);
    float inv = 0.0f, sc = 0.0f;
    if (amax > 0.0f) {
        inv = 127.0f / amax;
        sc = amax / 127.0f;
    }
    for (int i = threadIdx.x * 4; i < F; i += 1024) {
        const float4 v = load4<DEV>(hr + i);
        const float vv[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float rr = fminf(fmaxf(rintf(vv[j] * inv), -127.0f), 127.0f);
            packed |= ((uint32_t)(int)rr & 0xffu) << (8 * j);
        }
        *reinterpret_cast<uint32_t *>(qr + i) = packed;
    }
    if (threadIdx.x == 0)
        *s_out = sc;
}

// ---------------------------------------------------------------------------
// Gate/up projections fused with SwiGLU.  Block (active expert, n-block b)
// computes G and U for rows [16b, 16b+16) of every row routed to the expert:
//   G, U = exact sum * token scale (fp64),  h = fp32(G/(1+exp(-G)) * U).
// SwiGLU is the reading taken for the experts' activation (the pages do not
// name one; DeepSeek-V3-family experts use it).
// ---------------------------------------------------------------------------
template <int MG, int U, bool TAIL, bool CACHED>
__global__ __launch_bounds__(256) void gateup_gemv_kernel(ProjArgs a, float *__restrict__ h,
                                                          int ldh, TailArgs t)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int ai = blockIdx.x;
    if (ai >= *a.rt.n_active)
        return;
    const int e = a.rt.active[ai];
    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);
    const int b = blockIdx.y;
    const uint8_t *wt0 = blob + a.w_off + (size_t)(2 * b) * a.tile_w;
    const uint8_t *wt1 = wt0 + a.tile_w;
    const uint16_t *st0 = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)(2 * b) * a.tile_s);
    const uint16_t *st1 = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)(2 * b + 1) * a.tile_s);
    const int n = a.rt.cnt[e];
    const int32_t *lst = a.rt.list + (size_t)e * a.rt.list_stride;
    gemv_tile_pair<MG, U, CACHED>(a, wt0, wt1, st0, st1, lst, n, smem,
                          [&](int, int mc, const double *part, const float *lsa, const int *lslot) {
                              if (threadIdx.x < 16 * mc) {
                                  const int m = threadIdx.x >> 4, rr = threadIdx.x & 15;
                                  const double sa = (double)lsa[m];
                                  const double G = (part[(0 * MG + m) * 16 + rr] + part[(1 * MG + m) * 16 + rr]) * sa;
                                  const double Uv = (part[(2 * MG + m) * 16 + rr] + part[(3 * MG + m) * 16 + rr]) * sa;
                                  const double silu = G / (1.0 + exp(-G));
                                  float *hp = h + (size_t)lslot[m] * ldh + 16 * b + rr;
                                  if (TAIL)
                                      store_dev(hp, (float)(silu * Uv));
                                  else
                                      *hp = (float)(silu * Uv);
                              }
                          });
    if (!TAIL)
        return;
    __shared__ int s_flag;
    __shared__ float red[4];
    if (!block_arrives_last(t.ctr + ai, gridDim.y, &s_flag))
        return;
    for (int m = 0; m < n; ++m) {
        const int slot = lst[m];
        requant_row_dev(h + (size_t)slot * ldh, t.F, t.qh + (size_t)slot * t.F, t.sh + slot, red);
    }
    if (threadIdx.x == 0)
        t.ctr[ai] = 0u;
}

// ---------------------------------------------------------------------------
// Plain projection of a pair of tiles (down projection, or one part of the
// gate/up section): y = fp32(exact sum * row scale) into
// out[slot*ldo + 32*pair + 16*j + r].  With TAIL, the last block of output
// tile `pair` combines: out[t, n] = Y_shared + sum_i w_i * Y_i (fp64, shared
// first then rank order, rounded once).
// ---------------------------------------------------------------------------
template <int MG, int U, bool TAIL, bool CACHED>
__global__ __launch_bounds__(256) void proj_gemv_kernel(ProjArgs a, TailArgs t)
{
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_flag;
    const int ai = blockIdx.x;
    const int n_act = *a.rt.n_active;
    if (ai >= n_act)
        return;
    const int e = a.rt.active[ai];
    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);
    const int p = blockIdx.y;
    const int tile0 = a.tile_base + p * a.pair_stride, tile1 = tile0 + a.j_stride;
    const uint8_t *wt0 = blob + a.w_off + (size_t)tile0 * a.tile_w;
    const uint8_t *wt1 = blob + a.w_off + (size_t)tile1 * a.tile_w;
    const uint16_t *st0 = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)tile0 * a.tile_s);
    const uint16_t *st1 = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)tile1 * a.tile_s);
    const int n = a.rt.cnt[e];
    const int32_t *lst = a.rt.list + (size_t)e * a.rt.list_stride;
    gemv_tile_pair<MG, U, CACHED>(a, wt0, wt1, st0, st1, lst, n, smem,
                          [&](int, int mc, const double *part, const float *lsa, const int *lslot) {
                              if (threadIdx.x < 32 * mc) {
                                  const int m = threadIdx.x >> 5, j = (threadIdx.x >> 4) & 1, rr = threadIdx.x & 15;
                                  const double y = (part[((2 * j) * MG + m) * 16 + rr] + part[((2 * j + 1) * MG + m) * 16 + rr]) *
                                                   (double)lsa[m];
                                  float *yp = a.out + (size_t)lslot[m] * a.ldo + 32 * p + 16 * j + rr;
                                  if (TAIL)
                                      store_dev(yp, (float)y);
                                  else
                                      *yp = (float)y;
                              }
                          });
    if (!TAIL)
        return;
    if (!block_arrives_last(t.ctr + p, (uint32_t)n_act, &s_flag))
        return;
    const int S = t.k + t.n_shared;
    for (int q = threadIdx.x; q < t.T * 32; q += 256) {
        const int tok = q >> 5, col = 32 * p + (q & 31);
        const float *yt = a.out + (size_t)tok * S * t.H;
        float y[17];
#pragma unroll
        for (int i = 0; i < 17; ++i)               // all loads in flight at once
            if (i < S)
                y[i] = load_dev(yt + (size_t)i * t.H + col);
        double o = t.n_shared ? (double)y[t.k] : 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < t.k) {
                const int ex = t.idx[(size_t)tok * t.k + i];
                if (ex >= 0 && ex < t.E)
                    o = fma((double)t.w[(size_t)tok * t.k + i], (double)y[i], o);
            }
        }
        const float f = (float)o;
        if (t.out_dtype == MOE_DT_BF16)
            reinterpret_cast<uint16_t *>(t.out)[(size_t)tok * t.H + col] = f32_to_bf16(f);
        else
            reinterpret_cast<float *>(t.out)[(size_t)tok * t.H + col] = f;
    }
    if (threadIdx.x == 0)
        t.ctr[p] = 0u;
}

static size_t lds_bytes(int mg, int K)
{
    return (size_t)mg * K + 4 * (size_t)mg * 16 * 8 + (size_t)mg * 8;
}

static int pick_mg(int mg, int K)
{
    while (mg > 1 && lds_bytes(mg, K) > 65536)
        mg >>= 1;
    return mg;
}

// Loads per lane per batch: 12 measured best on the GLM-shaped decode layer
// (24: fewer, larger batches oversubscribe HBM; 8: too few).  Gate/up never
// takes more than a wave has (niter = K/256: unused load registers only cost
// waves; hidden 2048: 39 against 44.5 us on the 16-token tiny layer).  The
// plain projection takes 8 for K <= 2048 only with 4 or more rows per pass
// (4-16 tokens: 1-5 % faster; with 1-2 rows per pass 8 measured 38 % slower).
template <int MG, bool TAIL, bool CACHED>
static void launch_gateup_uc(const ProjArgs &a, dim3 grid, size_t lds, float *h, int ldh,
                             const TailArgs &t, int niter, hipStream_t st)
{
    if (niter <= 4)
        launch(gateup_gemv_kernel<MG, 4, TAIL, CACHED>, grid, 256, lds, st, a, h, ldh, t);
    else if (niter <= 8)
        launch(gateup_gemv_kernel<MG, 8, TAIL, CACHED>, grid, 256, lds, st, a, h, ldh, t);
    else
        launch(gateup_gemv_kernel<MG, 12, TAIL, CACHED>, grid, 256, lds, st, a, h, ldh, t);
}

template <int MG, bool TAIL>
static void launch_gateup_u(const ProjArgs &a, dim3 grid, size_t lds, float *h, int ldh,
                            const TailArgs &t, int niter, hipStream_t st)
{
    if (a.cached)
        launch_gateup_uc<MG, TAIL, true>(a, grid, lds, h, ldh, t, niter, st);
    else
        launch_gateup_uc<MG, TAIL, false>(a, grid, lds, h, ldh, t, niter, st);
}

template <int MG, bool TAIL, bool CACHED>
static void launch_proj_uc(const ProjArgs &a, dim3 grid, size_t lds, const TailArgs &t, int niter,
                           hipStream_t st)
{
    if (MG >= 4 && niter <= 8)
        launch(proj_gemv_kernel<MG, 8, TAIL, CACHED>, grid, 256, lds, st, a, t);
    else
        launch(proj_gemv_kernel<MG, 12, TAIL, CACHED>, grid, 256, lds, st, a, t);
}

template <int MG, bool TAIL>
static void launch_proj_u(const ProjArgs &a, dim3 grid, size_t lds, const TailArgs &t, int niter,
                          hipStream_t st)
{
    if (a.cached)
        launch_proj_uc<MG, TAIL, true>(a, grid, lds, t, niter, st);
    else
        launch_proj_uc<MG, TAIL, false>(a, grid, lds, t, niter, st);
}

hipError_t launch_gateup_gemv(const ProjArgs &a, int max_active, int F, int mg, float *h, int ldh,
                              const TailArgs *tail, hipStream_t st)
{
    mg = pick_mg(mg, a.K);
    const dim3 grid(max_active, F / 16);
    const size_t lds = lds_bytes(mg, a.K);
    const int niter = a.K / 256;
    TailArgs t = tail ? *tail : TailArgs{};
    const bool fuse = tail != nullptr;
#define GU(M)                                                              \
    (fuse ? launch_gateup_u<M, true>(a, grid, lds, h, ldh, t, niter, st)   \
          : launch_gateup_u<M, false>(a, grid, lds, h, ldh, t, niter, st))
    switch (mg) {
    case 1: GU(1); break;
    case 2: GU(2); break;
    case 4: GU(4); break;
    default: GU(8); break;
    }
#undef GU
    return hipGetLastError();
}

hipError_t launch_proj_gemv(const ProjArgs &a, int max_active, int n_pairs, int mg,
                            const TailArgs *tail, hipStream_t st)
{
    mg = pick_mg(mg, a.K);
    const dim3 grid(max_active, n_pairs);
    const size_t lds = lds_bytes(mg, a.K);
    const int niter = a.K / 256;
    TailArgs t = tail ? *tail : TailArgs{};
    const bool fuse = tail != nullptr;
#define PJ(M) (fuse ? launch_proj_u<M, true>(a, grid, lds, t, niter, st) \
                    : launch_proj_u<M, false>(a, grid, lds, t, niter, st))
    switch (mg) {
    case 1: PJ(1); break;
    case 2: PJ(2); break;
    case 4: PJ(4); break;
    default: PJ(8); break;
    }
#undef PJ
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Requantisation of each SwiGLU row (one per token and expert) to int8, same
// rule as the token quantisation (many-token path).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void requant_kernel(const float *__restrict__ h, int F,
                                                      int8_t *__restrict__ q,
                                                      float *__restrict__ s)
{
    __shared__ float red[4];
    const int row = blockIdx.x;
    const float *hr = h + (size_t)row * F;
    if (F > 4096) {
        requant_row<false>(hr, F, q + (size_t)row * F, s + row, red);
        return;
    }
    // up to 4096 values: every load of the thread in flight at once, the
    // row read once
    float4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = threadIdx.x * 4 + 1024 * j;
        v[j] = (i < F) ? *reinterpret_cast<const float4 *>(hr + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    amax = block_max_256(amax, red);
    float inv = 0.0f, sc = 0.0f;
    if (amax > 0.0f) {
        inv = 127.0f / amax;
        sc = amax / 127.0f;
    }
    int8_t *qr = q + (size_t)row * F;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = threadIdx.x * 4 + 1024 * j;
        if (i < F) {
            const float vv[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
            uint32_t packed = 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float rr = fminf(fmaxf(rintf(vv[b] * inv), -127.0f), 127.0f);
                packed |= ((uint32_t)(int)rr & 0xffu) << (8 * b);
            }
            *reinterpret_cast<uint32_t *>(qr + i) = packed;
        }
    }
    if (threadIdx.x == 0)
        s[row] = sc;
}

hipError_t launch_requant(const float *h, int rows, int F, int8_t *q, float *s, hipStream_t st)
{
    if (rows <= 0)
        return hipSuccess;
    launch(requant_kernel, rows, 256, 0, st, h, F, q, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine (many-token path): out[t,n] = Y_shared + sum_i w_i * Y_i in fp64,
// shared first then rank order, rounded once (fp32, or bf16 from that fp32).
// A thread owns one output and issues the loads of all S slots before the
// first sum (S = k + n_shared <= SMAX; slots past S reload slot S-1), so each
// wave keeps 9 coalesced 256-byte loads in flight instead of one at a time
// (about 1.7x faster on the 4096-token layer).  Wider vectors per thread
// (2 or 4 outputs) measured slower.  Y is read once: non-temporal loads.
// ---------------------------------------------------------------------------
template <int SMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ Y,
                                                      const int32_t *__restrict__ idx,
                                                      const float *__restrict__ w, int k, int E,
                                                      int n_shared, int H, void *__restrict__ out,
                                                      int out_dtype)
{
    const int t = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= H)
        return;
    const int S = k + n_shared;
    const float *yt = Y + (size_t)t * S * H + n;
    float y[SMAX];
#pragma unroll
    for (int i = 0; i < SMAX; ++i)
        y[i] = __builtin_nontemporal_load(yt + (size_t)min(i, S - 1) * H);
    double o = n_shared ? (double)y[k] : 0.0;
#pragma unroll
    for (int i = 0; i < SMAX; ++i) {
        if (i < k) {
            const int e = idx[(size_t)t * k + i];
            if (e >= 0 && e < E)
                o = fma((double)w[(size_t)t * k + i], (double)y[i], o);
        }
    }
    const float f = (float)o;
    if (out_dtype == MOE_DT_BF16)
        reinterpret_cast<uint16_t *>(out)[(size_t)t * H + n] = f32_to_bf16(f);
    else
        reinterpret_cast<float *>(out)[(size_t)t * H + n] = f;
}

hipError_t launch_combine(const float *Y, const int32_t *idx, const float *w, int T, int k, int E,
                          int n_shared, int H, void *out, int out_dtype, hipStream_t st)
{
    if (T <= 0)
        return hipSuccess;
    dim3 grid((H + 255) / 256, T);
    if (k + n_shared <= 9)
        launch(combine_kernel<9>, grid, 256, 0, st, Y, idx, w, k, E, n_shared, H, out, out_dtype);
    else if (k + n_shared <= 17)
        launch(combine_kernel<17>, grid, 256, 0, st, Y, idx, w, k, E, n_shared, H, out, out_dtype);
    else
        launch(combine_kernel<33>, grid, 256, 0, st, Y, idx, w, k, E, n_shared, H, out, out_dtype);
    return hipGetLastError();
}

}  // namespace moe
