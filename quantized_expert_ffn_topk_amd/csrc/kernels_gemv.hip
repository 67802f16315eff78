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
#include "device_common.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Exact partial sums of a pair of 16-row tiles for up to MG activation rows.
// Wave w handles tile w>>1 and half w&1 of the K chunks.  Lane l owns row
// l&15 and every 4th chunk starting at l>>4, so one 16-byte load per lane
// reads 1 KiB of contiguous blob (4 chunks x 16 rows).  Results go to
// part[wave][m][r] in LDS.
// ---------------------------------------------------------------------------
template <int MG>
__device__ __forceinline__ void tile_pair_partials(const uint8_t *__restrict__ wt0,
                                                   const uint8_t *__restrict__ wt1,
                                                   const uint16_t *__restrict__ st0,
                                                   const uint16_t *__restrict__ st1, int KC,
                                                   int gshift, int mc,
                                                   const int8_t *__restrict__ lq, int K,
                                                   double *__restrict__ part)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = wave >> 1, half = wave & 1;
    const uint8_t *wt = j ? wt1 : wt0;
    const uint16_t *st = j ? st1 : st0;
    const int r = lane & 15, c4 = lane >> 4;
    const int nk = KC >> 1;
    const int cb = half * nk;
    const int niter = nk >> 2;
    double p[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m)
        p[m] = 0.0;
    constexpr int U = 8;
    for (int it0 = 0; it0 < niter; it0 += U) {
        uint4 wv[U];
        uint16_t sv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (it0 + u < niter) {
                int c = cb + (it0 + u) * 4 + c4;
                wv[u] = *reinterpret_cast<const uint4 *>(wt + ((size_t)c * 16 + r) * 16);
                sv[u] = st[(size_t)(c >> gshift) * 16 + r];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (it0 + u < niter) {
                int c = cb + (it0 + u) * 4 + c4;
                double sd = (double)f16_to_f32(sv[u]) * 0.0625;
                uint32_t wd[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
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
                        int4 a0 = qa[0], a1 = qa[1];
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
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        p[m] += shfl_xor_d(p[m], 16);
        p[m] += shfl_xor_d(p[m], 32);
    }
    if (c4 == 0) {
#pragma unroll
        for (int m = 0; m < MG; ++m)
            part[(wave * MG + m) * 16 + r] = p[m];
    }
}

template <int MG>
__device__ __forceinline__ size_t gemv_lds_bytes(int K)
{
    return (size_t)MG * K + 4 * MG * 16 * 8 + MG * 8;
}

// Stages up to MG activation rows of the expert's list into LDS.
template <int MG>
__device__ __forceinline__ void stage_rows(const ProjArgs &a, const int32_t *lst, int base,
                                           int mc, int8_t *lq, float *lsa, int *lslot)
{
    const int K = a.K;
    for (int m = 0; m < mc; ++m) {
        int slot = lst[base + m];
        int row = a.in_by_token ? slot / a.rt.S : slot;
        const uint4 *src = reinterpret_cast<const uint4 *>(a.q + (size_t)row * K);
        uint4 *dst = reinterpret_cast<uint4 *>(lq + m * K);
        for (int i = threadIdx.x; i < K / 16; i += 256)
            dst[i] = src[i];
        if (threadIdx.x == 0) {
            lsa[m] = a.s[row];
            lslot[m] = slot;
        }
    }
}

// ---------------------------------------------------------------------------
// Gate/up projections fused with SwiGLU.  Block (active expert, n-block b)
// computes G and U for rows [16b, 16b+16) of every row routed to the expert:
//   G, U = exact sum * token scale (fp64),  h = fp32(G/(1+exp(-G)) * U).
// SwiGLU is the reading taken for the experts' activation (the pages do not
// name one; DeepSeek-V3-family experts use it).
// ---------------------------------------------------------------------------
template <int MG>
__global__ __launch_bounds__(256) void gateup_gemv_kernel(ProjArgs a, float *__restrict__ h,
                                                          int ldh)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int ai = blockIdx.x;
    if (ai >= *a.rt.n_active)
        return;
    const int e = a.rt.active[ai];
    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);
    const int b = blockIdx.y;
    const int K = a.K, KC = K >> 5;
    const uint8_t *wt0 = blob + a.w_off + (size_t)(2 * b) * a.tile_w;
    const uint8_t *wt1 = wt0 + a.tile_w;
    const uint16_t *st0 =
        reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)(2 * b) * a.tile_s);
    const uint16_t *st1 = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)(2 * b + 1) * a.tile_s);
    int8_t *lq = reinterpret_cast<int8_t *>(smem);
    double *part = reinterpret_cast<double *>(smem + MG * K);
    float *lsa = reinterpret_cast<float *>(part + 4 * MG * 16);
    int *lslot = reinterpret_cast<int *>(lsa + MG);
    const int n = a.rt.cnt[e];
    const int32_t *lst = a.rt.list + (size_t)e * a.rt.list_stride;
    for (int base = 0; base < n; base += MG) {
        const int mc = min(MG, n - base);
        stage_rows<MG>(a, lst, base, mc, lq, lsa, lslot);
        __syncthreads();
        tile_pair_partials<MG>(wt0, wt1, st0, st1, KC, a.group_shift, mc, lq, K, part);
        __syncthreads();
        if (threadIdx.x < 16 * mc) {
            const int m = threadIdx.x >> 4, rr = threadIdx.x & 15;
            const double sa = (double)lsa[m];
            double G = (part[(0 * MG + m) * 16 + rr] + part[(1 * MG + m) * 16 + rr]) * sa;
            double U = (part[(2 * MG + m) * 16 + rr] + part[(3 * MG + m) * 16 + rr]) * sa;
            double silu = G / (1.0 + exp(-G));
            h[(size_t)lslot[m] * ldh + 16 * b + rr] = (float)(silu * U);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Plain projection of a pair of tiles (down projection, or one part of the
// gate/up section): y = fp32(exact sum * row scale) into
// out[slot*ldo + 32*pair + 16*j + r].
// ---------------------------------------------------------------------------
template <int MG>
__global__ __launch_bounds__(256) void proj_gemv_kernel(ProjArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int ai = blockIdx.x;
    if (ai >= *a.rt.n_active)
        return;
    const int e = a.rt.active[ai];
    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);
    const int p = blockIdx.y;
    const int K = a.K, KC = K >> 5;
    const int tile0 = a.tile_base + p * a.pair_stride, tile1 = tile0 + a.j_stride;
    const uint8_t *wt0 = blob + a.w_off + (size_t)tile0 * a.tile_w;
    const uint8_t *wt1 = blob + a.w_off + (size_t)tile1 * a.tile_w;
    const uint16_t *st0 = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)tile0 * a.tile_s);
    const uint16_t *st1 = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)tile1 * a.tile_s);
    int8_t *lq = reinterpret_cast<int8_t *>(smem);
    double *part = reinterpret_cast<double *>(smem + MG * K);
    float *lsa = reinterpret_cast<float *>(part + 4 * MG * 16);
    int *lslot = reinterpret_cast<int *>(lsa + MG);
    const int n = a.rt.cnt[e];
    const int32_t *lst = a.rt.list + (size_t)e * a.rt.list_stride;
    for (int base = 0; base < n; base += MG) {
        const int mc = min(MG, n - base);
        stage_rows<MG>(a, lst, base, mc, lq, lsa, lslot);
        __syncthreads();
        tile_pair_partials<MG>(wt0, wt1, st0, st1, KC, a.group_shift, mc, lq, K, part);
        __syncthreads();
        if (threadIdx.x < 32 * mc) {
            const int m = threadIdx.x >> 5, j = (threadIdx.x >> 4) & 1, rr = threadIdx.x & 15;
            double y = (part[((2 * j) * MG + m) * 16 + rr] + part[((2 * j + 1) * MG + m) * 16 + rr]) *
                       (double)lsa[m];
            a.out[(size_t)lslot[m] * a.ldo + 32 * p + 16 * j + rr] = (float)y;
        }
        __syncthreads();
    }
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

hipError_t launch_gateup_gemv(const ProjArgs &a, int max_active, int F, int mg, float *h,
                              int ldh, hipStream_t st)
{
    mg = pick_mg(mg, a.K);
    dim3 grid(max_active, F / 16);
    size_t lds = lds_bytes(mg, a.K);
    switch (mg) {
    case 1: gateup_gemv_kernel<1><<<grid, 256, lds, st>>>(a, h, ldh); break;
    case 2: gateup_gemv_kernel<2><<<grid, 256, lds, st>>>(a, h, ldh); break;
    case 4: gateup_gemv_kernel<4><<<grid, 256, lds, st>>>(a, h, ldh); break;
    default: gateup_gemv_kernel<8><<<grid, 256, lds, st>>>(a, h, ldh); break;
    }
    return hipGetLastError();
}

hipError_t launch_proj_gemv(const ProjArgs &a, int max_active, int n_pairs, int mg,
                            hipStream_t st)
{
    mg = pick_mg(mg, a.K);
    dim3 grid(max_active, n_pairs);
    size_t lds = lds_bytes(mg, a.K);
    switch (mg) {
    case 1: proj_gemv_kernel<1><<<grid, 256, lds, st>>>(a); break;
    case 2: proj_gemv_kernel<2><<<grid, 256, lds, st>>>(a); break;
    case 4: proj_gemv_kernel<4><<<grid, 256, lds, st>>>(a); break;
    default: proj_gemv_kernel<8><<<grid, 256, lds, st>>>(a); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Requantisation of each SwiGLU row (one per token and expert) to int8, same
// rule as the token quantisation.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void requant_kernel(const float *__restrict__ h, int F,
                                                      int8_t *__restrict__ q,
                                                      float *__restrict__ s)
{
    __shared__ float red[4];
    const int row = blockIdx.x;
    const float *hr = h + (size_t)row * F;
    float amax = 0.0f;
    for (int i = threadIdx.x * 4; i < F; i += 1024) {
        float4 v = *reinterpret_cast<const float4 *>(hr + i);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = block_max_256(amax, red);
    float inv = 0.0f, sc = 0.0f;
    if (amax > 0.0f) {
        inv = 127.0f / amax;
        sc = amax / 127.0f;
    }
    int8_t *qr = q + (size_t)row * F;
    for (int i = threadIdx.x * 8; i < F; i += 2048) {
        float4 v0 = *reinterpret_cast<const float4 *>(hr + i);
        float4 v1 = *reinterpret_cast<const float4 *>(hr + i + 4);
        float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float r = rintf(vv[j] * inv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            int qi = (int)r;
            packed[j >> 2] |= ((uint32_t)qi & 0xffu) << (8 * (j & 3));
        }
        *reinterpret_cast<uint2 *>(qr + i) = make_uint2(packed[0], packed[1]);
    }
    if (threadIdx.x == 0)
        s[row] = sc;
}

hipError_t launch_requant(const float *h, int rows, int F, int8_t *q, float *s, hipStream_t st)
{
    if (rows <= 0)
        return hipSuccess;
    requant_kernel<<<rows, 256, 0, st>>>(h, F, q, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: out[t,n] = Y_shared + sum_i w_i * Y_i in fp64, shared first then
// rank order, rounded once (fp32, or bf16 from that fp32).
// ---------------------------------------------------------------------------
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
    const float *yt = Y + (size_t)t * S * H;
    double o = n_shared ? (double)yt[(size_t)k * H + n] : 0.0;
    for (int i = 0; i < k; ++i) {
        int e = idx[(size_t)t * k + i];
        if (e >= 0 && e < E)
            o = fma((double)w[(size_t)t * k + i], (double)yt[(size_t)i * H + n], o);
    }
    float f = (float)o;
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
    combine_kernel<<<grid, 256, 0, st>>>(Y, idx, w, k, E, n_shared, H, out, out_dtype);
    return hipGetLastError();
}

}  // namespace moe
