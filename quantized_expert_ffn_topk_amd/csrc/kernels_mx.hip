// kernels_mx.hip -- MXFP4 expert FFNs for gfx950: E2M1 weights with one E8M0
// scale per 32 inputs (OCP Microscaling v1.0), bf16 activations, fp32
// accumulation, on the gfx950 MX MFMA v_mfma_scale_f32_16x16x128_f8f6f4.
// MXFP4 experts are the format the AIFP guide ("Step 3") names for the Kimi
// family; the Kongchang page lists the same families.
//
// The MX MFMA takes the weights as they are stored: a lane's B operand is the
// blob's 16 bytes of one weight row and one chunk of 32 inputs (low nibble =
// the even input), with that chunk's E8M0 byte as its scale.  Its other
// operand must be fp8/fp6/fp4, so every bf16 activation row is split once per
// call (split_fp8_kernel) into two OCP E4M3 parts with one E8M0 scale each per
// 32 inputs: hi = RNE(v * 2^-X) with X = floor(log2 amax) - 7 (so |hi| < 256),
// lo = RNE((v * 2^-X - hi) * 2^5), i.e. scale 2^(X-5).  A bf16 value has 8
// significant bits and E4M3 4, so hi + lo reproduces v exactly for every
// element within 2^13 of its block's largest (only smaller ones round); each
// weight chunk then runs two MFMAs, hi and lo, into the same fp32
// accumulator.  The MX MFMA's internal sums are not plain fp32 ones: on the
// test layers its outputs sit up to ~3e-4 of the largest output from the
// exact result.
//
// MOE_PATH_MX_BF16 selects the other kernel: each weight chunk widened in
// registers by v_cvt_scalef32_pk_bf16_fp4 (which applies the chunk's scale, so
// every weight is an exact bf16 value) against the bf16 rows on
// v_mfma_f32_16x16x32_bf16: exact products, fp32 sums (~1e-7 of the largest
// output), no split launches.  Its operands: lane l supplies A row l%16 and B
// column l%16 with k = 8*(l/16) + i, i < 8; result register i of lane l is
// row 4*(l/16) + i, column l%16.
//
// Operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (fp8 A, fp4 B; checked
// on the device): lane l supplies A row l%16 and B column l%16; with g = l/16,
// A bytes 0-15 are inputs [16g, 16g+16) and bytes 16-31 inputs
// [64+16g, 64+16g+16) of the 128, B holds inputs [32g, 32g+32); the scale of
// inputs [32p, 32p+32) of a row (column) comes from lane row + 16p.  Result
// register i of lane l is row 4g + i, column l%16.  A 64-lane load of 16 B per
// lane reads 1 KiB of a weight tile (blob layout [tile][kc][r][16 B]): lane l
// gets row l%16 of chunk c0 + l/16, i.e. exactly its B operand.
//
// Work list: tiles of 16 rows of one expert (mx_tiles); a block covers one row
// tile and 4 TPW weight tiles (4 waves x TPW tiles of 16 rows; TPW = 8 for
// gate/up, 4 or 2 with few row tiles, and 4 for down).
//   gate/up: waves hold the gate and up tiles of TPW/2 row pairs; the epilogue is
//            h = bf16(fp32(G/(1+exp(-G)) * U)) with G, U the fp32 projections;
//            the h rows are split like the activations before the down launch.
//   down   : Y[slot, n] in fp32, combined afterwards by combine_kernel.
#include "device_common.h"
#include "host_common.h"
#include "permute_common.h"

namespace moe {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int MX_MT = 16;          // activation rows per tile

struct MxArgs {
    Experts ex;
    Routing rt;
    // activation rows split into two E4M3 parts [rows][K] and their E8M0
    // scales [rows][K/32] (MX MFMA), or the bf16 rows themselves (bf16 MFMA)
    const uint8_t *a_hi, *a_lo, *e_hi, *e_lo;
    const uint16_t *act;
    int in_by_token;               // 1: row = slot / S (tokens), 0: row = slot
    int K;
    size_t w_off, s_off, tile_w, tile_s;
    int n_wtiles;                  // 16-row weight tiles in the section
    void *out;                     // gate/up: bf16 h [slots][ldo]; down: fp32 Y [slots][ldo]
    int ldo;
};

// ---------------------------------------------------------------------------
// bf16 rows -> two E4M3 parts with E8M0 scales per 32 (see the file header).
// One thread per (row, 32 inputs).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_fp8_group(const uint16_t *__restrict__ x, long i,
                                                uint8_t *__restrict__ hi, uint8_t *__restrict__ lo,
                                                uint8_t *__restrict__ e_hi,
                                                uint8_t *__restrict__ e_lo)
{
    const uint4 *src = reinterpret_cast<const uint4 *>(x + i * 32);
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        v[j] = src[j];
    float f[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[8 * j + 2 * q] = bf16_to_f32(w[q] & 0xffffu);
            f[8 * j + 2 * q + 1] = bf16_to_f32(w[q] >> 16);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j)
        amax = fmaxf(amax, fabsf(f[j]));
    // X = floor(log2 amax) - 7 (the exponent field of amax, or of its
    // normalised value for fp32 subnormals), clamped to the E8M0 range
    int X = 0;
    if (amax > 0.0f) {
        int ex;
        frexpf(amax, &ex);                  // amax = m * 2^ex, m in [0.5, 1)
        X = max(ex - 1 - 7, -127);
    }
    const int Xl = max(X - 5, -127);
    const float to_hi = ldexpf(1.0f, -X), to_lo = ldexpf(1.0f, X - Xl);
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
        const float a0 = f[j] * to_hi, a1 = f[j + 1] * to_hi;        // exact scalings
        const int h2 = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
        const float r0 = (a0 - __builtin_amdgcn_cvt_f32_fp8(h2, 0)) * to_lo;
        const float r1 = (a1 - __builtin_amdgcn_cvt_f32_fp8(h2, 1)) * to_lo;
        const int l2 = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
        const int sh = 16 * ((j >> 1) & 1);
        if (((j >> 1) & 1) == 0) {
            ph[j >> 2] = (uint32_t)h2 & 0xffffu;
            pl[j >> 2] = (uint32_t)l2 & 0xffffu;
        } else {
            ph[j >> 2] |= ((uint32_t)h2 & 0xffffu) << sh;
            pl[j >> 2] |= ((uint32_t)l2 & 0xffffu) << sh;
        }
    }
    uint4 *dh = reinterpret_cast<uint4 *>(hi + i * 32);
    uint4 *dl = reinterpret_cast<uint4 *>(lo + i * 32);
    dh[0] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    dh[1] = make_uint4(ph[4], ph[5], ph[6], ph[7]);
    dl[0] = make_uint4(pl[0], pl[1], pl[2], pl[3]);
    dl[1] = make_uint4(pl[4], pl[5], pl[6], pl[7]);
    e_hi[i] = (uint8_t)(X + 127);
    e_lo[i] = (uint8_t)(Xl + 127);
}

__global__ __launch_bounds__(256) void split_fp8_kernel(const uint16_t *__restrict__ x, int rows,
                                                        int K, uint8_t *__restrict__ hi,
                                                        uint8_t *__restrict__ lo,
                                                        uint8_t *__restrict__ e_hi,
                                                        uint8_t *__restrict__ e_lo)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < (long)rows * (K >> 5))
        split_fp8_group(x, i, hi, lo, e_hi, e_lo);
}

// A few tokens (at most 256 routing entries) in one launch: block 0 runs the
// routing permutation and then the row tile list over the counts it has just
// written (the block barrier makes the block's global writes visible to the
// block), the other blocks split the tokens' bf16 rows (rows = 0 on the
// bf16-MFMA path).  Saves two launches of a decode step.
template <bool BALLOT>
__global__ __launch_bounds__(1024) void mx_prep_small_kernel(
    const int32_t *__restrict__ idx, int T, int k, int E, int n_shared, int32_t *__restrict__ cnt,
    int32_t *__restrict__ list, int list_stride, int32_t *__restrict__ active,
    int32_t *__restrict__ n_active, int mt, int2 *__restrict__ tiles, int32_t *__restrict__ n_tiles,
    const uint16_t *__restrict__ x, int rows, int K, uint8_t *__restrict__ hi,
    uint8_t *__restrict__ lo, uint8_t *__restrict__ e_hi, uint8_t *__restrict__ e_lo)
{
    if (blockIdx.x == 0) {
        if (BALLOT)
            permute_small_ballot_block(idx, T, k, E, n_shared, cnt, list, list_stride, active,
                                       n_active);
        else
            permute_small_block(idx, T, k, E, n_shared, cnt, list, list_stride, active, n_active);
        __syncthreads();
        row_tiles_block(cnt, E + n_shared, mt, tiles, n_tiles);
        return;
    }
    const long i = (long)(blockIdx.x - 1) * 1024 + threadIdx.x;
    if (i < (long)rows * (K >> 5))
        split_fp8_group(x, i, hi, lo, e_hi, e_lo);
}

hipError_t launch_split_fp8(const uint16_t *x, int rows, int K, uint8_t *hi, uint8_t *lo,
                            uint8_t *e_hi, uint8_t *e_lo, hipStream_t st)
{
    const long n = (long)rows * (K >> 5);
    if (n <= 0)
        return hipSuccess;
    launch(split_fp8_kernel, (int)((n + 255) / 256), 256, 0, st, x, rows, K, hi, lo, e_hi, e_lo);
    return hipGetLastError();
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 2^(e-127) as fp32 (e = 0 is the subnormal 2^-127; 255 never reaches here:
// the packer rejects it).
__device__ __forceinline__ float e8m0_scale(uint32_t e)
{
    return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// Eight E2M1 codes (one dword, inputs 8j..8j+7 of a chunk) -> eight exact bf16
// values times the chunk scale (v_cvt_scalef32_pk_bf16_fp4).
__device__ __forceinline__ bf16x8 widen8(uint32_t d, float sc)
{
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3);
    bf16x8 r;
    r[0] = p0[0];
    r[1] = p0[1];
    r[2] = p1[0];
    r[3] = p1[1];
    r[4] = p2[0];
    r[5] = p2[1];
    r[6] = p3[0];
    r[7] = p3[1];
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ v8i_t as_v8(uint4 a, uint4 b)
{
    v8i_t r;
    r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
    r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
    return r;
}

// Block -> (weight group nb, row tile mt), each XCD walking a contiguous run
// of row tiles of one weight group (grid padded to a multiple of 8).
__device__ __forceinline__ void mx_block_coords(int mt_max, int *nb, int *mt)
{
    const int nwg = gridDim.x;
    const int b = blockIdx.x;
    const int logical = (b & 7) * (nwg >> 3) + (b >> 3);
    *nb = logical / mt_max;
    *mt = logical - *nb * mt_max;
}

// MXMMA: the MX MFMA on the split activations; otherwise the weights widened
// to exact bf16 (v_cvt_scalef32_pk_bf16_fp4) against the bf16 rows on
// v_mfma_f32_16x16x32_bf16 (exact products, plain fp32 accumulation).
template <bool GATEUP, int TPW, bool MXMMA, int UNR>
__global__ __launch_bounds__(256) void mx_proj_kernel(MxArgs a, const int2 *__restrict__ tiles,
                                                      const int32_t *__restrict__ n_tiles,
                                                      int mt_max, int n_groups)
{
    int nb, mt;
    mx_block_coords(mt_max, &nb, &mt);
    if (nb >= n_groups || mt >= *n_tiles)
        return;
    const int2 tl = tiles[mt];
    const int e = tl.x, m0 = tl.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int t0 = (nb * 4 + wave) * TPW;         // first weight tile of this wave
    if (t0 >= a.n_wtiles)
        return;
    const int cnt = a.rt.cnt[e];
    const int32_t *lst = a.rt.list + (size_t)e * a.rt.list_stride;
    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);

    // activation row of this lane (A row r of the tile); padding rows use
    // zero codes
    const int m = m0 + r;
    const bool row_ok = m < cnt;
    int slot_r = 0;
    const uint8_t *ahr = nullptr, *alr = nullptr, *ehr = nullptr, *elr = nullptr;
    const uint4 *arow = nullptr;
    if (row_ok) {
        slot_r = lst[m];
        const int row = a.in_by_token ? slot_r / a.rt.S : slot_r;
        if (MXMMA) {
            ahr = a.a_hi + (size_t)row * a.K;
            alr = a.a_lo + (size_t)row * a.K;
            ehr = a.e_hi + (size_t)row * (a.K >> 5);
            elr = a.e_lo + (size_t)row * (a.K >> 5);
        } else {
            arow = reinterpret_cast<const uint4 *>(a.act + (size_t)row * a.K);
        }
    }
    const uint4 *wt[TPW];
    const uint8_t *st[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tt = min(t0 + t, a.n_wtiles - 1);  // clamped: loads stay in bounds
        wt[t] = reinterpret_cast<const uint4 *>(blob + a.w_off + (size_t)tt * a.tile_w) + lane;
        st[t] = blob + a.s_off + (size_t)tt * a.tile_s + (size_t)g * 16 + r;
    }

    f32x4 acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the lane's A bytes 0-15: chunk c0 + g/2, inputs 16 (g%2) ..; bytes
    // 16-31: chunk c0 + 2 + g/2, same inputs; its scale: chunk c0 + g
    const int ao0 = (g >> 1) * 32 + (g & 1) * 16, ao1 = ao0 + 64;
    const int KC = a.K >> 5;
    // UNR steps of 4 chunks per pass, all their weight loads issued first:
    // with few rows (one-token decode) the weight tiles are few and each
    // wave's 1 KiB per step would leave the memory system idle
    for (int cu = 0; cu < KC; cu += 4 * UNR) {
    uint4 wu[UNR][TPW];
    uint32_t su[UNR][TPW];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int c0 = cu + 4 * u;
            wu[u][t] = load_stream16(wt[t] + (size_t)c0 * 16);   // 1 KiB per wave: chunks c0..c0+3, 16 rows
            su[u][t] = st[t][(size_t)c0 * 16];
        }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        const int c0 = cu + 4 * u;
        const uint4 (&w)[TPW] = wu[u];
        const uint32_t (&s8)[TPW] = su[u];
        if (MXMMA) {
            uint4 h0 = {}, h1 = {}, l0 = {}, l1 = {};
            int sh = 127, sl = 127;
            if (row_ok) {
                const size_t kb = (size_t)c0 * 32;
                h0 = *reinterpret_cast<const uint4 *>(ahr + kb + ao0);
                h1 = *reinterpret_cast<const uint4 *>(ahr + kb + ao1);
                l0 = *reinterpret_cast<const uint4 *>(alr + kb + ao0);
                l1 = *reinterpret_cast<const uint4 *>(alr + kb + ao1);
                sh = ehr[c0 + g];
                sl = elr[c0 + g];
            }
            const v8i_t ah = as_v8(h0, h1), al = as_v8(l0, l1);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const v8i_t bw = as_v8(w[t], make_uint4(0u, 0u, 0u, 0u));
                // cbsz 0: A is E4M3; blgp 4: B is E2M1
                acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, bw, acc[t], 0, 4, 0, sh,
                                                                          0, (int)s8[t]);
                acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(al, bw, acc[t], 0, 4, 0, sl,
                                                                          0, (int)s8[t]);
            }
        } else {
            // bf16 16x16x32 MFMA j of the four chunks takes, from lane group
            // g, inputs [8j, 8j+8) of chunk c0 + g (any order of k is exact to
            // sum; each chunk's scale is applied in its conversion)
            uint4 av[4] = {};
            if (row_ok) {
                const uint4 *ap = arow + (size_t)(c0 + g) * 4;   // chunk c0+g: 32 bf16 = 4 x 16 B
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    av[j] = ap[j];
            }
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const float sc = e8m0_scale(s8[t]);
                const uint32_t wd[4] = {w[t].x, w[t].y, w[t].z, w[t].w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[j]),
                                                                     widen8(wd[j], sc), acc[t], 0, 0, 0);
            }
        }
    }
    }

    // result register i: activation row 4g + i of the tile, weight row r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int mm = m0 + 4 * g + i;
        if (mm >= cnt)
            continue;
        const int slot = lst[mm];
        if (GATEUP) {
            uint16_t *hb = reinterpret_cast<uint16_t *>(a.out) + (size_t)slot * a.ldo;
#pragma unroll
            for (int p = 0; p < TPW / 2; ++p) {
                const int b = (t0 >> 1) + p;          // gate tile 2b, up tile 2b+1
                if (2 * b + 1 >= a.n_wtiles)
                    break;
                const double G = (double)acc[2 * p][i], U = (double)acc[2 * p + 1][i];
                const float hv = (float)(G / (1.0 + exp(-G)) * U);
                hb[16 * b + r] = f32_to_bf16(hv);
            }
        } else {
            float *y = reinterpret_cast<float *>(a.out) + (size_t)slot * a.ldo;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
                if (t0 + t < a.n_wtiles)
                    y[16 * (t0 + t) + r] = acc[t][i];
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: routing lists -> 16-row tiles -> gate/up -> down -> combine.
// ---------------------------------------------------------------------------
size_t mx_max_tiles(int T, int E, int n_shared, int S)
{
    // ceil(rows/16) summed over experts <= rows/16 + number of experts
    return (size_t)T * S / MX_MT + 1 + (size_t)E + (size_t)n_shared;
}

static hipError_t launch_mx_prep_small(const int32_t *idx, int T, int k, int E, int n_shared,
                                       moe_ctx *c, int mt, const uint16_t *x, int rows, int K,
                                       hipStream_t st)
{
    const long n = (long)rows * (K >> 5);
    const int grid = 1 + (int)((n + 1023) / 1024);
    const int N = T * k, nE = E + n_shared;
    int2 *tl = reinterpret_cast<int2 *>(c->tiles);
    // the permutation form launch_permute picks for these sizes
    if (((nE + 15) / 16) * ((N + 63) / 64) < N / 4)
        launch(mx_prep_small_kernel<true>, grid, 1024, 0, st, idx, T, k, E, n_shared, c->cnt,
               c->list, c->max_tokens, c->active, c->n_active, mt, tl, c->n_tiles, x, rows, K,
               c->mx_hi, c->mx_lo, c->mx_ehi, c->mx_elo);
    else
        launch(mx_prep_small_kernel<false>, grid, 1024, 0, st, idx, T, k, E, n_shared, c->cnt,
               c->list, c->max_tokens, c->active, c->n_active, mt, tl, c->n_tiles, x, rows, K,
               c->mx_hi, c->mx_lo, c->mx_ehi, c->mx_elo);
    return hipGetLastError();
}

static int grid8(int n)
{
    return (n + 7) & ~7;
}

template <bool GATEUP, int TPW, int UNR>
static hipError_t mx_launch(bool mxmma, int mt_max, int ng, const MxArgs &a, const int2 *tl,
                            const int32_t *n_tiles, hipStream_t st)
{
    const dim3 grid(grid8(mt_max * ng));
    if (mxmma)
        launch(mx_proj_kernel<GATEUP, TPW, true, UNR>, grid, 256, 0, st, a, tl, n_tiles, mt_max, ng);
    else
        launch(mx_proj_kernel<GATEUP, TPW, false, UNR>, grid, 256, 0, st, a, tl, n_tiles, mt_max, ng);
    return hipGetLastError();
}

moe_status mx_ffn_enqueue(moe_ctx *c, const void *x, int T, const moe_layer_weights *w,
                          const void *const *expert_ptrs, const int32_t *idx, const float *gw,
                          void *out, hipStream_t st)
{
    const moe_layer_desc &d = c->d;
    const int H = d.hidden, F = d.ffn, E = d.n_experts, k = d.top_k;
    hipError_t e;
#define MX_LAUNCH(kind, what, expr)                 \
    do {                                            \
        prof_begin(c, (kind), st);                  \
        if ((e = (expr)) != hipSuccess)             \
            return hip_fail(e, what);               \
        prof_end(c, (kind), st);                    \
    } while (0)
    const bool mxmma = c->path != MOE_PATH_MX_BF16;
    // at most 256 routing entries: permutation, tile list and the tokens'
    // split in one launch
    const bool prep = T * k <= 256 && E + d.n_shared <= 1024;
    if (prep) {
        MX_LAUNCH(MOE_PROF_PERMUTE, "permute/tiles/split launch",
                  launch_mx_prep_small(idx, T, k, E, d.n_shared, c, MX_MT,
                                       mxmma ? static_cast<const uint16_t *>(x) : nullptr,
                                       mxmma ? T : 0, H, st));
    } else {
        MX_LAUNCH(MOE_PROF_PERMUTE, "permute launch",
                  launch_permute(idx, T, k, E, d.n_shared, c->cnt, c->list, c->max_tokens,
                                 c->active, c->n_active, c->done, st));
        MX_LAUNCH(MOE_PROF_TILES, "tile list launch", launch_row_tiles(c, MX_MT, st));
    }
    const int mt_max = (T * c->S + MX_MT - 1) / MX_MT + ((T * k < E ? T * k : E) + d.n_shared);

    MxArgs a{};
    a.ex.ptrs = expert_ptrs;
    a.ex.shared = w->shared;
    a.ex.E = E;
    a.rt.active = c->active;
    a.rt.n_active = c->n_active;
    a.rt.cnt = c->cnt;
    a.rt.list = c->list;
    a.rt.list_stride = c->max_tokens;
    a.rt.S = c->S;
    const int2 *tl = reinterpret_cast<const int2 *>(c->tiles);

    // the tokens' bf16 rows split into E4M3 hi/lo parts with E8M0 scales
    if (mxmma && !prep)
        MX_LAUNCH(MOE_PROF_QUANT, "split launch",
                  launch_split_fp8(static_cast<const uint16_t *>(x), T, H, c->mx_hi, c->mx_lo,
                                   c->mx_ehi, c->mx_elo, st));
    // gate/up + SwiGLU -> bf16 h [T*S, F]
    a.act = static_cast<const uint16_t *>(x);
    a.a_hi = c->mx_hi;
    a.a_lo = c->mx_lo;
    a.e_hi = c->mx_ehi;
    a.e_lo = c->mx_elo;
    a.in_by_token = 1;
    a.K = H;
    a.w_off = c->L.gu_w;
    a.s_off = c->L.gu_s;
    a.tile_w = c->L.gu_tile_w;
    a.tile_s = c->L.gu_tile_s;
    a.n_wtiles = F / 8;
    a.out = c->hb;
    a.ldo = F;
    // Weight tiles per wave (TPW) and steps of loads issued ahead (UNR) by the
    // number of row tiles: with few (decode) the waves are few and each
    // holds few bytes in flight, so loads go several steps ahead.  Measured on
    // hidden 7168 / FFN 2048 (routed gate/up of a one-token step 67 -> 39 us,
    // two tokens 70 -> 63 us); from about 3 tokens on, 8 tiles per wave one
    // step ahead is as fast or faster.  Deeper load queues made the down
    // launch slower at every size tried, so it keeps 4 tiles per wave (8 ran
    // ~2 % slower: the down blocks are shorter, K = F).
    const bool ahead = (H >> 5) % 16 == 0;
    {
        const int tpw = (ahead && mt_max <= 12) ? 4 : (ahead && mt_max <= 24) ? 2 : 8;
        const int ng = (a.n_wtiles + 4 * tpw - 1) / (4 * tpw);
        MX_LAUNCH(MOE_PROF_GATEUP, "gate/up launch",
                  (tpw == 4   ? mx_launch<true, 4, 4>(mxmma, mt_max, ng, a, tl, c->n_tiles, st)
                   : tpw == 2 ? mx_launch<true, 2, 4>(mxmma, mt_max, ng, a, tl, c->n_tiles, st)
                              : mx_launch<true, 8, 1>(mxmma, mt_max, ng, a, tl, c->n_tiles, st)));
    }
    // the SwiGLU rows split the same way, then down -> Y [T*S, H]
    if (mxmma)
        MX_LAUNCH(MOE_PROF_REQUANT, "split launch",
                  launch_split_fp8(c->hb, T * c->S, F, c->mx_hi, c->mx_lo, c->mx_ehi, c->mx_elo,
                                   st));
    a.act = c->hb;
    a.in_by_token = 0;
    a.K = F;
    a.w_off = c->L.dn_w;
    a.s_off = c->L.dn_s;
    a.tile_w = c->L.dn_tile_w;
    a.tile_s = c->L.dn_tile_s;
    a.n_wtiles = H / 16;
    a.out = c->Y;
    a.ldo = H;
    {
        const int ng = (a.n_wtiles + 15) / 16;
        MX_LAUNCH(MOE_PROF_DOWN, "down launch",
                  (mx_launch<false, 4, 1>(mxmma, mt_max, ng, a, tl, c->n_tiles, st)));
    }
    MX_LAUNCH(MOE_PROF_COMBINE, "combine launch",
              launch_combine(c->Y, idx, gw, T, k, E, d.n_shared, H, out, d.out_dtype, st));
#undef MX_LAUNCH
    return MOE_OK;
}

}  // namespace moe
