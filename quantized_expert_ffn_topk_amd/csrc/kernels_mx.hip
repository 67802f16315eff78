// kernels_mx.hip -- MXFP4 expert FFNs for gfx950: E2M1 weights with one E8M0
// scale per 32 inputs (OCP Microscaling v1.0), bf16 activations, fp32
// accumulation.  MXFP4 experts are the format the AIFP guide ("Step 3") names
// for the Kimi family; the Kongchang page lists the same families.
//
// Each weight chunk (32 E2M1 codes of one row, 16 bytes) is widened in
// registers by the gfx950 MX conversion instruction v_cvt_scalef32_pk_bf16_fp4,
// which also applies the chunk's power-of-two scale, so every weight becomes an
// exact bf16 value; the products with the bf16 activations then run on
// v_mfma_f32_16x16x32_bf16 (exact products, fp32 accumulation).  The MX MFMA
// (v_mfma_scale_f32_*_f8f6f4) would take the fp4 codes as they are, but it needs
// the activations in fp8/fp6/fp4 as well, which would round the bf16 inputs.
//
// MFMA operands (checked on the device): lane l supplies A row l%16 and B
// column l%16 with k = 8*(l/16) + i, i < 8; result register i of lane l is row
// 4*(l/16) + i, column l%16.  A 64-lane load of 16 B per lane reads 1 KiB of a
// weight tile (blob layout [tile][kc][r][16 B]): lane l gets row l%16 of chunk
// c0 + l/16.  Because the sum over k may be taken in any order, MFMA j of a
// group of four chunks takes, from lane group g, the inputs [8j, 8j+8) of chunk
// c0 + g; the activation operand follows the same assignment.  Scales differ
// per chunk and are applied in the conversion, so mixing chunks is exact.
//
// Work list: tiles of 16 rows of one expert (mx_tiles); a block covers one row
// tile and 4 TPW weight tiles (4 waves x TPW tiles of 16 rows; TPW = 8 for
// gate/up, 4 for down).
//   gate/up: waves hold the gate and up tiles of TPW/2 row pairs; the epilogue is
//            h = bf16(fp32(G/(1+exp(-G)) * U)) with G, U the fp32 projections.
//   down   : Y[slot, n] in fp32, combined afterwards by combine_kernel.
#include "device_common.h"
#include "host_common.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int MX_MT = 16;          // activation rows per tile

struct MxArgs {
    Experts ex;
    Routing rt;
    const uint16_t *act;           // bf16 activation rows
    int in_by_token;               // 1: row = slot / S (tokens), 0: row = slot
    int K;
    size_t w_off, s_off, tile_w, tile_s;
    int n_wtiles;                  // 16-row weight tiles in the section
    void *out;                     // gate/up: bf16 h [slots][ldo]; down: fp32 Y [slots][ldo]
    int ldo;
};

// 2^(e-127) as fp32 (e = 0 is the subnormal 2^-127; 255 never reaches here:
// the packer rejects it).
__device__ __forceinline__ float e8m0_scale(uint32_t e)
{
    return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// Eight E2M1 codes (one dword, inputs 8j..8j+7 of a chunk) -> eight exact bf16
// values times the chunk scale.
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

template <bool GATEUP, int TPW>
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

    // activation row of this lane (A row r of the tile); padding rows read 0
    const int m = m0 + r;
    const bool row_ok = m < cnt;
    int slot_r = 0;
    const uint4 *arow = nullptr;
    if (row_ok) {
        slot_r = lst[m];
        const int row = a.in_by_token ? slot_r / a.rt.S : slot_r;
        arow = reinterpret_cast<const uint4 *>(a.act + (size_t)row * a.K);
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

    const int KC = a.K >> 5;
    for (int c0 = 0; c0 < KC; c0 += 4) {
        uint4 w[TPW];
        uint32_t s8[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            w[t] = load_stream16(wt[t] + (size_t)c0 * 16);   // 1 KiB per wave: chunks c0..c0+3, 16 rows
            s8[t] = st[t][(size_t)c0 * 16];
        }
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
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[j]), widen8(wd[j], sc),
                                                                 acc[t], 0, 0, 0);
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

static int grid8(int n)
{
    return (n + 7) & ~7;
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
    MX_LAUNCH(MOE_PROF_PERMUTE, "permute launch",
              launch_permute(idx, T, k, E, d.n_shared, c->cnt, c->list, c->max_tokens, c->active,
                             c->n_active, c->done, st));
    MX_LAUNCH(MOE_PROF_TILES, "tile list launch", launch_row_tiles(c, MX_MT, st));
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

    // gate/up + SwiGLU -> bf16 h [T*S, F]
    a.act = static_cast<const uint16_t *>(x);
    a.in_by_token = 1;
    a.K = H;
    a.w_off = c->L.gu_w;
    a.s_off = c->L.gu_s;
    a.tile_w = c->L.gu_tile_w;
    a.tile_s = c->L.gu_tile_s;
    a.n_wtiles = F / 8;
    a.out = c->hb;
    a.ldo = F;
    {
        // 8 weight tiles per wave for gate/up (4 ran the same), 4 for down
        // (8 ran ~2 % slower: the down blocks are shorter, K = F)
        const int ng = (a.n_wtiles + 4 * 8 - 1) / (4 * 8);
        MX_LAUNCH(MOE_PROF_GATEUP, "gate/up launch",
                  (launch(mx_proj_kernel<true, 8>, grid8(mt_max * ng), 256, 0, st, a, tl, c->n_tiles,
                          mt_max, ng),
                   hipGetLastError()));
    }
    // down -> Y [T*S, H]
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
        const int ng = (a.n_wtiles + 4 * 4 - 1) / (4 * 4);
        MX_LAUNCH(MOE_PROF_DOWN, "down launch",
                  (launch(mx_proj_kernel<false, 4>, grid8(mt_max * ng), 256, 0, st, a, tl, c->n_tiles,
                          mt_max, ng),
                   hipGetLastError()));
    }
    MX_LAUNCH(MOE_PROF_COMBINE, "combine launch",
              launch_combine(c->Y, idx, gw, T, k, E, d.n_shared, H, out, d.out_dtype, st));
#undef MX_LAUNCH
    return MOE_OK;
}

}  // namespace moe
