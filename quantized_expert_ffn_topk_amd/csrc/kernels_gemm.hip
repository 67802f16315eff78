// kernels_gemm.hip -- grouped int4 x int8 GEMM on the gfx950 int8 MFMA for
// many rows per expert (prefill).
//
// Same arithmetic as the GEMV path (the integer-dot scheme of the Colibri
// guide, table "Points techniques cles"; batched prefill runs on the integer
// kernel, section "Analyse approfondie"): per chunk of 32 inputs one
// v_mfma_i32_32x32x32_i8 gives 16 x the exact int32 group dots of 32 rows x
// 32 columns; each is multiplied by its fp16 scale / 16 and added in fp64,
// which is exact, so results are bit-identical to the GEMV kernels.
//
// Operand mapping (v_mfma_i32_32x32x32_i8, wave64): lane l supplies A row
// l%32 (an activation row) and B column l%32 (a weight row), 16 bytes each, for
// inputs [16*(l/32), 16*(l/32)+16) of the chunk: exactly the low (l<32) or
// high (l>=32) nibbles of the weight row's 16-byte chunk in the blob.  The
// 32x32 int32 result sits in 16 registers: register r of lane l is activation
// row 8*(r/4) + 4*(l/32) + r%4, weight row l%32.  Each lane therefore needs a
// single scale per chunk.
//
// Work list: tiles of up to 64 rows of one expert (built on the device from
// the per-expert counts, no host synchronisation).  Blocks are remapped so
// that each XCD walks a contiguous run of tiles of the same expert and weight
// block, keeping that block in its own L2.
#include "device_common.h"
#include "host_common.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int MT = 64;     // activation rows per tile

bool use_mfma(const moe_ctx *c, int T)
{
    if (c->d.wfmt != MOE_WFMT_INT4)
        return false;
    if (c->path == MOE_PATH_MFMA)
        return true;
    if (c->path == MOE_PATH_GEMV)
        return false;
    return T >= 64;
}

size_t mfma_max_tiles(int T, int E, int n_shared)
{
    // every expert with rows adds at most one partial tile
    return (size_t)T * 17 / MT + 1 + (size_t)E + (size_t)n_shared;
}

static int tiles_bound(const moe_ctx *c, int T)
{
    const int k = c->d.top_k, E = c->d.n_experts;
    const int busy = (T * k < E ? T * k : E) + c->d.n_shared;
    return (T * c->S + MT - 1) / MT + busy;
}

// ---------------------------------------------------------------------------
// Tile list: for experts 0..n_exp-1 in order, ceil(cnt/64) tiles (e, m0).
// One block of 1024 threads; n_exp <= 2048.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void mfma_tiles_kernel(const int32_t *__restrict__ cnt,
                                                          int n_exp, int2 *__restrict__ tiles,
                                                          int32_t *__restrict__ n_tiles)
{
    __shared__ int sc[1024];
    const int t = threadIdx.x;
    const int e0 = 2 * t, e1 = 2 * t + 1;
    const int c0 = e0 < n_exp ? (cnt[e0] + MT - 1) / MT : 0;
    const int c1 = e1 < n_exp ? (cnt[e1] + MT - 1) / MT : 0;
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
        tiles[base + j] = make_int2(e0, j * MT);
    for (int j = 0; j < c1; ++j)
        tiles[base + c0 + j] = make_int2(e1, j * MT);
    if (t == 1023)
        *n_tiles = sc[1023];
}

hipError_t launch_mfma_tiles(moe_ctx *c, int T, hipStream_t st)
{
    (void)T;
    mfma_tiles_kernel<<<1, 1024, 0, st>>>(c->cnt, c->d.n_experts + c->d.n_shared,
                                          reinterpret_cast<int2 *>(c->tiles), c->n_tiles);
    return hipGetLastError();
}

hipError_t launch_mfma_tiles_single(moe_ctx *c, int T, hipStream_t st)
{
    (void)T;
    mfma_tiles_kernel<<<1, 1024, 0, st>>>(c->dbg_cnt, 1, reinterpret_cast<int2 *>(c->tiles),
                                          c->n_tiles);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Shared pieces.
// ---------------------------------------------------------------------------
struct TileRows {
    int e, m0, mc;
};

// Block index -> (weight block nb, tile mt): each XCD (blocks b with the same
// b % 8) gets a contiguous run of logical indices, tile index fastest.  The
// grid is padded to a multiple of 8; padding blocks get nb >= n_blocks.
__device__ __forceinline__ void block_coords(int mt_max, int *nb, int *mt)
{
    const int nwg = gridDim.x;
    const int b = blockIdx.x;
    const int logical = (b & 7) * (nwg >> 3) + (b >> 3);
    *nb = logical / mt_max;
    *mt = logical - *nb * mt_max;
}

// Stages the tile's slots and row scales; -1 marks rows past the expert's end.
__device__ __forceinline__ void stage_tile(const ProjArgs &a, int e, int m0, int mc, int *s_slot,
                                           int *s_row, float *s_sc)
{
    if (threadIdx.x < MT) {
        const int i = threadIdx.x;
        int slot = -1, row = -1;
        float sc = 0.0f;
        if (i < mc) {
            slot = a.rt.list[(size_t)e * a.rt.list_stride + m0 + i];
            row = a.in_by_token ? slot / a.rt.S : slot;
            sc = a.s[row];
        }
        s_slot[i] = slot;
        s_row[i] = row;
        s_sc[i] = sc;
    }
    __syncthreads();
}

__device__ __forceinline__ v4i nibble_bytes(uint4 w, int shift)
{
    v4i b;
    b[0] = (int)((w.x << shift) & 0xf0f0f0f0u);
    b[1] = (int)((w.y << shift) & 0xf0f0f0f0u);
    b[2] = (int)((w.z << shift) & 0xf0f0f0f0u);
    b[3] = (int)((w.w << shift) & 0xf0f0f0f0u);
    return b;
}

__device__ __forceinline__ v4i as_v4i(uint4 w)
{
    v4i b;
    b[0] = (int)w.x;
    b[1] = (int)w.y;
    b[2] = (int)w.z;
    b[3] = (int)w.w;
    return b;
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU.  Block = 64 rows x 64 outputs n (64 gate + 64 up weight
// rows); wave (wm, wn) = rows [32wm, +32) x n [32wn, +32), two MFMAs per chunk.
// GS = chunks per scale group (1 for group 32, 2 for group 64).
// ---------------------------------------------------------------------------
template <int GS>
__global__ __launch_bounds__(256) void gateup_mfma_kernel(ProjArgs a, const int2 *__restrict__ tiles,
                                                          const int32_t *__restrict__ n_tiles,
                                                          int mt_max, int n_blocks,
                                                          float *__restrict__ h, int ldh)
{
    __shared__ int s_slot[MT], s_row[MT];
    __shared__ float s_sc[MT];
    int nb, mt;
    block_coords(mt_max, &nb, &mt);
    if (nb >= n_blocks || mt >= *n_tiles)
        return;
    const int2 tl = tiles[mt];
    const int e = tl.x, m0 = tl.y;
    const int mc = min(MT, a.rt.cnt[e] - m0);
    stage_tile(a, e, m0, mc, s_slot, s_row, s_sc);

    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);
    const int K = a.K, KC = K >> 5;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave & 1, wn = wave >> 1;
    const int hh = lane >> 5, li = lane & 31;
    const int arow = s_row[32 * wm + li];
    const uint8_t *ap = reinterpret_cast<const uint8_t *>(a.q) + (size_t)(arow < 0 ? 0 : arow) * K + 16 * hh;
    const int n = 64 * nb + 32 * wn + li;
    const int bt = 2 * (n >> 4), br = n & 15;
    const uint8_t *bg = blob + a.w_off + (size_t)bt * a.tile_w + br * 16;
    const uint8_t *bu = bg + a.tile_w;
    const uint16_t *sg = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)bt * a.tile_s) + br;
    const uint16_t *su = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)(bt + 1) * a.tile_s) + br;
    const int shift = hh ? 0 : 4;

    double pg[16], pu[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        pg[r] = 0.0;
        pu[r] = 0.0;
    }
    constexpr int U = 4;
    for (int c0 = 0; c0 < KC; c0 += U) {
        uint4 av[U], gv[U], uv[U];
        uint16_t sgv[U / GS], suv[U / GS];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            av[u] = *reinterpret_cast<const uint4 *>(ap + (size_t)(c0 + u) * 32);
            gv[u] = *reinterpret_cast<const uint4 *>(bg + (size_t)(c0 + u) * 256);
            uv[u] = *reinterpret_cast<const uint4 *>(bu + (size_t)(c0 + u) * 256);
        }
#pragma unroll
        for (int u = 0; u < U / GS; ++u) {
            sgv[u] = sg[(size_t)(c0 / GS + u) * 16];
            suv[u] = su[(size_t)(c0 / GS + u) * 16];
        }
#pragma unroll
        for (int u = 0; u < U; u += GS) {
            v16i dg = {0}, du = {0};
#pragma unroll
            for (int v = 0; v < GS; ++v) {
                v4i A = as_v4i(av[u + v]);
                dg = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, nibble_bytes(gv[u + v], shift), dg, 0, 0, 0);
                du = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, nibble_bytes(uv[u + v], shift), du, 0, 0, 0);
            }
            const double sgd = (double)f16_to_f32(sgv[u / GS]) * 0.0625;
            const double sud = (double)f16_to_f32(suv[u / GS]) * 0.0625;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                pg[r] = fma((double)dg[r], sgd, pg[r]);
                pu[r] = fma((double)du[r], sud, pu[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int tok = 32 * wm + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int slot = s_slot[tok];
        if (slot >= 0) {
            const double sa = (double)s_sc[tok];
            const double G = pg[r] * sa, Uv = pu[r] * sa;
            h[(size_t)slot * ldh + n] = (float)(G / (1.0 + exp(-G)) * Uv);
        }
    }
}

// ---------------------------------------------------------------------------
// Plain projection (down, or one part of gate/up for inspection).  Block =
// 64 rows x 128 outputs; wave (wm, wn) = rows [32wm, +32) x outputs
// [64wn, +64) as two 32-wide MFMA columns.  Output row n lives in tile
// tile_base + (n/32)*pair_stride + ((n/16)%2)*j_stride, row n%16.
// ---------------------------------------------------------------------------
template <int GS>
__global__ __launch_bounds__(256) void proj_mfma_kernel(ProjArgs a, const int2 *__restrict__ tiles,
                                                        const int32_t *__restrict__ n_tiles,
                                                        int mt_max, int n_blocks)
{
    __shared__ int s_slot[MT], s_row[MT];
    __shared__ float s_sc[MT];
    int nb, mt;
    block_coords(mt_max, &nb, &mt);
    if (nb >= n_blocks || mt >= *n_tiles)
        return;
    const int2 tl = tiles[mt];
    const int e = tl.x, m0 = tl.y;
    const int mc = min(MT, a.rt.cnt[e] - m0);
    stage_tile(a, e, m0, mc, s_slot, s_row, s_sc);

    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);
    const int K = a.K, KC = K >> 5;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave & 1, wn = wave >> 1;
    const int hh = lane >> 5, li = lane & 31;
    const int arow = s_row[32 * wm + li];
    const uint8_t *ap = reinterpret_cast<const uint8_t *>(a.q) + (size_t)(arow < 0 ? 0 : arow) * K + 16 * hh;
    const int n0 = 128 * nb + 64 * wn + li, n1 = n0 + 32;
    const int t0 = a.tile_base + (n0 >> 5) * a.pair_stride + ((n0 >> 4) & 1) * a.j_stride;
    const int t1 = a.tile_base + (n1 >> 5) * a.pair_stride + ((n1 >> 4) & 1) * a.j_stride;
    const uint8_t *b0 = blob + a.w_off + (size_t)t0 * a.tile_w + (n0 & 15) * 16;
    const uint8_t *b1 = blob + a.w_off + (size_t)t1 * a.tile_w + (n1 & 15) * 16;
    const uint16_t *s0 = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)t0 * a.tile_s) + (n0 & 15);
    const uint16_t *s1 = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)t1 * a.tile_s) + (n1 & 15);
    const int shift = hh ? 0 : 4;

    double p0[16], p1[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        p0[r] = 0.0;
        p1[r] = 0.0;
    }
    constexpr int U = 4;
    for (int c0 = 0; c0 < KC; c0 += U) {
        uint4 av[U], w0[U], w1[U];
        uint16_t sv0[U / GS], sv1[U / GS];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            av[u] = *reinterpret_cast<const uint4 *>(ap + (size_t)(c0 + u) * 32);
            w0[u] = *reinterpret_cast<const uint4 *>(b0 + (size_t)(c0 + u) * 256);
            w1[u] = *reinterpret_cast<const uint4 *>(b1 + (size_t)(c0 + u) * 256);
        }
#pragma unroll
        for (int u = 0; u < U / GS; ++u) {
            sv0[u] = s0[(size_t)(c0 / GS + u) * 16];
            sv1[u] = s1[(size_t)(c0 / GS + u) * 16];
        }
#pragma unroll
        for (int u = 0; u < U; u += GS) {
            v16i d0 = {0}, d1 = {0};
#pragma unroll
            for (int v = 0; v < GS; ++v) {
                v4i A = as_v4i(av[u + v]);
                d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, nibble_bytes(w0[u + v], shift), d0, 0, 0, 0);
                d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, nibble_bytes(w1[u + v], shift), d1, 0, 0, 0);
            }
            const double sd0 = (double)f16_to_f32(sv0[u / GS]) * 0.0625;
            const double sd1 = (double)f16_to_f32(sv1[u / GS]) * 0.0625;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p0[r] = fma((double)d0[r], sd0, p0[r]);
                p1[r] = fma((double)d1[r], sd1, p1[r]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int tok = 32 * wm + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int slot = s_slot[tok];
        if (slot >= 0) {
            const double sc = (double)s_sc[tok];
            float *o = a.out + (size_t)slot * a.ldo;
            o[n0] = (float)(p0[r] * sc);
            o[n1] = (float)(p1[r] * sc);
        }
    }
}

static int grid_for(int mt_max, int n_blocks)
{
    long n = (long)mt_max * n_blocks;
    return (int)((n + 7) / 8 * 8);      // the XCD remap needs a multiple of 8
}

hipError_t launch_gateup_mfma(const ProjArgs &a, const moe_ctx *c, int T, int F, float *h, int ldh,
                              hipStream_t st)
{
    const int mt_max = tiles_bound(c, T);
    const int grid = grid_for(mt_max, F / 64);
    const int2 *tl = reinterpret_cast<const int2 *>(c->tiles);
    if (a.group_shift)
        gateup_mfma_kernel<2><<<grid, 256, 0, st>>>(a, tl, c->n_tiles, mt_max, F / 64, h, ldh);
    else
        gateup_mfma_kernel<1><<<grid, 256, 0, st>>>(a, tl, c->n_tiles, mt_max, F / 64, h, ldh);
    return hipGetLastError();
}

hipError_t launch_proj_mfma(const ProjArgs &a, const moe_ctx *c, int T, int n_rows, hipStream_t st)
{
    // debug projections use a single blob (one expert holding T rows)
    const int mt_max = (a.ex.E == 0) ? (T + MT - 1) / MT : tiles_bound(c, T);
    const int grid = grid_for(mt_max, n_rows / 128);
    const int2 *tl = reinterpret_cast<const int2 *>(c->tiles);
    if (a.group_shift)
        proj_mfma_kernel<2><<<grid, 256, 0, st>>>(a, tl, c->n_tiles, mt_max, n_rows / 128);
    else
        proj_mfma_kernel<1><<<grid, 256, 0, st>>>(a, tl, c->n_tiles, mt_max, n_rows / 128);
    return hipGetLastError();
}

}  // namespace moe
