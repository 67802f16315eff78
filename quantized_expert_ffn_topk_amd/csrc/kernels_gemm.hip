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
// Work list: tiles of up to 128 rows of one expert (built on the device from
// the per-expert counts, no host synchronisation).  Blocks are remapped so
// that each XCD walks a contiguous run of tiles of the same expert and weight
// block, keeping that block in its own L2.
#include "device_common.h"
#include "host_common.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int MT = 128;    // activation rows per tile
#ifndef MOE_GEMM_NW
#define MOE_GEMM_NW 16
#endif

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
// Tile list: for experts 0..n_exp-1 in order, ceil(cnt/mt) tiles (e, m0).
// One block of 1024 threads; n_exp <= 2048.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void mfma_tiles_kernel(const int32_t *__restrict__ cnt,
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

hipError_t launch_mfma_tiles(moe_ctx *c, int T, hipStream_t st)
{
    (void)T;
    launch(mfma_tiles_kernel, 1, 1024, 0, st, c->cnt, c->d.n_experts + c->d.n_shared, MT,
                                          reinterpret_cast<int2 *>(c->tiles), c->n_tiles);
    return hipGetLastError();
}

hipError_t launch_row_tiles(moe_ctx *c, int mt, hipStream_t st)
{
    launch(mfma_tiles_kernel, 1, 1024, 0, st, c->cnt, c->d.n_experts + c->d.n_shared, mt,
           reinterpret_cast<int2 *>(c->tiles), c->n_tiles);
    return hipGetLastError();
}

hipError_t launch_mfma_tiles_single(moe_ctx *c, int T, hipStream_t st)
{
    (void)T;
    launch(mfma_tiles_kernel, 1, 1024, 0, st, c->dbg_cnt, 1, MT, reinterpret_cast<int2 *>(c->tiles),
                                          c->n_tiles);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Shared pieces.
// ---------------------------------------------------------------------------
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
// One kernel body for both projections.  A block (8 waves) owns a tile of up
// to 128 activation rows of one expert and 128 weight rows:
//   GATEUP: gate rows n and up rows n for n in [64nb, 64nb+64), output
//           h = fp32(silu(G)*U) (G, U scaled by the token scale);
//   PROJ  : weight rows [128nb, 128nb+128) (down projection, or one part of
//           the gate/up section), output fp32(sum * row scale).
// K is walked in stages of 4 chunks (128 inputs).  Each stage's activation
// rows (128 x 128 B), its weights already widened from nibbles to the signed
// bytes 16q (128 x 128 B) and its group scales / 16 as fp32 are staged in LDS,
// double buffered, rows padded so that 16-byte LDS reads are free of bank
// conflicts.  Widening and scale conversion happen once per block in the
// staging, so the waves' VALU work is the exact epilogue alone.
// Wave w: activation block w&3 (32 rows) and weight blocks rb0, rb1 (32 rows
// each): two MFMAs per chunk.  Waves whose block is past the expert's rows
// only help staging.  80 KB of LDS: two blocks per CU.
// ---------------------------------------------------------------------------
constexpr int KB = 4;                      // chunks per stage
constexpr int A_LD = KB * 32 + 16;         // LDS row pitch of activations (bytes)
constexpr int B_LD = KB * 32 + 16;         // LDS row pitch of widened weights
constexpr int A_STAGE = MT * A_LD;
constexpr int B_STAGE = 128 * B_LD;
constexpr int S_STAGE = 128 * KB;          // fp32 scales / 16 per stage (GS = 1)

template <bool GATEUP, int GS>
__global__ __launch_bounds__(512)
void mfma_proj_kernel(ProjArgs a, const int2 *__restrict__ tiles,
                                                           const int32_t *__restrict__ n_tiles,
                                                           int mt_max, int n_blocks,
                                                           float *__restrict__ out, int ldo)
{
    __shared__ __align__(16) uint8_t lds_a[2 * A_STAGE];
    __shared__ __align__(16) uint8_t lds_b[2 * B_STAGE];
    __shared__ float lds_s[2 * S_STAGE];
    __shared__ int s_slot[MT], s_row[MT];
    __shared__ float s_sc[MT];
    __shared__ int s_tile[8];

    int nb, mt;
    block_coords(mt_max, &nb, &mt);
    if (nb >= n_blocks || mt >= *n_tiles)
        return;
    const int2 tl = tiles[mt];
    const int e = tl.x, m0 = tl.y;
    const int mc = min(MT, a.rt.cnt[e] - m0);
    const int tid = threadIdx.x;
    if (tid < MT) {
        int slot = -1, row = -1;
        float sc = 0.0f;
        if (tid < mc) {
            slot = a.rt.list[(size_t)e * a.rt.list_stride + m0 + tid];
            row = a.in_by_token ? slot / a.rt.S : slot;
            sc = a.s[row];
        }
        s_slot[tid] = slot;
        s_row[tid] = row;
        s_sc[tid] = sc;
    }
    if (tid < 8) {
        // blob tile of LDS weight rows [16*tid, 16*tid+16)
        int t;
        if (GATEUP) {
            t = (tid < 4) ? 2 * (4 * nb + tid) : 2 * (4 * nb + tid - 4) + 1;
        } else {
            const int n = 128 * nb + 16 * tid;
            t = a.tile_base + (n >> 5) * a.pair_stride + ((n >> 4) & 1) * a.j_stride;
        }
        s_tile[tid] = t;
    }
    __syncthreads();

    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);
    const int K = a.K, KC = K >> 5, n_stages = KC / KB;
    const uint8_t *qbase = reinterpret_cast<const uint8_t *>(a.q);

    // global -> LDS assignment: activations 1024 pieces of 16 B (2/thread),
    // weight nibbles 512 pieces (1/thread, widened to 32 B), scales 128 rows x
    // KB/GS groups (one per thread for the first 128*KB/GS threads)
    const uint8_t *ga0, *ga1;
    int la0, la1;
    {
        const int tok0 = tid >> 3, tok1 = (tid + 512) >> 3, seg = tid & 7;
        const int row0 = s_row[tok0], row1 = s_row[tok1];
        ga0 = qbase + (size_t)(row0 < 0 ? s_row[0] : row0) * K + seg * 16;
        ga1 = qbase + (size_t)(row1 < 0 ? s_row[0] : row1) * K + seg * 16;
        la0 = tok0 * A_LD + seg * 16;
        la1 = tok1 * A_LD + seg * 16;
    }
    const uint8_t *gb;
    int lb;
    {
        const int r = tid & 15, kcl = (tid >> 4) & 3, tj = tid >> 6;
        gb = blob + a.w_off + (size_t)s_tile[tj] * a.tile_w + kcl * 256 + r * 16;
        lb = (16 * tj + r) * B_LD + kcl * 32;
    }
    constexpr int NG = KB / GS;                // scale groups per stage
    const bool s_thread = tid < 128 * NG;
    const uint16_t *gs_ = nullptr;
    int ls_ = 0;
    if (s_thread) {
        const int row = tid / NG, u = tid % NG;
        gs_ = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)s_tile[row >> 4] * a.tile_s) +
              u * 16 + (row & 15);
        ls_ = row * KB + u;
    }

    const int wave = tid >> 6, lane = tid & 63;
    const int hh = lane >> 5, li = lane & 31;
    const int mb = wave & 3, np = wave >> 2;
    const int rb0 = GATEUP ? np : 2 * np;
    const int rb1 = GATEUP ? 2 + np : 2 * np + 1;
    const bool active = __builtin_amdgcn_readfirstlane(32 * mb < mc ? 1 : 0) != 0;
    const int R0 = 32 * rb0 + li, R1 = 32 * rb1 + li;
    const int arow = 32 * mb + li;

    double acc[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[i][r] = 0.0;

    uint4 ra0, ra1, rbv;
    uint16_t rs = 0;
#define GLOAD(stage)                                                              \
    do {                                                                          \
        const size_t ko_ = (size_t)(stage) * KB;                                  \
        ra0 = *reinterpret_cast<const uint4 *>(ga0 + ko_ * 32);                   \
        ra1 = *reinterpret_cast<const uint4 *>(ga1 + ko_ * 32);                   \
        rbv = *reinterpret_cast<const uint4 *>(gb + ko_ * 256);                   \
        if (s_thread)                                                             \
            rs = gs_[(size_t)(stage) * NG * 16];                                  \
    } while (0)
    // nibble j of a byte: low = input j, high = input j+16 (4-bit two's
    // complement); masked into the top of a byte it is the signed byte 16q
#define LSTORE(buf)                                                               \
    do {                                                                          \
        *reinterpret_cast<uint4 *>(lds_a + (buf) * A_STAGE + la0) = ra0;          \
        *reinterpret_cast<uint4 *>(lds_a + (buf) * A_STAGE + la1) = ra1;          \
        *reinterpret_cast<uint4 *>(lds_b + (buf) * B_STAGE + lb) =                \
            make_uint4((rbv.x << 4) & 0xf0f0f0f0u, (rbv.y << 4) & 0xf0f0f0f0u,    \
                       (rbv.z << 4) & 0xf0f0f0f0u, (rbv.w << 4) & 0xf0f0f0f0u);   \
        *reinterpret_cast<uint4 *>(lds_b + (buf) * B_STAGE + lb + 16) =           \
            make_uint4(rbv.x & 0xf0f0f0f0u, rbv.y & 0xf0f0f0f0u,                  \
                       rbv.z & 0xf0f0f0f0u, rbv.w & 0xf0f0f0f0u);                 \
        if (s_thread)                                                             \
            lds_s[(buf) * S_STAGE + ls_] = f16_to_f32(rs) * 0.0625f; /* exact */  \
    } while (0)

    GLOAD(0);
    LSTORE(0);
    __syncthreads();
    for (int st = 0; st < n_stages; ++st) {
        const int buf = st & 1;
        if (st + 1 < n_stages)
            GLOAD(st + 1);
        if (active) {
            const uint8_t *A = lds_a + buf * A_STAGE + arow * A_LD + 16 * hh;
            const uint8_t *B0 = lds_b + buf * B_STAGE + R0 * B_LD + 16 * hh;
            const uint8_t *B1 = lds_b + buf * B_STAGE + R1 * B_LD + 16 * hh;
            const float *S0 = lds_s + buf * S_STAGE + R0 * KB;
            const float *S1 = lds_s + buf * S_STAGE + R1 * KB;
#pragma unroll
            for (int u = 0; u < KB; u += GS) {
                const v16i zero = {0};
                v16i d0 = zero, d1 = zero;
#pragma unroll
                for (int v = 0; v < GS; ++v) {
                    const v4i av = as_v4i(*reinterpret_cast<const uint4 *>(A + (u + v) * 32));
                    d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        av, as_v4i(*reinterpret_cast<const uint4 *>(B0 + (u + v) * 32)), d0, 0, 0, 0);
                    d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        av, as_v4i(*reinterpret_cast<const uint4 *>(B1 + (u + v) * 32)), d1, 0, 0, 0);
                }
                const double s0 = (double)S0[u / GS], s1 = (double)S1[u / GS];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    acc[0][r] = fma((double)d0[r], s0, acc[0][r]);
                    acc[1][r] = fma((double)d1[r], s1, acc[1][r]);
                }
            }
        }
        if (st + 1 < n_stages)
            LSTORE(buf ^ 1);
        __syncthreads();
    }
#undef GLOAD
#undef LSTORE
    if (!active)
        return;

    // epilogue: register r of lane l holds activation row 8(r/4)+4(l/32)+r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int tok = 32 * mb + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int slot = s_slot[tok];
        if (slot < 0)
            continue;
        const double sc = (double)s_sc[tok];
        float *o = out + (size_t)slot * ldo;
        if (GATEUP) {
            const double G = acc[0][r] * sc, U = acc[1][r] * sc;
            o[64 * nb + 32 * np + li] = (float)(G / (1.0 + exp(-G)) * U);
        } else {
            o[128 * nb + 32 * rb0 + li] = (float)(acc[0][r] * sc);
            o[128 * nb + 32 * rb1 + li] = (float)(acc[1][r] * sc);
        }
    }
}

// ---------------------------------------------------------------------------
// The same tile with 16 waves (1024 threads): wave w owns activation block
// w>>2 and one 32-row weight block w&3 (the four waves of a SIMD hold the four
// activation blocks, so a partial tile still spreads over all SIMDs), 16 sums
// per lane.  GATEUP: weight blocks 0, 1 are gate rows, 2, 3 the matching up
// rows; after the K loop the up waves hand their sums to the gate waves
// through LDS (the staging buffers, free by then).
//
// Exact epilogue in 64-bit integers.  A nonzero fp16 scale is m * 2^(E-25)
// (m = 1024 + fraction and E the exponent field for normal numbers, m =
// fraction and E = 1 for subnormals).  A first pass over the block's scales
// finds, per weight row, the smallest E of its nonzero scales, Emin; group j
// then contributes the integer M_j = +-m_j << (E_j - Emin) and the row sum is
//   sum_j s_j * dot_j = 2^(Emin-29) * sum_j M_j * dot16_j
// with dot16 = 16 x the group dot (the MFMA sees the nibbles as 16q).  One
// v_mad_i64_i32 per output and group accumulates it without rounding
// (|dot16| < 2^20, |M| < 2^31, at most 256 groups), and the row sum, whose
// significant bits fit fp64 under the packer's exponent-spread bound, turns
// into the same fp64 value as the fp64 epilogue would give.  A block holding a
// row whose scale exponents span more than 20 binades (M would not fit 31
// bits) takes that fp64 epilogue instead: each product dot16 * s/16 is exact in
// fp64, and so is the sum under the same bound.
// KS chunks of 32 inputs per stage (4: two blocks fit one CU's LDS).
// ---------------------------------------------------------------------------
template <int KS>
struct Stage16 {
    static constexpr int LD = KS * 32 + 16;       // LDS row pitch (bytes)
    static constexpr int A = MT * LD;             // activation rows
    static constexpr int B = 128 * LD;            // widened weight rows
    static constexpr int S = 128 * KS;            // per-group scale words
};

constexpr int MAX_INT_SPREAD = 20;    // m (11 bits) << 20 stays below 2^31

// fp16 scale -> (signed integer significand shifted to the row's smallest
// exponent), 0 for a zero scale
__device__ __forceinline__ int scale_int(uint16_t h, int emin)
{
    if ((h & 0x7fff) == 0)
        return 0;
    const int ef = (h >> 10) & 31;
    const int m = (h & 0x3ff) | (ef ? 0x400 : 0);
    const int v = m << ((ef ? ef : 1) - emin);
    return (h & 0x8000) ? -v : v;
}

template <bool GATEUP, int GS, int KS>
__global__ __launch_bounds__(1024) void mfma_proj16_kernel(ProjArgs a, const int2 *__restrict__ tiles,
                                                           const int32_t *__restrict__ n_tiles,
                                                           int mt_max, int n_blocks,
                                                           float *__restrict__ out, int ldo)
{
    static_assert(KS == 4, "one 16-byte activation piece per thread and stage");
    typedef Stage16<KS> L;
    __shared__ __align__(16) uint8_t lds_ab[2 * L::A + 2 * L::B];
    __shared__ float lds_s[2 * L::S];
    __shared__ int s_slot[MT], s_row[MT];
    __shared__ float s_sc[MT];
    __shared__ int s_tile[8];
    __shared__ int s_emin[128], s_emax[128];
    uint8_t *lds_a = lds_ab, *lds_b = lds_ab + 2 * L::A;

    int nb, mt;
    block_coords(mt_max, &nb, &mt);
    if (nb >= n_blocks || mt >= *n_tiles)
        return;
    const int2 tl = tiles[mt];
    const int e = tl.x, m0 = tl.y;
    const int mc = min(MT, a.rt.cnt[e] - m0);
    const int tid = threadIdx.x;
    if (tid < MT) {
        int slot = -1, row = -1;
        float sc = 0.0f;
        if (tid < mc) {
            slot = a.rt.list[(size_t)e * a.rt.list_stride + m0 + tid];
            row = a.in_by_token ? slot / a.rt.S : slot;
            sc = a.s[row];
        }
        s_slot[tid] = slot;
        s_row[tid] = row;
        s_sc[tid] = sc;
        s_emin[tid] = 99;
        s_emax[tid] = -99;
    }
    if (tid < 8) {
        int t;
        if (GATEUP) {
            t = (tid < 4) ? 2 * (4 * nb + tid) : 2 * (4 * nb + tid - 4) + 1;
        } else {
            const int n = 128 * nb + 16 * tid;
            t = a.tile_base + (n >> 5) * a.pair_stride + ((n >> 4) & 1) * a.j_stride;
        }
        s_tile[tid] = t;
    }
    __syncthreads();

    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);
    const int K = a.K, KC = K >> 5, n_stages = KC / KS, G = KC / GS;
    const uint8_t *qbase = reinterpret_cast<const uint8_t *>(a.q);

    // exponent range of each weight row's nonzero scales ([tile][group][r]
    // layout: thread = (tile, row r, group phase j0), groups j0, j0+8, ...)
    {
        const int tj = tid >> 7, r = tid & 15;
        const uint16_t *sp =
            reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)s_tile[tj] * a.tile_s) + r;
        int lo = 99, hi = -99;
        for (int j = (tid >> 4) & 7; j < G; j += 8) {
            const uint16_t h = sp[(size_t)j * 16];
            if (h & 0x7fff) {
                const int ef = (h >> 10) & 31;
                const int ev = ef ? ef : 1;
                lo = min(lo, ev);
                hi = max(hi, ev);
            }
        }
        atomicMin(&s_emin[16 * tj + r], lo);
        atomicMax(&s_emax[16 * tj + r], hi);
    }
    __syncthreads();
    const int wide_row =
        (tid < 128 && s_emax[tid] - s_emin[tid] > MAX_INT_SPREAD) ? 1 : 0;   // all-zero rows: -198
    const bool wide = __syncthreads_or(wide_row) != 0;

    // global -> LDS per stage: activations 128 rows x KS*32 B in 16-byte
    // pieces (one per thread); weight nibbles 128 rows x KS chunks of 16 B
    // (one piece per thread for the first 128*KS threads, widened to 32 B);
    // scales 128 rows x KS/GS groups
    const uint8_t *ga;
    int la;
    {
        const int tok = tid / (2 * KS), seg = tid % (2 * KS);
        const int row = s_row[tok];
        ga = qbase + (size_t)(row < 0 ? s_row[0] : row) * K + seg * 16;
        la = tok * L::LD + seg * 16;
    }
    // every thread issues every load (threads past a piece list reload a
    // valid piece and skip the store): with no branch around the loads the
    // compiler waits for exactly the older stage's loads
    const bool b_thread = tid < 128 * KS;
    const uint8_t *gb;
    int lb;
    {
        const int bt = tid % (128 * KS);
        const int r = bt & 15, kcl = (bt >> 4) % KS, tj = bt / (16 * KS);
        gb = blob + a.w_off + (size_t)s_tile[tj] * a.tile_w + kcl * 256 + r * 16;
        lb = (16 * tj + r) * L::LD + kcl * 32;
    }
    constexpr int NG = KS / GS;
    const int sq = (KS == 4) ? tid - 512 : tid;
    const bool s_thread = sq >= 0 && sq < 128 * NG;
    const uint16_t *gs_;
    int ls_, em_;
    {
        const int sqc = s_thread ? sq : 0;
        const int row = sqc / NG, u = sqc % NG;
        gs_ = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)s_tile[row >> 4] * a.tile_s) +
              u * 16 + (row & 15);
        ls_ = row * KS + u;
        em_ = s_emin[row];
    }

    const int wave = tid >> 6, lane = tid & 63;
    const int hh = lane >> 5, li = lane & 31;
    const int mb = wave >> 2, wb = wave & 3;
    const bool active = __builtin_amdgcn_readfirstlane(32 * mb < mc ? 1 : 0) != 0;
    const int R = 32 * wb + li;
    const int arow = 32 * mb + li;

    // staging registers: set P (ra<P>, rbv<P>, rs<P>) holds the loads of the
    // stages of parity P
    uint4 ra0 = {}, ra1 = {}, rbv0 = {}, rbv1 = {};
    uint16_t rs0 = 0, rs1 = 0;
#define GLOAD(P, stage)                                                           \
    do {                                                                          \
        const size_t ko_ = (size_t)(stage) * KS;                                  \
        ra##P = *reinterpret_cast<const uint4 *>(ga + ko_ * 32);                  \
        rbv##P = *reinterpret_cast<const uint4 *>(gb + ko_ * 256);                \
        rs##P = gs_[(size_t)(stage) * NG * 16];                                   \
    } while (0)
    // nibble j of a byte: low = input j, high = input j+16 (4-bit two's
    // complement); masked into the top of a byte it is the signed byte 16q.
    // Scale words: the integer M (INTM) or the fp32 scale / 16 (exact).
#define LSTORE(P, buf, INTM)                                                      \
    do {                                                                          \
        *reinterpret_cast<uint4 *>(lds_a + (buf) * L::A + la) = ra##P;            \
        if (b_thread) {                                                           \
            const uint4 w_ = rbv##P;                                              \
            *reinterpret_cast<uint4 *>(lds_b + (buf) * L::B + lb) =               \
                make_uint4((w_.x << 4) & 0xf0f0f0f0u, (w_.y << 4) & 0xf0f0f0f0u,  \
                           (w_.z << 4) & 0xf0f0f0f0u, (w_.w << 4) & 0xf0f0f0f0u); \
            *reinterpret_cast<uint4 *>(lds_b + (buf) * L::B + lb + 16) =          \
                make_uint4(w_.x & 0xf0f0f0f0u, w_.y & 0xf0f0f0f0u,                \
                           w_.z & 0xf0f0f0f0u, w_.w & 0xf0f0f0f0u);               \
        }                                                                         \
        if (s_thread)                                                             \
            lds_s[(buf) * L::S + ls_] = (INTM) ? __int_as_float(scale_int(rs##P, em_)) \
                                               : f16_to_f32(rs##P) * 0.0625f;     \
    } while (0)
    // the K loop: stage st sits in LDS buffer st&1 while the loads of stages
    // st+1 (register set (st+1)&1, written to the other buffer at the end of
    // the stage) and st+2 (set st&1) are in flight; EPI(d, sword) folds one
    // group's 32x32 dots in.  The stage count is even (K is a multiple of
    // 256) and the loads past the last stage repeat it, so the loop is
    // straight-line code and each LDS store waits for its own loads only.
#define KSTAGE(P, Q, st, INTM, EPI)                                               \
    do {                                                                          \
        GLOAD(P, min((st) + 2, n_stages - 1));                                    \
        if (active) {                                                             \
            const uint8_t *A_ = lds_a + (P) * L::A + arow * L::LD + 16 * hh;      \
            const uint8_t *B_ = lds_b + (P) * L::B + R * L::LD + 16 * hh;         \
            const float *S_ = lds_s + (P) * L::S + R * KS;                        \
            _Pragma("unroll") for (int u = 0; u < KS; u += GS) {                  \
                const v16i zero = {0};                                            \
                v16i d = zero;                                                    \
                _Pragma("unroll") for (int v = 0; v < GS; ++v)                    \
                    d = __builtin_amdgcn_mfma_i32_32x32x32_i8(                    \
                        as_v4i(*reinterpret_cast<const uint4 *>(A_ + (u + v) * 32)), \
                        as_v4i(*reinterpret_cast<const uint4 *>(B_ + (u + v) * 32)), \
                        d, 0, 0, 0);                                              \
                EPI(d, S_[u / GS]);                                               \
            }                                                                     \
        }                                                                         \
        LSTORE(Q, Q, INTM);                                                       \
        __syncthreads();                                                          \
    } while (0)
#define KLOOP(INTM, EPI)                                                          \
    do {                                                                          \
        GLOAD(0, 0);                                                              \
        GLOAD(1, 1);                                                              \
        LSTORE(0, 0, INTM);                                                       \
        __syncthreads();                                                          \
        for (int st = 0; st < n_stages; st += 2) {                                \
            KSTAGE(0, 1, st, INTM, EPI);                                          \
            KSTAGE(1, 0, st + 1, INTM, EPI);                                      \
        }                                                                         \
    } while (0)

    double acc[16];
    if (!wide) {
        int64_t iacc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            iacc[r] = 0;
#define EPI_INT(d, sw)                                                            \
        do {                                                                      \
            const int64_t m_ = __float_as_int(sw);                                \
            _Pragma("unroll") for (int r = 0; r < 16; ++r)                        \
                iacc[r] += (int64_t)d[r] * m_;                                    \
        } while (0)
        KLOOP(true, EPI_INT);
#undef EPI_INT
        // the exact row sum 2^(Emin-29) * sum M*dot16 as fp64: hi*2^32 + lo is
        // exact since the sum's significant bits fit 53
        const int emin = s_emin[R];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const double v = (double)(int)(iacc[r] >> 32) * 4294967296.0 +
                             (double)(unsigned)(iacc[r] & 0xffffffffu);
            acc[r] = ldexp(v, emin - 29);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[r] = 0.0;
#define EPI_F64(d, sw)                                                            \
        do {                                                                      \
            const double s_ = (double)(sw);                                       \
            _Pragma("unroll") for (int r = 0; r < 16; ++r)                        \
                acc[r] = fma((double)d[r], s_, acc[r]);                           \
        } while (0)
        KLOOP(false, EPI_F64);
#undef EPI_F64
    }
#undef KLOOP
#undef KSTAGE
#undef GLOAD
#undef LSTORE

    // result register r of lane l: activation row 8(r/4)+4(l/32)+r%4
    if (GATEUP) {
        // up waves (wb 2, 3) hand their sums to the gate waves (wb 0, 1)
        double *xch = reinterpret_cast<double *>(lds_ab);   // [2][4][16][64]
        if (active && wb >= 2) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                xch[(((wb - 2) * 4 + mb) * 16 + r) * 64 + lane] = acc[r];
        }
        __syncthreads();
        if (!active || wb >= 2)
            return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = 32 * mb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const int slot = s_slot[tok];
            if (slot < 0)
                continue;
            const double sc = (double)s_sc[tok];
            const double G_ = acc[r] * sc;
            const double U = xch[((wb * 4 + mb) * 16 + r) * 64 + lane] * sc;
            out[(size_t)slot * ldo + 64 * nb + 32 * wb + li] = (float)(G_ / (1.0 + exp(-G_)) * U);
        }
    } else {
        if (!active)
            return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tok = 32 * mb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const int slot = s_slot[tok];
            if (slot < 0)
                continue;
            out[(size_t)slot * ldo + 128 * nb + 32 * wb + li] = (float)(acc[r] * (double)s_sc[tok]);
        }
    }
}

#ifndef MOE_GEMM_KS
#define MOE_GEMM_KS 4
#endif


static int grid_for(int mt_max, int n_blocks)
{
    long n = (long)mt_max * n_blocks;
    return (int)((n + 7) / 8 * 8);      // the XCD remap needs a multiple of 8
}

hipError_t launch_gateup_mfma(const ProjArgs &a, const moe_ctx *c, int T, int F, float *h, int ldh,
                              hipStream_t st)
{
    const int mt_max = tiles_bound(c, T);
    const int2 *tl = reinterpret_cast<const int2 *>(c->tiles);
#if MOE_GEMM_NW == 16
    const int grid = grid_for(mt_max, F / 64);
    if (a.group_shift)
        launch(mfma_proj16_kernel<true, 2, MOE_GEMM_KS>, grid, 1024, 0, st, a, tl, c->n_tiles, mt_max, F / 64, h, ldh);
    else
        launch(mfma_proj16_kernel<true, 1, MOE_GEMM_KS>, grid, 1024, 0, st, a, tl, c->n_tiles, mt_max, F / 64, h, ldh);
#else
    const int grid = grid_for(mt_max, F / 64);
    if (a.group_shift)
        launch(mfma_proj_kernel<true, 2>, grid, 512, 0, st, a, tl, c->n_tiles, mt_max, F / 64, h, ldh);
    else
        launch(mfma_proj_kernel<true, 1>, grid, 512, 0, st, a, tl, c->n_tiles, mt_max, F / 64, h, ldh);
#endif
    return hipGetLastError();
}

hipError_t launch_proj_mfma(const ProjArgs &a, const moe_ctx *c, int T, int n_rows, hipStream_t st)
{
    // inspection projections use a single blob (one expert holding T rows)
    const int mt_max = (a.ex.E == 0) ? (T + MT - 1) / MT : tiles_bound(c, T);
    const int2 *tl = reinterpret_cast<const int2 *>(c->tiles);
#if MOE_GEMM_NW == 16
    const int grid = grid_for(mt_max, n_rows / 128);
    if (a.group_shift)
        launch(mfma_proj16_kernel<false, 2, MOE_GEMM_KS>, grid, 1024, 0, st, a, tl, c->n_tiles, mt_max, n_rows / 128, a.out, a.ldo);
    else
        launch(mfma_proj16_kernel<false, 1, MOE_GEMM_KS>, grid, 1024, 0, st, a, tl, c->n_tiles, mt_max, n_rows / 128, a.out, a.ldo);
#else
    const int grid = grid_for(mt_max, n_rows / 128);
    if (a.group_shift)
        launch(mfma_proj_kernel<false, 2>, grid, 512, 0, st, a, tl, c->n_tiles, mt_max, n_rows / 128, a.out, a.ldo);
    else
        launch(mfma_proj_kernel<false, 1>, grid, 512, 0, st, a, tl, c->n_tiles, mt_max, n_rows / 128, a.out, a.ldo);
#endif
    return hipGetLastError();
}

}  // namespace moe
