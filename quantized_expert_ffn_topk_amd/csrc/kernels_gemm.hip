// kernels_gemm.hip -- grouped int4 x int8 GEMM on the gfx950 int8 MFMA for
// many rows per expert (prefill).
//
// Same arithmetic as the GEMV path (the integer-dot scheme of the Colibri
// guide, table "Points techniques cles"; batched prefill runs on the integer
// kernel, section "Analyse approfondie"): per chunk of 32 inputs one
// v_mfma_i32_32x32x32_i8 gives 16 x the exact int32 group dots of 32 rows x
// 32 columns; the groups are combined with their fp16 scales without
// rounding, so results are bit-identical to the GEMV kernels.
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
#include "permute_common.h"

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

size_t mfma_max_tiles(int T, int E, int n_shared, int S)
{
    // every expert with rows adds at most one partial tile
    return (size_t)T * S / MT + 1 + (size_t)E + (size_t)n_shared;
}

static int tiles_bound(const moe_ctx *c, int T)
{
    const int k = c->d.top_k, E = c->d.n_experts;
    const int busy = (T * k < E ? T * k : E) + c->d.n_shared;
    return (T * c->S + MT - 1) / MT + busy;
}

// Tile list (row_tiles_block): for experts 0..n_exp-1 in order,
// ceil(cnt/mt) tiles (e, m0); one block of 1024 threads, n_exp <= 2048.
__global__ __launch_bounds__(1024) void mfma_tiles_kernel(const int32_t *__restrict__ cnt,
                                                          int n_exp, int mt,
                                                          int2 *__restrict__ tiles,
                                                          int32_t *__restrict__ n_tiles)
{
    row_tiles_block(cnt, n_exp, mt, tiles, n_tiles);
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
// One kernel body for both projections.  A block (8 waves, 512 threads) owns
// a tile of up to 64 activation rows of one expert and 128 weight rows:
//   GATEUP: gate rows n and up rows n for n in [64nb, 64nb+64), output
//           h = fp32(silu(G)*U) (G, U scaled by the token scale);
//   PROJ  : weight rows [128nb, 128nb+128) (down projection, or one part of
//           the gate/up section), output fp32(sum * token scale).
// Wave w owns activation block w>>2 (32 rows) and weight block w&3 (32 rows):
// one 32x32 MFMA per chunk, 16 sums per lane.  GATEUP: weight blocks 0, 1
// are gate rows, 2, 3 the matching up rows; after the K loop the up waves hand
// their sums to the gate waves through LDS.  Waves whose activation block is
// past the expert's rows only help staging.  A 64-row tile suits the many
// experts with few rows under skewed routing, and two blocks share a CU, so
// one block's barrier wait is covered by the other's work.
//
// K is walked in stages of 4 chunks (128 inputs): activation rows (64 x 128
// B), weights already widened from nibbles to the signed bytes 16q (128 x 128
// B) and one scale word per row and group are staged in LDS, double buffered,
// rows padded so that 16-byte LDS reads are free of bank conflicts; the global
// loads run two stages ahead.
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
// into the same fp64 value as an fp64 epilogue would give.  A block holding a
// row whose scale exponents span more than 20 binades (M would not fit 31
// bits) takes that fp64 epilogue instead: each product dot16 * s/16 is exact in
// fp64, and so is the sum under the same bound.
// ---------------------------------------------------------------------------
constexpr int KS = 4;                       // chunks per stage
constexpr int NT = 128;                     // weight rows per block
constexpr int LDP = KS * 32 + 16;           // LDS row pitch (bytes)
constexpr int A_ST = MT * LDP;              // activation rows per stage
constexpr int B_ST = NT * LDP;              // widened weight rows per stage
constexpr int S_ST = NT * KS;               // scale words per stage
constexpr int MAX_INT_SPREAD = 20;          // m (11 bits) << 20 stays below 2^31

// fp16 scale s = m * 2^(E-25) -> the integer +-m << (E - emin), i.e.
// s * 2^(25-emin); every step is exact (fp16 -> fp32, a power-of-two scaling,
// an integer of at most 31 bits back from fp32), and a zero scale gives 0
__device__ __forceinline__ int scale_int(uint16_t h, int emin)
{
    return (int)ldexpf(f16_to_f32(h), 25 - emin);
}

template <bool GATEUP, int GS>
__global__ __launch_bounds__(512, 2) void mfma_proj_kernel(ProjArgs a, const int2 *__restrict__ tiles,
                                                           const int32_t *__restrict__ n_tiles,
                                                           int mt_max, int n_blocks,
                                                           float *__restrict__ out, int ldo)
{
    __shared__ __align__(16) uint8_t lds_ab[2 * A_ST + 2 * B_ST];
    __shared__ float lds_s[2 * S_ST];
    __shared__ int s_slot[MT], s_row[MT];
    __shared__ float s_sc[MT];
    __shared__ int s_tile[8];
    __shared__ int s_emin[NT], s_emax[NT];
    uint8_t *lds_a = lds_ab, *lds_b = lds_ab + 2 * A_ST;

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
            const int n = NT * nb + 16 * tid;
            t = a.tile_base + (n >> 5) * a.pair_stride + ((n >> 4) & 1) * a.j_stride;
        }
        s_tile[tid] = t;
    }
    __syncthreads();

    const uint8_t *blob =
        reinterpret_cast<const uint8_t *>((e == a.ex.E) ? a.ex.shared : a.ex.ptrs[e]);
    const int K = a.K, KC = K >> 5, n_stages = KC / KS, G = KC / GS;
    const uint8_t *qbase = reinterpret_cast<const uint8_t *>(a.q);

    // global -> LDS per stage, one piece of each kind per thread: activations
    // 64 rows x 8 pieces of 16 B; weight nibbles 8 tiles x 4 chunks x 16 rows
    // of 16 B (widened to 32 B); scales 128 rows x KS/GS groups (threads past
    // that reload a valid scale and skip the store).  No branch around the
    // loads, so each LDS store waits for its own stage's loads only.
    const uint8_t *ga;
    int la;
    {
        const int tok = tid >> 3, seg = tid & 7;
        const int row = s_row[tok];
        ga = qbase + (size_t)(row < 0 ? s_row[0] : row) * K + seg * 16;
        la = tok * LDP + seg * 16;
    }
    const uint8_t *gb;
    int lb;
    {
        const int r = tid & 15, kcl = (tid >> 4) & 3, tj = tid >> 6;
        gb = blob + a.w_off + (size_t)s_tile[tj] * a.tile_w + kcl * 256 + r * 16;
        lb = (16 * tj + r) * LDP + kcl * 32;
    }
    constexpr int NG = KS / GS;
    const bool s_thread = tid < NT * NG;
    const uint16_t *gs_;
    int ls_;
    {
        const int sq = s_thread ? tid : 0;
        const int row = sq / NG, u = sq % NG;
        gs_ = reinterpret_cast<const uint16_t *>(blob + a.s_off + (size_t)s_tile[row >> 4] * a.tile_s) +
              u * 16 + (row & 15);
        ls_ = row * KS + u;
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
        *reinterpret_cast<uint4 *>(lds_a + (buf) * A_ST + la) = ra##P;            \
        {                                                                         \
            const uint4 w_ = rbv##P;                                              \
            *reinterpret_cast<uint4 *>(lds_b + (buf) * B_ST + lb) =               \
                make_uint4((w_.x << 4) & 0xf0f0f0f0u, (w_.y << 4) & 0xf0f0f0f0u,  \
                           (w_.z << 4) & 0xf0f0f0f0u, (w_.w << 4) & 0xf0f0f0f0u); \
            *reinterpret_cast<uint4 *>(lds_b + (buf) * B_ST + lb + 16) =          \
                make_uint4(w_.x & 0xf0f0f0f0u, w_.y & 0xf0f0f0f0u,                \
                           w_.z & 0xf0f0f0f0u, w_.w & 0xf0f0f0f0u);               \
        }                                                                         \
        if (s_thread)                                                             \
            lds_s[(buf) * S_ST + ls_] = (INTM) ? __int_as_float(scale_int(rs##P, em_)) \
                                               : f16_to_f32(rs##P) * 0.0625f;     \
    } while (0)
    // the K loop: stage st sits in LDS buffer st&1 while the loads of stages
    // st+1 (register set (st+1)&1, written to the other buffer at the end of
    // the stage) and st+2 (set st&1) are in flight; EPI(d, sword) folds one
    // group's 32x32 dots in.  The stage count is even (K is a multiple of
    // 256) and the loads past the last stage repeat it, so the loop is
    // straight-line code.
#define KSTAGE(P, Q, st, INTM, EPI)                                               \
    do {                                                                          \
        GLOAD(P, min((st) + 2, n_stages - 1));                                    \
        if (active) {                                                             \
            const uint8_t *A_ = lds_a + (P) * A_ST + arow * LDP + 16 * hh;        \
            const uint8_t *B_ = lds_b + (P) * B_ST + R * LDP + 16 * hh;           \
            const float *S_ = lds_s + (P) * S_ST + R * KS;                        \
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
        LSTORE(0, 0, INTM);                                                       \
        __syncthreads();                                                          \
        for (int st = 0; st < n_stages; st += 2) {                                \
            KSTAGE(0, 1, st, INTM, EPI);                                          \
            KSTAGE(1, 0, st + 1, INTM, EPI);                                      \
        }                                                                         \
    } while (0)

    // Exponent range of each weight row's nonzero scales.  The scales of a
    // tile are [group][16 rows] (fp16): wave w reads tile w, lane l the rows
    // [8(l>>5), 8(l>>5)+8) of groups (l&31) + 32i, 16 bytes per load, a batch
    // of SCAN_LOADS loads in flight at once (the first batch also beside the
    // first two stages' loads, which go out right after it); each lane marks
    // the exponents it sees per row in a 32-bit set (subnormals count as
    // exponent 1), the sets are OR-ed over the 32 lanes of each half-wave, and
    // the lowest and highest member are the row's Emin and Emax (99 and -99
    // for a row of zero scales).
    {
        constexpr int SCAN_LOADS = 8;
        const int hf = lane >> 5, p = lane & 31;
        const uint4 *sp = reinterpret_cast<const uint4 *>(blob + a.s_off +
                                                          (size_t)s_tile[wave] * a.tile_s) + hf;
        uint32_t eset[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        uint4 v[SCAN_LOADS];
        // (a batch issues only the loads whose groups start below G; lanes
        // whose group is past G load a valid group and ignore it)
#define SCAN_ISSUE(b)                                                             \
        _Pragma("unroll") for (int i = 0; i < SCAN_LOADS; ++i)                    \
            if ((b) + 32 * i < G)                                                 \
                v[i] = sp[2 * min((b) + 32 * i + p, G - 1)]
#define SCAN_MARK(b)                                                              \
        _Pragma("unroll") for (int i = 0; i < SCAN_LOADS; ++i) {                  \
            if ((b) + 32 * i >= G)                                                \
                break;                                                            \
            const bool ok_ = (b) + 32 * i + p < G;                                \
            const uint32_t wd_[4] = {v[i].x, v[i].y, v[i].z, v[i].w};             \
            _Pragma("unroll") for (int q = 0; q < 8; ++q) {                       \
                const uint32_t h_ = (wd_[q >> 1] >> (16 * (q & 1))) & 0xffffu;   \
                const uint32_t ef_ = (h_ >> 10) & 31u;                            \
                eset[q] |= (ok_ && (h_ & 0x7fffu)) ? (1u << (ef_ ? ef_ : 1u)) : 0u; \
            }                                                                     \
        }
        SCAN_ISSUE(0);
        GLOAD(0, 0);
        GLOAD(1, 1);
        __builtin_amdgcn_sched_barrier(0);      // keep those loads ahead of the marking
        SCAN_MARK(0);
        for (int b = 32 * SCAN_LOADS; b < G; b += 32 * SCAN_LOADS) {
            SCAN_ISSUE(b);
            SCAN_MARK(b);
        }
#undef SCAN_ISSUE
#undef SCAN_MARK
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            uint32_t m = eset[q];
            m |= (uint32_t)xor_lane<1>((int)m);
            m |= (uint32_t)xor_lane<2>((int)m);
            m |= (uint32_t)xor_lane<4>((int)m);
            m |= (uint32_t)xor_lane<8>((int)m);
            m |= (uint32_t)xor_lane<16>((int)m);
            eset[q] = m;
        }
        if (p == 0) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int row = 16 * wave + 8 * hf + q;
                s_emin[row] = eset[q] ? __builtin_ctz(eset[q]) : 99;
                s_emax[row] = eset[q] ? 31 - __builtin_clz(eset[q]) : -99;
            }
        }
    }
    __syncthreads();
    const int wide_row =
        (tid < NT && s_emax[tid] - s_emin[tid] > MAX_INT_SPREAD) ? 1 : 0;   // all-zero rows: -198
    const bool wide = __syncthreads_or(wide_row) != 0;
    const int em_ = s_emin[(s_thread ? tid : 0) / NG];

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

    // result register r of lane l: activation row 8(r/4)+4(l/32)+r%4; the
    // outputs are read once by the next launch, so they are stored with the
    // non-temporal hint
    if (GATEUP) {
        // up waves (wb 2, 3) hand their sums to the gate waves (wb 0, 1)
        double *xch = reinterpret_cast<double *>(lds_ab);   // [2][2][16][64]
        if (active && wb >= 2) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                xch[(((wb - 2) * 2 + mb) * 16 + r) * 64 + lane] = acc[r];
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
            const double U = xch[((wb * 2 + mb) * 16 + r) * 64 + lane] * sc;
            __builtin_nontemporal_store((float)(G_ / (1.0 + exp(-G_)) * U), out + (size_t)slot * ldo + 64 * nb + 32 * wb + li);
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
            __builtin_nontemporal_store((float)(acc[r] * (double)s_sc[tok]), out + (size_t)slot * ldo + NT * nb + 32 * wb + li);
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
    const int2 *tl = reinterpret_cast<const int2 *>(c->tiles);
    const int grid = grid_for(mt_max, F / 64);
    if (a.group_shift)
        launch(mfma_proj_kernel<true, 2>, grid, 512, 0, st, a, tl, c->n_tiles, mt_max, F / 64, h, ldh);
    else
        launch(mfma_proj_kernel<true, 1>, grid, 512, 0, st, a, tl, c->n_tiles, mt_max, F / 64, h, ldh);
    return hipGetLastError();
}

hipError_t launch_proj_mfma(const ProjArgs &a, const moe_ctx *c, int T, int n_rows, hipStream_t st)
{
    // inspection projections use a single blob (one expert holding T rows)
    const int mt_max = (a.ex.E == 0) ? (T + MT - 1) / MT : tiles_bound(c, T);
    const int2 *tl = reinterpret_cast<const int2 *>(c->tiles);
    const int grid = grid_for(mt_max, n_rows / NT);
    if (a.group_shift)
        launch(mfma_proj_kernel<false, 2>, grid, 512, 0, st, a, tl, c->n_tiles, mt_max, n_rows / NT, a.out, a.ldo);
    else
        launch(mfma_proj_kernel<false, 1>, grid, 512, 0, st, a, tl, c->n_tiles, mt_max, n_rows / NT, a.out, a.ldo);
    return hipGetLastError();
}

}  // namespace moe
