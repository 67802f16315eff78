// pack.cpp -- host-side packing of expert weights into the blob layout
// described in moe_internal.h.  No GPU is needed.
//
// Source of the formats: "Run a 744B-parameter model on your own machine"
// (aifrontierpost), "Step 3": group-scaled int4 expert containers, and native
// MXFP4 experts for Kimi K3 (OCP Microscaling v1.0: E2M1 elements with one
// E8M0 power-of-two scale per 32).
#include <cstring>

#include "host_common.h"

using namespace moe;

extern "C" size_t moe_blob_bytes(const moe_layer_desc *desc)
{
    if (validate_desc(desc) != MOE_OK)
        return 0;
    return blob_layout(desc->hidden, desc->ffn, desc->group, desc->wfmt).total;
}

// fp16 exponent field of a finite nonzero value, with subnormals counted as 1.
static int f16_exp(uint16_t h)
{
    int e = (h >> 10) & 31;
    return e == 0 ? 1 : e;
}

// Checks the scales of one [N, K/group] matrix: finite, and per row the nonzero
// scales span few enough binades that the sum over groups of (int32 group sum
// x scale) is exactly representable in fp64: each term is an integer of at
// most 26 bits (|group sum| < 2^15 for g = 32, < 2^16 for g = 64, times an
// 11-bit significand) times 2^(e-25); the sum of G terms adds ceil(log2 G) bits.
static moe_status check_scales(const uint16_t *s, int N, int K, int g, const char *what)
{
    const int G = K / g;
    int lg = 0;
    while ((1 << lg) < G)
        ++lg;
    const int term_bits = (g == 64) ? 27 : 26;
    for (int n = 0; n < N; ++n) {
        int emin = 99, emax = -99;
        for (int j = 0; j < G; ++j) {
            uint16_t h = s[(size_t)n * G + j];
            if (((h >> 10) & 31) == 31)
                return fail(MOE_E_INVAL, "%s scale [%d,%d] is not finite", what, n, j);
            if ((h & 0x7fff) == 0)
                continue;
            int e = f16_exp(h);
            emin = e < emin ? e : emin;
            emax = e > emax ? e : emax;
        }
        if (emax >= emin && term_bits + lg + (emax - emin) > 53)
            return fail(MOE_E_INVAL,
                        "%s row %d: scales span %d binades; exact group sums need <= %d", what,
                        n, emax - emin, 53 - term_bits - lg);
    }
    return MOE_OK;
}

static moe_status check_codes(const int8_t *q, size_t n, const char *what)
{
    for (size_t i = 0; i < n; ++i)
        if (q[i] < -8 || q[i] > 7)
            return fail(MOE_E_INVAL, "%s code %d at %zu outside [-8,7]", what, (int)q[i], i);
    return MOE_OK;
}

// One 16-row tile of an int4 matrix q[N,K] (rows r0..r0+15) into dst.
static void pack_tile_int4(const int8_t *q, int K, int r0, uint8_t *dst)
{
    const int KC = K / 32;
    for (int kc = 0; kc < KC; ++kc)
        for (int r = 0; r < 16; ++r) {
            const int8_t *src = q + (size_t)(r0 + r) * K + (size_t)kc * 32;
            uint8_t *o = dst + ((size_t)kc * 16 + r) * 16;
            for (int j = 0; j < 16; ++j) {
                uint8_t lo = (uint8_t)(src[j] & 15), hi = (uint8_t)(src[j + 16] & 15);
                o[j] = (uint8_t)(lo | (hi << 4));
            }
        }
}

static void pack_tile_scales_f16(const uint16_t *s, int K, int g, int r0, uint8_t *dst)
{
    const int G = K / g;
    uint16_t *o = reinterpret_cast<uint16_t *>(dst);
    for (int j = 0; j < G; ++j)
        for (int r = 0; r < 16; ++r)
            o[(size_t)j * 16 + r] = s[(size_t)(r0 + r) * G + j];
}

extern "C" moe_status moe_pack_expert_int4(const moe_layer_desc *desc, const int8_t *q_gate,
                                           const uint16_t *s_gate, const int8_t *q_up,
                                           const uint16_t *s_up, const int8_t *q_down,
                                           const uint16_t *s_down, void *blob_host)
{
    moe_status st = validate_desc(desc);
    if (st)
        return st;
    if (desc->wfmt != MOE_WFMT_INT4)
        return fail(MOE_E_INVAL, "desc is not an int4 layer");
    if (!q_gate || !s_gate || !q_up || !s_up || !q_down || !s_down || !blob_host)
        return fail(MOE_E_INVAL, "NULL argument");
    const int H = desc->hidden, F = desc->ffn, g = desc->group;
    const size_t n1 = (size_t)F * H;
    if ((st = check_codes(q_gate, n1, "gate")) || (st = check_codes(q_up, n1, "up")) ||
        (st = check_codes(q_down, n1, "down")))
        return st;
    if ((st = check_scales(s_gate, F, H, g, "gate")) || (st = check_scales(s_up, F, H, g, "up")) ||
        (st = check_scales(s_down, H, F, g, "down")))
        return st;
    const BlobLayout L = blob_layout(H, F, g, MOE_WFMT_INT4);
    uint8_t *b = static_cast<uint8_t *>(blob_host);
    for (int nb = 0; nb < F / 16; ++nb) {
        pack_tile_int4(q_gate, H, nb * 16, b + L.gu_w + (size_t)(2 * nb) * L.gu_tile_w);
        pack_tile_int4(q_up, H, nb * 16, b + L.gu_w + (size_t)(2 * nb + 1) * L.gu_tile_w);
        pack_tile_scales_f16(s_gate, H, g, nb * 16, b + L.gu_s + (size_t)(2 * nb) * L.gu_tile_s);
        pack_tile_scales_f16(s_up, H, g, nb * 16, b + L.gu_s + (size_t)(2 * nb + 1) * L.gu_tile_s);
    }
    for (int t = 0; t < H / 16; ++t) {
        pack_tile_int4(q_down, F, t * 16, b + L.dn_w + (size_t)t * L.dn_tile_w);
        pack_tile_scales_f16(s_down, F, g, t * 16, b + L.dn_s + (size_t)t * L.dn_tile_s);
    }
    return MOE_OK;
}

// MXFP4: byte j of a chunk holds inputs 2j (low nibble) and 2j+1 (high).
static void pack_tile_mx(const uint8_t *c, int K, int r0, uint8_t *dst)
{
    const int KC = K / 32;
    for (int kc = 0; kc < KC; ++kc)
        for (int r = 0; r < 16; ++r) {
            const uint8_t *src = c + (size_t)(r0 + r) * K + (size_t)kc * 32;
            uint8_t *o = dst + ((size_t)kc * 16 + r) * 16;
            for (int j = 0; j < 16; ++j)
                o[j] = (uint8_t)((src[2 * j] & 15) | ((src[2 * j + 1] & 15) << 4));
        }
}

static void pack_tile_e8m0(const uint8_t *e, int K, int r0, uint8_t *dst)
{
    const int KC = K / 32;
    for (int kc = 0; kc < KC; ++kc)
        for (int r = 0; r < 16; ++r)
            dst[(size_t)kc * 16 + r] = e[(size_t)(r0 + r) * KC + kc];
}

static moe_status check_mx(const uint8_t *c, const uint8_t *e, size_t n, const char *what)
{
    for (size_t i = 0; i < n; ++i)
        if (c[i] > 15)
            return fail(MOE_E_INVAL, "%s E2M1 code %d at %zu is not a nibble", what, (int)c[i], i);
    for (size_t i = 0; i < n / 32; ++i)
        if (e[i] == 0xff)
            return fail(MOE_E_INVAL, "%s E8M0 scale at %zu is NaN (0xFF)", what, i);
    return MOE_OK;
}

extern "C" moe_status moe_pack_expert_mxfp4(const moe_layer_desc *desc, const uint8_t *c_gate,
                                            const uint8_t *e_gate, const uint8_t *c_up,
                                            const uint8_t *e_up, const uint8_t *c_down,
                                            const uint8_t *e_down, void *blob_host)
{
    moe_status st = validate_desc(desc);
    if (st)
        return st;
    if (desc->wfmt != MOE_WFMT_MXFP4)
        return fail(MOE_E_INVAL, "desc is not an mxfp4 layer");
    if (!c_gate || !e_gate || !c_up || !e_up || !c_down || !e_down || !blob_host)
        return fail(MOE_E_INVAL, "NULL argument");
    const int H = desc->hidden, F = desc->ffn;
    const size_t n1 = (size_t)F * H;
    if ((st = check_mx(c_gate, e_gate, n1, "gate")) || (st = check_mx(c_up, e_up, n1, "up")) ||
        (st = check_mx(c_down, e_down, n1, "down")))
        return st;
    const BlobLayout L = blob_layout(H, F, 32, MOE_WFMT_MXFP4);
    uint8_t *b = static_cast<uint8_t *>(blob_host);
    for (int nb = 0; nb < F / 16; ++nb) {
        pack_tile_mx(c_gate, H, nb * 16, b + L.gu_w + (size_t)(2 * nb) * L.gu_tile_w);
        pack_tile_mx(c_up, H, nb * 16, b + L.gu_w + (size_t)(2 * nb + 1) * L.gu_tile_w);
        pack_tile_e8m0(e_gate, H, nb * 16, b + L.gu_s + (size_t)(2 * nb) * L.gu_tile_s);
        pack_tile_e8m0(e_up, H, nb * 16, b + L.gu_s + (size_t)(2 * nb + 1) * L.gu_tile_s);
    }
    for (int t = 0; t < H / 16; ++t) {
        pack_tile_mx(c_down, F, t * 16, b + L.dn_w + (size_t)t * L.dn_tile_w);
        pack_tile_e8m0(e_down, F, t * 16, b + L.dn_s + (size_t)t * L.dn_tile_s);
    }
    return MOE_OK;
}
