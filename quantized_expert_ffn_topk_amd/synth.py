"""Seeded synthetic inputs for the quantised MoE layer.

This module only draws random numbers and turns them into the input formats
of the layer (bf16 activations, fp32 router weights and bias, int4 / MXFP4
expert weights, routing traces).  It holds none of the layer's own arithmetic
(no activation quantisation, no router, no projections); it is shared by the
tests, the benchmark and the oracle side alike.

Every tensor has its own named random stream:
``numpy.random.Generator(PCG64(SeedSequence(seed, spawn_key=<hash of name>)))``.
"""
import hashlib

import numpy as np


def stream(seed, *name):
    """Independent generator for the tensor called ``name`` under ``seed``."""
    key = hashlib.sha256("/".join(str(n) for n in name).encode()).digest()
    spawn = tuple(int.from_bytes(key[i:i + 4], "little") for i in range(0, 16, 4))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=spawn)))


# ---------------------------------------------------------------------------
# format conversions used to build inputs
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a):
    """Round fp32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = (u & 0x7F800000) == 0x7F800000
    nan &= (u & 0x007FFFFF) != 0
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quant_int4_groups(w, g):
    """Group-wise symmetric int4 of a [N,K] fp32 matrix along K.

    Per group of g inputs: scale = fp16(amax/7) (round to nearest even); codes
    q = clamp(rint(w/scale), -8, 7), all zero when the scale is zero.
    Returns (q int8 [N,K], scale fp16 bits uint16 [N,K/g]).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    wg = w.reshape(N, K // g, g)
    amax = np.abs(wg).max(axis=-1)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s = s16.astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s)
    q = np.rint(wg / safe[..., None])
    q = np.where((s == 0)[..., None], 0.0, q)
    q = np.clip(q, -8, 7).astype(np.int8).reshape(N, K)
    return q, s16.view(np.uint16)


_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def quant_mxfp4(w):
    """OCP Microscaling v1.0 MXFP4 of a [N,K] fp32 matrix along K.

    Per block of 32: X = floor(log2(amax)) - 2 clamped to [-127,127]
    (emax of E2M1 is 2), E8M0 byte = X + 127; each element is rounded to the
    nearest E2M1 value of w * 2^-X (ties to the even code), saturating at 6.
    Returns (codes uint8 [N,K] low nibble, e8m0 uint8 [N,K/32]).
    """
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    wb = w.reshape(N, K // 32, 32)
    amax = np.abs(wb).max(axis=-1)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    X = np.clip(X, -127, 127).astype(np.int64)
    v = wb * np.ldexp(1.0, -X)[..., None]
    mag = np.minimum(np.abs(v), 6.0)
    # nearest grid point, ties to the even code
    d = np.abs(mag[..., None] - _E2M1_MAG)
    best = np.argmin(d, axis=-1)
    dmin = np.take_along_axis(d, best[..., None], -1)[..., 0]
    nxt = np.minimum(best + 1, 7)
    tie = (np.take_along_axis(d, nxt[..., None], -1)[..., 0] == dmin) & (nxt != best)
    best = np.where(tie & (best % 2 == 1), nxt, best)
    code = best.astype(np.uint8)
    code = np.where((v < 0) & (code != 0), code | 8, code).astype(np.uint8)
    return code.reshape(N, K), (X + 127).astype(np.uint8)


# ---------------------------------------------------------------------------
# tensors of one layer
# ---------------------------------------------------------------------------
def activations(seed, T, H, tag="x"):
    """x ~ N(0,1) rounded to bf16: uint16 bits [T,H]."""
    r = stream(seed, tag, T, H)
    return f32_to_bf16_bits(r.standard_normal((T, H), dtype=np.float32))


def router_weights(seed, E, H, w_std=0.02, bias_std=0.01, tag="router"):
    r = stream(seed, tag, "W", E, H)
    W = (r.standard_normal((E, H), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    rb = stream(seed, tag, "b", E)
    b = (rb.standard_normal(E, dtype=np.float32) * np.float32(bias_std)).astype(np.float32)
    return W, b


def uniform_bias(seed, E, half_width=0.01, tag="router"):
    r = stream(seed, tag, "ub", E)
    return r.uniform(-half_width, half_width, E).astype(np.float32)


def expert_int4(seed, e, H, F, g, std=0.02, tag="expert"):
    """One routed (e >= 0) or shared (e = -1) expert, weights N(0, std)
    quantised to group-g int4.  gate/up are [F,H], down is [H,F]."""
    out = {}
    for name, shape in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
        r = stream(seed, tag, e, name, H, F)
        w = r.standard_normal(shape, dtype=np.float32) * np.float32(std)
        q, s = quant_int4_groups(w, g)
        out["q_" + name] = q
        out["s_" + name] = s
    return out


def expert_mxfp4(seed, e, H, F, std=0.02, tag="mxexpert"):
    out = {}
    for name, shape in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
        r = stream(seed, tag, e, name, H, F)
        w = r.standard_normal(shape, dtype=np.float32) * np.float32(std)
        c, x = quant_mxfp4(w)
        out["c_" + name] = c
        out["e_" + name] = x
    return out


# ---------------------------------------------------------------------------
# routing skew
# ---------------------------------------------------------------------------
ZIPF_S = 1.1
# Bias slope of the skewed-prefill workload: b_e = BETA * ln p_rank(e) plus the
# N(0, 0.01) per-expert noise.  Chosen offline so that 4096 tokens routed with
# top-8 over 256 experts give loads close to capped Zipf(1.1) (top expert near
# every token, a tail of a few dozen rows); the realised histogram is reported
# by the benchmark.
ZIPF_BETA = 0.13


def zipf_probs(E, s=ZIPF_S):
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def zipf_bias(seed, E, beta=ZIPF_BETA, s=ZIPF_S, tag="zipf"):
    """Selection bias that skews expert load like Zipf(s) over a seeded
    permutation of the experts."""
    r = stream(seed, tag, "perm", E)
    perm = r.permutation(E)               # perm[rank] = expert
    lp = np.log(zipf_probs(E, s))
    lp = lp - lp.mean()
    b = np.empty(E, np.float64)
    b[perm] = beta * lp
    noise = stream(seed, tag, "noise", E).standard_normal(E) * 0.01
    return (b + noise).astype(np.float32)


def zipf_trace(seed, L, E, k, steps, corr=0.7, s=ZIPF_S, tag="trace", model_seed=None):
    """Expert-streaming trace: per (step, layer) k distinct experts drawn by
    Zipf(s) rank over a per-layer seeded permutation; for layer l+1 each rank
    slot keeps, with probability corr, the successor (same Zipf rank in the
    next layer's permutation) of the expert at that rank in layer l.
    The permutations (which experts are hot: the model) come from model_seed
    (default: seed), the draws from seed, so two traces with one model_seed
    and different seeds are two sessions of the same model.
    Returns (demand [steps,L,k] int32, predict [steps,L,k] int32) where
    predict[t,l] is the successor set of demand[t,l], i.e. the lookahead
    guess for layer l+1 (for l = L-1: layer 0 of step t+1)."""
    r = stream(seed, tag, L, E, k, steps)
    ms = seed if model_seed is None else model_seed
    perms = np.stack([stream(ms, tag, "perm", l, E).permutation(E) for l in range(L)])
    rank_of = np.empty_like(perms)
    for l in range(L):
        rank_of[l, perms[l]] = np.arange(E)
    p = zipf_probs(E, s)
    cdf = np.cumsum(p)

    def draw_rank():
        return int(min(np.searchsorted(cdf, r.random()), E - 1))

    demand = np.empty((steps, L, k), np.int32)
    predict = np.empty((steps, L, k), np.int32)

    def succ(l, e):
        nl = (l + 1) % L
        return perms[nl, rank_of[l, e]]

    prev = None
    for t in range(steps):
        for l in range(L):
            chosen = []
            for i in range(k):
                cand = None
                if prev is not None and r.random() < corr:
                    cand = int(prev[i])
                while cand is None or cand in chosen:
                    cand = int(perms[l, draw_rank()])
                chosen.append(cand)
            demand[t, l] = chosen
            predict[t, l] = [succ(l, e) for e in chosen]
            prev = predict[t, l]
    return demand, predict


def forcing_bias(E, ids, boost=4.0):
    """Selection bias that makes the router pick exactly ``ids`` (when the
    sigmoid scores are in (0,1) and no other bias exceeds 0)."""
    b = np.zeros(E, np.float32)
    b[np.asarray(ids)] = np.float32(boost)
    return b
