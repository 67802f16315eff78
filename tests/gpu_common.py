"""Shared helpers of the GPU parity tests: building a layer from seeded
synthetic inputs and comparing its outputs with the oracle's."""
import concurrent.futures as cf
import os

import numpy as np

import oracle
from quantized_expert_ffn_topk_amd import abi, synth
from quantized_expert_ffn_topk_amd.layer import Layer, make_desc

# Spec bar for floating-point layer outputs: max |y - r| / max |r|.
MAX_REL_ERR = 2e-3


def expert_map(seed, E, nd):
    """Routed expert e uses distinct weight set emap[e].  With fewer distinct
    sets than experts the map is a seeded random one (every set used), so a
    kernel that reads the blob of a wrong expert id (off by one, a multiple of
    nd, a wrong stride) meets different weights almost surely."""
    if nd >= E:
        return list(range(E))
    r = np.random.default_rng([seed, E, nd, 977])
    m = np.concatenate([np.arange(nd), r.integers(0, nd, E - nd)])
    r.shuffle(m)
    return [int(v) for v in m]


def oracle_threads():
    # at most 16 host threads (one GPU's share of a multi-GPU host); the oracle
    # itself stays single-threaded per call, independent calls run side by side
    return max(1, min(16, os.cpu_count() or 1))


def oracle_rows_parallel(fn, x, tokens, **kw):
    """Runs fn(x[chunk], **kw) -> (idx, w, out) for chunks of the token rows
    `tokens` on a thread pool (ctypes releases the GIL inside the C oracle)
    and stacks the results in token order."""
    tokens = np.asarray(tokens)
    n = oracle_threads()
    chunks = [c for c in np.array_split(tokens, min(n, len(tokens))) if len(c)]
    with cf.ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(lambda c: fn(x[c], **kw), chunks))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))


class Case:
    """Inputs of one int4 layer: distinct experts plus a map (expert e uses
    distinct[emap[e]]), router weights and bias, tokens."""

    def __init__(self, seed, T, H, F, E, k, n_shared, g=32, r=1.0, n_distinct=None,
                 bias=None, x=None):
        self.T, self.H, self.F, self.E, self.k, self.n_shared, self.g, self.r = \
            T, H, F, E, k, n_shared, g, r
        nd = E if n_distinct is None else n_distinct
        self.distinct = [synth.expert_int4(seed, e, H, F, g) for e in range(nd)]
        self.emap = expert_map(seed, E, nd)
        self.shared = synth.expert_int4(seed, -1, H, F, g) if n_shared else None
        self.Wr, b = synth.router_weights(seed, E, H)
        self.b = b if bias is None else np.asarray(bias, np.float32)
        self.x = synth.activations(seed, T, H) if x is None else x

    def desc(self, out_dtype=abi.DT_F32):
        return make_desc(self.H, self.F, self.E, self.k, self.n_shared, self.g, self.r,
                         abi.WFMT_INT4, out_dtype)

    def layer(self, max_tokens=None, path=abi.PATH_AUTO, out_dtype=abi.DT_F32):
        return Layer(self.desc(out_dtype), self.Wr, self.b, self.distinct, self.shared, self.emap,
                     max_tokens=max_tokens or self.T, path=path)

    def oracle_layer(self, out_rows=None):
        return oracle.layer(self.x, self.Wr, self.b, self.distinct, self.shared, self.k, self.r,
                            self.g, out_rows=out_rows, expert_map=self.emap)

    def oracle_router(self):
        return oracle.router(self.x, self.Wr, self.b, self.k, self.r, want=True)


def check_routing(idx_gpu, w_gpu, idx_orc, w_orc, choice, tie_eps=1e-12, r=None):
    """Indices must match the oracle's exactly, in rank order.  The one
    exemption is the near-tie of the design reading on router precision: where
    the oracle's k-th and (k+1)-th choice values (in its own order: value
    descending, index ascending) are closer than tie_eps, the fp64 sums of the
    GPU may order them differently.  Then the ranks before the run of
    near-equal values around that boundary must still equal the oracle's, and
    the remaining ranks must be distinct members of that run.  Weights of
    tokens with identical routing are within a few fp32 ulps of the oracle's;
    the weights of an exempted token are checked to sum to the routed scale r
    (when given)."""
    T, k = idx_orc.shape
    same = np.ones(T, bool)
    for t in range(T):
        if np.array_equal(idx_gpu[t], idx_orc[t]):
            continue
        same[t] = False
        c = np.asarray(choice[t], np.float64)
        order = np.lexsort((np.arange(c.size), -c))        # value desc, index asc
        assert np.array_equal(order[:k], idx_orc[t]), "oracle order is not its own ranking"
        assert k < c.size, "token %d: all experts selected, yet routing differs" % t
        cs = c[order]
        assert cs[k - 1] - cs[k] < tie_eps, \
            "token %d: routing differs with no near-tie at the k/(k+1) boundary: %s vs %s" % (
                t, idx_gpu[t], idx_orc[t])
        a = k - 1
        while a > 0 and cs[a - 1] - cs[a] < tie_eps:
            a -= 1
        b = k
        while b + 1 < c.size and cs[b] - cs[b + 1] < tie_eps:
            b += 1
        assert np.array_equal(idx_gpu[t, :a], idx_orc[t, :a]), \
            "token %d: ranks before the tied run differ: %s vs %s" % (t, idx_gpu[t], idx_orc[t])
        tail = idx_gpu[t, a:].tolist()
        assert len(set(tail)) == len(tail), "token %d: repeated expert" % t
        assert set(tail) <= set(order[a:b + 1].tolist()), \
            "token %d: ranks %d.. are not from the tied run" % (t, a)
        if r is not None:
            assert abs(float(np.sum(w_gpu[t], dtype=np.float64)) - r) <= 1e-6 * max(r, 1.0)
    np.testing.assert_allclose(w_gpu[same], w_orc[same], rtol=4e-7, atol=1e-30)


def rel_err(y, r):
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    den = np.abs(r).max()
    return float(np.abs(y - r).max() / den) if den > 0 else float(np.abs(y).max())


def check_out(out_gpu, out_orc, min_exact=0.999):
    e = rel_err(out_gpu, out_orc)
    assert e <= MAX_REL_ERR, "max relative error %.3g" % e
    exact = float(np.mean(out_gpu.view(np.uint32) == out_orc.astype(np.float32).view(np.uint32)))
    assert exact >= min_exact, "only %.5f of outputs bit-exact (max rel err %.3g)" % (exact, e)
    return e, exact


def check_bf16_out(got_bits, want_f32, same_rounding=True):
    """bf16 output = the fp32 result rounded to nearest even.  With
    same_rounding (kernels whose fp32 sums are within a few fp32 ulps of the
    oracle's), every element equals the oracle's fp32 rounded the same way,
    except where the oracle's value lies next to a rounding midpoint (within
    1e-4 of its own magnitude or 1e-5 of the largest output: there the GPU's
    fp32 sum may fall on the other side): then one bf16 step apart.  In every
    case the output must be the rounding of a value within the 2e-3 bar: max
    over elements of (|y - r| - half a bf16 step of y) / max |r| <= 2e-3, r the
    oracle's fp32.  Returns that figure and the fraction equal to the oracle's
    rounding."""
    want_bits = synth.f32_to_bf16_bits(want_f32)
    got = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    wb = synth.bf16_bits_to_f32(want_bits).astype(np.float64)
    r = np.asarray(want_f32, np.float64)
    diff = got != wb
    if same_rounding and diff.any():
        # at most one bf16 step apart, and only next to a midpoint
        step = np.abs(got[diff] - wb[diff])
        ulp = np.abs(np.spacing(wb[diff].astype(np.float32)).astype(np.float64)) * 65536
        assert np.all(step <= ulp * 1.0000001), "more than one bf16 step apart"
        mid = 0.5 * (got[diff] + wb[diff])
        near = np.maximum(1e-4 * np.abs(r[diff]), 1e-5 * np.abs(r).max())
        assert np.all(np.abs(r[diff] - mid) <= near), \
            "bf16 differs away from a rounding midpoint"
    # half a bf16 step around each output (the larger one at a binade edge)
    half = 0.5 * np.abs(np.spacing(np.abs(got).astype(np.float32)).astype(np.float64)) * 65536
    den = np.abs(r).max()
    e = float(np.maximum(np.abs(got - r) - half, 0.0).max() / den) if den > 0 else 0.0
    assert e <= MAX_REL_ERR, "bf16 output %.3g away from the oracle beyond its rounding" % e
    return e, float(np.mean(~diff))
