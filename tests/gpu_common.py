"""Shared helpers of the GPU parity tests: building a layer from seeded
synthetic inputs and comparing its outputs with the oracle's."""
import numpy as np

import oracle
from quantized_expert_ffn_topk_amd import abi, synth
from quantized_expert_ffn_topk_amd.layer import Layer, make_desc

# Spec bar for floating-point layer outputs: max |y - r| / max |r|.
MAX_REL_ERR = 2e-3


class Case:
    """Inputs of one int4 layer: distinct experts plus a map (expert e uses
    distinct[emap[e]]), router weights and bias, tokens."""

    def __init__(self, seed, T, H, F, E, k, n_shared, g=32, r=1.0, n_distinct=None,
                 bias=None, x=None):
        self.T, self.H, self.F, self.E, self.k, self.n_shared, self.g, self.r = \
            T, H, F, E, k, n_shared, g, r
        nd = E if n_distinct is None else n_distinct
        self.distinct = [synth.expert_int4(seed, e, H, F, g) for e in range(nd)]
        self.emap = [e % nd for e in range(E)]
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


def check_routing(idx_gpu, w_gpu, idx_orc, w_orc, choice, tie_eps=1e-12):
    """Indices must match exactly; where the oracle's k-th and (k+1)-th choice
    values are closer than tie_eps, any order that is valid under the oracle's
    values is accepted.  Weights within a few fp32 ulps."""
    T, k = idx_orc.shape
    for t in range(T):
        if np.array_equal(idx_gpu[t], idx_orc[t]):
            continue
        c = choice[t]
        srt = np.sort(c)[::-1]
        gaps = np.abs(np.diff(srt[:k + 1]))
        assert gaps.min() < tie_eps, "token %d: routing differs with no near-tie: %s vs %s" % (
            t, idx_gpu[t], idx_orc[t])
        assert len(set(idx_gpu[t].tolist())) == k
        cg = c[idx_gpu[t]]
        assert np.all(cg >= srt[k - 1] - tie_eps)
    np.testing.assert_allclose(w_gpu, w_orc, rtol=4e-7, atol=1e-30)


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
