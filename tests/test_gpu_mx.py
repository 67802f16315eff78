"""GPU parity of the MXFP4 expert path (E2M1 weights with E8M0 scales per 32,
bf16 activations) through the C ABI against the oracle: routing, the bf16
SwiGLU rows, the layer outputs, given routing, and the wide MXFP4 layer at full
size on sampled outputs."""
import numpy as np
import pytest

import oracle
from quantized_expert_ffn_topk_amd import abi, synth
from quantized_expert_ffn_topk_amd.layer import Layer, make_desc
from tests.gpu_common import MAX_REL_ERR, check_routing, rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


class MxCase:
    def __init__(self, seed, T, H, F, E, k, n_shared, r=1.0, n_distinct=None, x=None):
        self.T, self.H, self.F, self.E, self.k, self.n_shared, self.r = T, H, F, E, k, n_shared, r
        nd = E if n_distinct is None else n_distinct
        self.distinct = [synth.expert_mxfp4(seed, e, H, F) for e in range(nd)]
        self.emap = [e % nd for e in range(E)]
        self.shared = synth.expert_mxfp4(seed, -1, H, F) if n_shared else None
        self.Wr, _ = synth.router_weights(seed, E, H)
        self.b = synth.uniform_bias(seed, E)
        self.x = synth.activations(seed, T, H) if x is None else x

    def layer(self, max_tokens=None, out_dtype=abi.DT_F32):
        desc = make_desc(self.H, self.F, self.E, self.k, self.n_shared, 32, self.r,
                         abi.WFMT_MXFP4, out_dtype)
        return Layer(desc, self.Wr, self.b, self.distinct, self.shared, self.emap,
                     max_tokens=max_tokens or self.T)

    def oracle_layer(self, out_rows=None):
        return oracle.mx_layer(self.x, self.Wr, self.b, self.distinct, self.shared, self.k,
                               self.r, out_rows=out_rows, expert_map=self.emap)


def _check_mx_out(got, want):
    # fp32 MFMA accumulation against the oracle's fp64 sums: within the
    # spec bar, not bit-exact
    e = rel_err(got, want)
    assert e <= MAX_REL_ERR, "max relative error %.3g" % e
    return e


@pytest.mark.parametrize("T,shared", [(1, 1), (5, 0), (23, 1)])
def test_mx_layer_matches_oracle(T, shared):
    c = MxCase(31, T, 512, 256, 16, 4, shared, r=1.5)
    lay = c.layer()
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch = oracle.router(c.x, c.Wr, c.b, c.k, c.r, want=True)
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch)
    e = _check_mx_out(out.cpu().numpy(), out_o)
    print("mx layer T=%d: max rel err %.3g" % (T, e))
    lay.close()


def test_mx_swiglu_rows_match_oracle():
    # bf16 h rows: equal to the oracle's except where the fp32 projection sits
    # at a bf16 rounding boundary (then one bf16 ulp apart)
    c = MxCase(32, 6, 1024, 512, 8, 2, 1)
    lay = c.layer()
    idx, _, _ = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    S = c.k + 1
    hb = lay.debug_read(7, (c.T, S, c.F), torch.int16).cpu().numpy().view(np.uint16)
    ig = idx.cpu().numpy()
    xf = synth.bf16_bits_to_f32(c.x)
    n_diff = 0
    for t in range(c.T):
        for i in range(S):
            ex = c.shared if i == c.k else c.distinct[c.emap[ig[t, i]]]
            want = oracle.mx_expert(xf[t], ex)["h_bf16"]
            d = np.abs(hb[t, i].astype(np.int32) - want.astype(np.int32))
            assert d.max() <= 1, (t, i)
            n_diff += int((d != 0).sum())
    assert n_diff <= 0.01 * c.T * S * c.F
    lay.close()


def test_mx_expert_ffn_given_routing_and_determinism():
    c = MxCase(33, 4, 512, 256, 12, 3, 1, r=2.0)
    lay = c.layer()
    xd = lay.x_tensor(c.x)
    idx, w, out1 = lay.forward(xd)
    out2 = lay.ffn(xd, idx, w)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32))
    lay.close()


def test_mx_bf16_output():
    c = MxCase(34, 3, 512, 256, 8, 2, 1)
    lay = c.layer(out_dtype=abi.DT_BF16)
    _, _, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    _, _, out_o = c.oracle_layer()
    got = synth.bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16))
    assert rel_err(got, out_o) <= 2 ** -8 + MAX_REL_ERR
    lay.close()


def test_mx_wide_layer_full_size_sampled():
    # MXFP4 wide layer: hidden 7168, 384 routed + 1 shared, F 2048, top-8, 64
    # tokens, uniform routing bias.  Routing checked for every token, outputs
    # of 3 sampled tokens on 64 sampled columns against the oracle.
    H, F, E, k, T = 7168, 2048, 384, 8, 64
    c = MxCase(0, T, H, F, E, k, 1, r=1.0, n_distinct=3)
    lay = c.layer()
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, lg, sc, ch = oracle.router(c.x, c.Wr, c.b, k, c.r, want=True)
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch)
    rng = np.random.default_rng(2)
    toks = np.sort(rng.choice(T, 3, replace=False))
    cols = np.sort(rng.choice(H, 64, replace=False)).astype(np.int32)
    sub = MxCase(0, 3, H, F, E, k, 1, r=1.0, n_distinct=3, x=c.x[toks])
    sub.distinct, sub.shared, sub.Wr, sub.b = c.distinct, c.shared, c.Wr, c.b
    _, _, out_o = sub.oracle_layer(out_rows=cols)
    e = _check_mx_out(out.cpu().numpy()[toks][:, cols], out_o)
    print("mx wide layer: max rel err %.3g on sampled outputs" % e)
    lay.close()
