"""GPU parity of the MXFP4 expert path (E2M1 weights with E8M0 scales per 32,
bf16 activations) through the C ABI against the oracle: routing, the bf16
SwiGLU rows, the layer outputs, given routing, and the wide MXFP4 layer at full
size on sampled outputs.  Both kernels are checked: the MX MFMA (default;
activations split into two E4M3 parts, the MFMA's own internal sums) and the
bf16 MFMA on exactly widened weights (MOE_PATH_MX_BF16)."""
import numpy as np
import pytest

import oracle
from quantized_expert_ffn_topk_amd import abi, synth
from quantized_expert_ffn_topk_amd.layer import Layer, make_desc
from tests.gpu_common import (MAX_REL_ERR, check_bf16_out, check_routing, expert_map,
                               oracle_rows_parallel, rel_err)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


class MxCase:
    def __init__(self, seed, T, H, F, E, k, n_shared, r=1.0, n_distinct=None, x=None):
        self.T, self.H, self.F, self.E, self.k, self.n_shared, self.r = T, H, F, E, k, n_shared, r
        nd = E if n_distinct is None else n_distinct
        self.distinct = [synth.expert_mxfp4(seed, e, H, F) for e in range(nd)]
        self.emap = expert_map(seed, E, nd)
        self.shared = synth.expert_mxfp4(seed, -1, H, F) if n_shared else None
        self.Wr, _ = synth.router_weights(seed, E, H)
        self.b = synth.uniform_bias(seed, E)
        self.x = synth.activations(seed, T, H) if x is None else x

    def layer(self, max_tokens=None, out_dtype=abi.DT_F32, path=abi.PATH_AUTO):
        desc = make_desc(self.H, self.F, self.E, self.k, self.n_shared, 32, self.r,
                         abi.WFMT_MXFP4, out_dtype)
        return Layer(desc, self.Wr, self.b, self.distinct, self.shared, self.emap,
                     max_tokens=max_tokens or self.T, path=path)

    def oracle_layer(self, out_rows=None):
        return oracle.mx_layer(self.x, self.Wr, self.b, self.distinct, self.shared, self.k,
                               self.r, out_rows=out_rows, expert_map=self.emap)


def _check_mx_out(got, want):
    # fp32 MFMA accumulation against the oracle's fp64 sums: within the
    # spec bar, not bit-exact
    e = rel_err(got, want)
    assert e <= MAX_REL_ERR, "max relative error %.3g" % e
    return e


PATHS = [pytest.param(abi.PATH_AUTO, id="mxmfma"), pytest.param(abi.PATH_MX_BF16, id="bf16mfma")]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T,shared", [(1, 1), (5, 0), (23, 1)])
def test_mx_layer_matches_oracle(T, shared, path):
    c = MxCase(31, T, 512, 256, 16, 4, shared, r=1.5)
    lay = c.layer(path=path)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch = oracle.router(c.x, c.Wr, c.b, c.k, c.r, want=True)
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch)
    e = _check_mx_out(out.cpu().numpy(), out_o)
    print("mx layer T=%d path %d: max rel err %.3g" % (T, path, e))
    lay.close()


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 2, 4])
def test_mx_decode_rows_take_the_few_row_kernels(T, path):
    # hidden a multiple of 512, top-8 + shared: one token (10 row tiles) runs
    # gate/up with 4 weight tiles per wave and two tokens (19) with 2, four
    # steps of loads ahead; four tokens (28) the many-row kernel; against the
    # oracle at the same bar
    c = MxCase(35, T, 2048, 1024, 24, 8, 1, r=1.0, n_distinct=4)
    lay = c.layer(path=path)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch = oracle.router(c.x, c.Wr, c.b, c.k, c.r, want=True)
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch)
    e = _check_mx_out(out.cpu().numpy(), out_o)
    print("mx decode T=%d path %d: max rel err %.3g" % (T, path, e))
    lay.close()


@pytest.mark.parametrize("path", PATHS)
def test_mx_few_row_kernels_equal_many_row_kernels(path):
    # the expert FFN of one token alone and of two tokens (few-row gate/up
    # kernels) and of the same tokens among 70 (many-row kernel), with the
    # routing given: the same bits, since each output's MFMA sums run over the
    # same steps in the same order
    T, H = 70, 2048
    c = MxCase(36, T, H, 1024, 24, 8, 1, r=1.0, n_distinct=4)
    lay = c.layer(path=path)
    x = lay.x_tensor(c.x)
    idx, w, _ = lay.forward(x)
    torch.cuda.synchronize()
    out_all = torch.empty((T, H), dtype=torch.float32, device="cuda")
    abi.moe_expert_ffn(lay.ctx, x, T, lay.weights, idx, w, out_all)
    for rows in ([0], [37], [5, 61]):
        sel = torch.tensor(rows, device="cuda")
        xs, ids, ws = (v.index_select(0, sel).contiguous() for v in (x, idx, w))
        out_few = torch.empty((len(rows), H), dtype=torch.float32, device="cuda")
        abi.moe_expert_ffn(lay.ctx, xs, len(rows), lay.weights, ids, ws, out_few)
        torch.cuda.synchronize()
        for j, t in enumerate(rows):
            assert torch.equal(out_few[j].view(torch.int32), out_all[t].view(torch.int32)), (rows, t)
    lay.close()


def test_mx_swiglu_rows_match_oracle_bf16_path():
    # exact bf16 products, fp32 sums: the bf16 h rows equal the oracle's except
    # where the fp32 projection sits at a bf16 rounding boundary (then one bf16
    # ulp apart)
    c = MxCase(32, 6, 1024, 512, 8, 2, 1)
    lay = c.layer(path=abi.PATH_MX_BF16)
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


def test_mx_swiglu_rows_mx_mfma():
    # MX MFMA: each h row within the output bar of the oracle's row (distance
    # to the row's largest |h|), the bf16 rounding of both sides included
    c = MxCase(32, 6, 1024, 512, 8, 2, 1)
    lay = c.layer()
    idx, _, _ = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    S = c.k + 1
    hb = lay.debug_read(7, (c.T, S, c.F), torch.int16).cpu().numpy().view(np.uint16)
    ig = idx.cpu().numpy()
    xf = synth.bf16_bits_to_f32(c.x)
    worst = 0.0
    for t in range(c.T):
        for i in range(S):
            ex = c.shared if i == c.k else c.distinct[c.emap[ig[t, i]]]
            want = synth.bf16_bits_to_f32(oracle.mx_expert(xf[t], ex)["h_bf16"]).astype(np.float64)
            got = synth.bf16_bits_to_f32(hb[t, i]).astype(np.float64)
            worst = max(worst, float(np.abs(got - want).max() / np.abs(want).max()))
    assert worst <= MAX_REL_ERR, worst
    print("mx-mfma SwiGLU rows: max distance / row max %.3g" % worst)
    lay.close()


@pytest.mark.parametrize("path", PATHS)
def test_mx_expert_ffn_given_routing_and_determinism(path):
    c = MxCase(33, 4, 512, 256, 12, 3, 1, r=2.0)
    lay = c.layer(path=path)
    xd = lay.x_tensor(c.x)
    idx, w, out1 = lay.forward(xd)
    out2 = lay.ffn(xd, idx, w)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32))
    lay.close()


@pytest.mark.parametrize("path", PATHS)
def test_mx_bf16_output(path):
    c = MxCase(34, 3, 512, 256, 8, 2, 1)
    lay = c.layer(out_dtype=abi.DT_BF16, path=path)
    _, _, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    _, _, out_o = c.oracle_layer()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    # the MX MFMA's sums differ from fp32 ones by more than a few fp32 ulps,
    # so only the 2e-3 bar beyond the bf16 rounding applies there
    e, same = check_bf16_out(got, out_o, same_rounding=(path == abi.PATH_MX_BF16))
    print("mx bf16 output: max rel err %.3g, equal to the oracle's rounding %.5f" % (e, same))
    lay.close()


def test_mx_wide_layer_full_size():
    # MXFP4 wide layer: hidden 7168, 384 routed + 1 shared, F 2048, top-8, 64
    # tokens, uniform routing bias.  Routing checked for every token; the
    # outputs of all 64 tokens on 256 sampled columns against the fp64 oracle
    # (11 distinct weight sets behind a seeded random map of the 384 experts).
    # Both kernels run on the same layer.
    H, F, E, k, T = 7168, 2048, 384, 8, 64
    c = MxCase(0, T, H, F, E, k, 1, r=1.0, n_distinct=11)
    lay = c.layer()
    xd = lay.x_tensor(c.x)
    outs = {}
    for path in (abi.PATH_AUTO, abi.PATH_MX_BF16):
        lay.set_path(path)
        idx, w, out = lay.forward(xd)
        torch.cuda.synchronize()
        outs[path] = (idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy())
    lay.close()
    idx_o, w_o, lg, sc, ch = oracle.router(c.x, c.Wr, c.b, k, c.r, want=True)
    rng = np.random.default_rng(2)
    cols = np.sort(rng.choice(H, 256, replace=False)).astype(np.int32)
    _, _, out_o = oracle_rows_parallel(
        lambda xs: oracle.mx_layer(xs, c.Wr, c.b, c.distinct, c.shared, k, c.r, out_rows=cols,
                                   expert_map=c.emap), c.x, np.arange(T))
    for path, (idx, w, out) in outs.items():
        check_routing(idx, w, idx_o, w_o, ch)
        e = _check_mx_out(out[:, cols], out_o)
        print("mx wide layer path %d: max rel err %.3g over 64 tokens x 256 columns" % (path, e))
