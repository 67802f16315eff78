"""GPU parity of the one-token path (the fused few-token router, the one-token
gate/up and down kernels) through the C ABI against the oracle: routing,
outputs, every intermediate, the combine with out-of-range expert ids, and the
shape corners of the kernels (batch sizes, 16 slots, E above 256, k = 1)."""
import numpy as np
import pytest

import oracle
from quantized_expert_ffn_topk_amd import abi, synth
from tests.gpu_common import Case, check_out, check_routing

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# H, F, E, k, n_shared, group
CASES = [
    (512, 256, 16, 4, 1, 32),
    (768, 512, 64, 8, 0, 64),      # H/128 = 6: batches of 2 loads per lane
    (1024, 2048, 256, 8, 1, 32),   # E = 256 (full wave sort), F at the one-token limit
    (512, 256, 300, 6, 1, 32),     # E > 256: rank-counting top-k
    (256, 256, 40, 15, 1, 64),     # 16 slots: 1024-thread down blocks
    (2048, 1024, 8, 1, 0, 32),     # k = 1
    (4096, 2048, 64, 8, 1, 64),    # two half tiles per down block, shared expert on quarter waves
    (8192, 2048, 32, 6, 0, 32),    # hidden at the one-token limit: 16-load gate/up batches, two half tiles
]


def _intermediates_match(lay, c, idx_g):
    """Token codes, SwiGLU rows, their codes and scales and the per-slot
    projections equal the oracle's bit for bit."""
    H, F, k = c.H, c.F, c.k
    S = k + c.n_shared
    xf = synth.bf16_bits_to_f32(c.x)
    q_o, s_o = oracle.quant_rows(xf)
    assert np.array_equal(lay.debug_read(0, (1, H), torch.int8).cpu().numpy(), q_o)
    assert lay.debug_read(1, (1,), torch.float32).cpu().numpy()[0] == np.float32(s_o[0])
    h = lay.debug_read(3, (S, F), torch.float32).cpu().numpy()
    qh = lay.debug_read(4, (S, F), torch.int8).cpu().numpy()
    sh = lay.debug_read(5, (S,), torch.float32).cpu().numpy()
    Y = lay.debug_read(6, (S, H), torch.float32).cpu().numpy()
    for i in range(S):
        ex = c.shared if i == k else c.distinct[c.emap[idx_g[0, i]]]
        ro = oracle.expert(q_o[0], s_o[0], ex, c.g)
        assert np.array_equal(h[i].view(np.uint32), ro["h"].view(np.uint32)), i
        assert np.array_equal(qh[i], ro["qh"]), i
        assert sh[i] == np.float32(ro["sh"]), i
        assert np.array_equal(Y[i].view(np.uint32), ro["y"].view(np.uint32)), i


@pytest.mark.parametrize("case", CASES, ids=lambda c: "H%d-F%d-E%d-k%d-s%d-g%d" % c)
def test_one_token_layer_matches_oracle(case):
    H, F, E, k, ns, g = case
    c = Case(21, 1, H, F, E, k, ns, g=g, r=2.5, n_distinct=min(E, 5))
    lay = c.layer(max_tokens=1)
    for step in range(3):
        c.x = synth.activations(300 + step, 1, H)
        idx, w, out = lay.forward(lay.x_tensor(c.x))
        torch.cuda.synchronize()
        idx_o, w_o, out_o = c.oracle_layer()
        _, _, _, _, ch_o = c.oracle_router()
        ig = idx.cpu().numpy()
        check_routing(ig, w.cpu().numpy(), idx_o, w_o, ch_o)
        check_out(out.cpu().numpy(), out_o)
        _intermediates_match(lay, c, ig)
    lay.close()


def test_one_token_router_only_matches_oracle():
    H, E, k = 1024, 256, 8
    c = Case(22, 1, H, 256, E, k, 1, r=2.5, n_distinct=2)
    lay = c.layer(max_tokens=1)
    for step in range(4):
        c.x = synth.activations(400 + step, 1, H)
        idx, w = lay.router(lay.x_tensor(c.x))
        torch.cuda.synchronize()
        idx_o, w_o, lg, sc, ch = c.oracle_router()
        check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch)
        # fp64 logits: the sum order differs from the oracle's, the choice does not
        np.testing.assert_allclose(lay.debug_read(2, (1, E), torch.float64).cpu().numpy(), lg,
                                   rtol=1e-12, atol=1e-13)
    lay.close()


def test_one_token_ties_take_the_lower_index():
    # experts 3, 17 and 40 share router row and bias: they tie on the biased
    # score and must rank 3, 17, 40; one more expert with a larger bias leads
    H, E, k = 512, 64, 4
    c = Case(23, 1, H, 256, E, k, 1, r=1.0, n_distinct=3)
    c.Wr[17] = c.Wr[3]
    c.Wr[40] = c.Wr[3]
    c.b[:] = -2.0
    c.b[3] = c.b[17] = c.b[40] = 1.0
    c.b[9] = 1.5
    lay = c.layer(max_tokens=1)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, out_o = c.oracle_layer()
    ig = idx.cpu().numpy()
    assert np.array_equal(ig, idx_o)
    assert ig[0].tolist()[1:] == [3, 17, 40] or ig[0].tolist()[:3] == [3, 17, 40]
    check_out(out.cpu().numpy(), out_o)
    lay.close()


def test_one_token_expert_ffn_skips_out_of_range_ids():
    # given routing with an id below 0, one at E and a duplicate: the bad ranks
    # add nothing, the duplicate counts twice; combine order is shared expert
    # first, then rank order, in fp64, rounded once
    H, F, E, k, g = 512, 256, 16, 5, 32
    c = Case(24, 1, H, F, E, k, 1, g=g, r=1.0, n_distinct=4)
    lay = c.layer(max_tokens=1)
    ids = np.array([[7, -1, E, 2, 7]], np.int32)
    gw = np.array([[0.5, 9.0, 9.0, -0.25, 0.125]], np.float32)
    xd = lay.x_tensor(c.x)
    out = lay.ffn(xd, torch.from_numpy(ids).cuda(), torch.from_numpy(gw).cuda())
    torch.cuda.synchronize()
    q_o, s_o = oracle.quant_rows(synth.bf16_bits_to_f32(c.x))
    ys = oracle.expert(q_o[0], s_o[0], c.shared, g)["y"].astype(np.float64)
    o = ys.copy()
    for i in range(k):
        e = ids[0, i]
        if 0 <= e < E:
            y = oracle.expert(q_o[0], s_o[0], c.distinct[c.emap[e]], g)["y"].astype(np.float64)
            o = o + np.float64(gw[0, i]) * y
    want = o.astype(np.float32)
    got = out.cpu().numpy()[0]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    lay.close()


def test_one_token_bf16_output():
    c = Case(25, 1, 512, 256, 16, 4, 1, r=2.5, n_distinct=4)
    lay = c.layer(max_tokens=1, out_dtype=abi.DT_BF16)
    _, _, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    _, _, out_o = c.oracle_layer()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, synth.f32_to_bf16_bits(out_o))
    lay.close()
