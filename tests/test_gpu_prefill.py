"""GPU parity of the grouped int4 x int8 GEMM on the int8 MFMA (prefill path)
through the C ABI: exact integer accumulators, bit-equality with the oracle
and with the GEMV path, and a skewed-routing prefill layer at full width."""
import numpy as np
import pytest

import oracle
from quantized_expert_ffn_topk_amd import abi, synth
from tests.gpu_common import Case, check_bf16_out, check_out, check_routing, oracle_rows_parallel

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _sync():
    torch.cuda.synchronize()


def _unit_case(seed, H, F, g):
    ex = synth.expert_int4(seed, 0, H, F, g)
    for k in ("s_gate", "s_up", "s_down"):
        ex[k] = np.full_like(ex[k], 0x3C00)
    c = Case(seed, 1, H, F, 4, 2, 0, g)
    c.distinct = [ex]
    c.emap = [0] * 4
    return c, ex


@pytest.mark.parametrize("T", [1, 37, 64, 130])
@pytest.mark.parametrize("part", [0, 1, 2])
def test_mfma_project_unit_scales_equal_integer_dots(T, part):
    H, F, g = 512, 256, 32
    c, ex = _unit_case(11, H, F, g)
    lay = c.layer(max_tokens=256, path=abi.PATH_MFMA)
    K = F if part == 2 else H
    N = H if part == 2 else F
    r = np.random.default_rng(T + 100 * part)
    q = r.integers(-127, 128, size=(T, K)).astype(np.int8)
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    abi.moe_debug_project(lay.ctx, lay.blobs[0], part, torch.from_numpy(q).cuda(),
                          torch.ones(T, dtype=torch.float32, device="cuda"), T, y)
    _sync()
    W = ex[("q_gate", "q_up", "q_down")[part]].astype(np.int64)
    assert np.array_equal(y.cpu().numpy().astype(np.int64), q.astype(np.int64) @ W.T)
    lay.close()


@pytest.mark.parametrize("g", [32, 64])
def test_mfma_project_bit_exact_vs_oracle_and_gemv(g):
    H, F, T = 768, 512, 70
    c = Case(12, 1, H, F, 4, 2, 0, g)
    ex = c.distinct[0]
    lay = c.layer(max_tokens=128)
    r = np.random.default_rng(g)
    for part in range(3):
        K = F if part == 2 else H
        N = H if part == 2 else F
        q = r.integers(-127, 128, size=(T, K)).astype(np.int8)
        s = r.uniform(1e-3, 1e-1, size=T).astype(np.float32)
        qd, sd = torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda()
        outs = []
        for path in (abi.PATH_MFMA, abi.PATH_GEMV):
            lay.set_path(path)
            y = torch.empty((T, N), dtype=torch.float32, device="cuda")
            abi.moe_debug_project(lay.ctx, lay.blobs[0], part, qd, sd, T, y)
            _sync()
            outs.append(y.cpu().numpy())
        assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), part
        W = ex[("q_gate", "q_up", "q_down")[part]]
        S = ex[("s_gate", "s_up", "s_down")[part]]
        for t in (0, 33, T - 1):
            ref = oracle.proj_i4i8(q[t], s[t], W, S, g)
            assert np.array_equal(outs[0][t].view(np.uint32), ref.view(np.uint32)), (part, t)
    lay.close()


@pytest.mark.parametrize("top_field", [21, 22])
def test_mfma_project_wide_scale_spread_bit_exact(top_field):
    # One row per part has a scale with exponent field top_field next to the
    # smallest subnormal (exponent counted as 1): a spread of 20 binades keeps
    # the kernel's 64-bit integer epilogue at its largest shift, 21 sends the
    # block to the fp64 epilogue.  Both must equal the oracle bit for bit.
    H, F, T, g = 512, 256, 70, 32
    c = Case(14, 1, H, F, 4, 2, 0, g)
    ex = c.distinct[0]
    for key, row in (("s_gate", 5), ("s_up", 40), ("s_down", 9)):
        ex[key] = ex[key].copy()
        ex[key][row, 0] = top_field << 10
        ex[key][row, 1] = 0x0001
        ex[key][row, 2] = 0x8000 | (top_field - 3) << 10      # negative scale
    lay = c.layer(max_tokens=128, path=abi.PATH_MFMA)
    r = np.random.default_rng(top_field)
    for part in range(3):
        K = F if part == 2 else H
        N = H if part == 2 else F
        q = r.integers(-127, 128, size=(T, K)).astype(np.int8)
        s = r.uniform(1e-3, 1e-1, size=T).astype(np.float32)
        y = torch.empty((T, N), dtype=torch.float32, device="cuda")
        abi.moe_debug_project(lay.ctx, lay.blobs[0], part, torch.from_numpy(q).cuda(),
                              torch.from_numpy(s).cuda(), T, y)
        _sync()
        got = y.cpu().numpy()
        W = ex[("q_gate", "q_up", "q_down")[part]]
        S = ex[("s_gate", "s_up", "s_down")[part]]
        for t in range(T):
            ref = oracle.proj_i4i8(q[t], s[t], W, S, g)
            assert np.array_equal(got[t].view(np.uint32), ref.view(np.uint32)), (part, t)
    lay.close()


@pytest.mark.parametrize("T,g", [(100, 32), (257, 64)])
def test_mfma_layer_equals_gemv_layer_and_oracle(T, g):
    c = Case(13, T, 512, 256, 16, 4, 1, g=g, r=2.5)
    lay = c.layer(max_tokens=T)
    xd = lay.x_tensor(c.x)
    res = {}
    for path in (abi.PATH_MFMA, abi.PATH_GEMV):
        lay.set_path(path)
        idx, w, out = lay.forward(xd)
        _sync()
        res[path] = (idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy())
    assert np.array_equal(res[abi.PATH_MFMA][2].view(np.uint32), res[abi.PATH_GEMV][2].view(np.uint32))
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch_o = c.oracle_router()
    check_routing(res[abi.PATH_MFMA][0], res[abi.PATH_MFMA][1], idx_o, w_o, ch_o)
    check_out(res[abi.PATH_MFMA][2], out_o)
    lay.close()



@pytest.mark.parametrize("k,n_shared,out_dtype", [(4, 1, "bf16"), (16, 1, "f32"), (8, 0, "f32")])
def test_many_token_combine(k, n_shared, out_dtype):
    # The many-token combine (4 outputs per thread, every slot's load issued
    # first) with k + n_shared from 8 to 17 slots and both output types.
    T, H, F, E = 90, 512, 256, 32
    c = Case(60 + k, T, H, F, E, k, n_shared, r=1.5, n_distinct=6)
    dt = abi.DT_BF16 if out_dtype == "bf16" else abi.DT_F32
    lay = c.layer(max_tokens=T, path=abi.PATH_MFMA, out_dtype=dt)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    _sync()
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch_o = c.oracle_router()
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
    if dt == abi.DT_BF16:
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        _, same = check_bf16_out(got, out_o)
        assert same >= 0.999
    else:
        check_out(out.cpu().numpy(), out_o)
    lay.close()


def test_mfma_layer_many_experts():
    # 600 routed experts + shared on the MFMA path: the tile list and the
    # block top-k with 16 waves; full outputs against the oracle
    T, H, F, E, k = 130, 512, 256, 600, 8
    c = Case(90, T, H, F, E, k, 1, r=2.5, n_distinct=7)
    lay = c.layer(max_tokens=T, path=abi.PATH_MFMA)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    _sync()
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch_o = c.oracle_router()
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
    check_out(out.cpu().numpy(), out_o)
    lay.close()


@pytest.mark.parametrize("T,path", [(100, abi.PATH_MFMA), (5, abi.PATH_AUTO)])
def test_graph_replay_matches_eager_many_tokens(T, path):
    # Two layer calls (MFMA path at 100 tokens; router GEMV, block top-k,
    # one-block permutation and GEMV projections at 5) captured as one HIP
    # graph and replayed three times with eager work and synchronisations in
    # between; every replay equals the eager results bit for bit.
    H, F, E, k = 512, 256, 32, 4
    c = Case(91 + T, T, H, F, E, k, 1, r=2.5, n_distinct=5)
    lay = c.layer(max_tokens=T, path=path)
    xs = [lay.x_tensor(synth.activations(95 + i, T, H)) for i in range(2)]
    s = torch.cuda.Stream()
    outs = [lay._outs(T) for _ in range(2)]
    with torch.cuda.stream(s):
        for i in range(2):
            lay.forward(xs[i], stream=s, outs=outs[i])
    s.synchronize()
    eager = [(o[0].clone(), o[2].clone()) for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(2):
            lay.forward(xs[i], stream=s, outs=outs[i])
    for rep in range(3):
        for o in outs:
            o[2].fill_(float("nan"))
            o[0].fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i][0], eager[i][0]), (rep, i)
            assert torch.equal(outs[i][2].view(torch.int32), eager[i][1].view(torch.int32)), (rep, i)
        lay.forward(xs[rep % 2])
        torch.cuda.synchronize()
    del g
    lay.close()

def test_glm_prefill_zipf_full_size_sampled():
    # GLM-shaped prefill: 4096 tokens, hidden 6144, 256 routed + 1 shared,
    # F 2048, group 32, top-8, routed scale 2.5, Zipf(1.1)-skewed selection
    # bias.  Routing is checked for every token; outputs of 128 sampled tokens
    # on 128 sampled columns against the oracle (7 distinct weight sets behind
    # a seeded random map of the 256 experts).
    H, F, E, k, T = 6144, 2048, 256, 8, 4096
    c = Case(0, T, H, F, E, k, 1, r=2.5, n_distinct=7, bias=synth.zipf_bias(0, E))
    lay = c.layer(max_tokens=T)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    _sync()
    ig, wg, og = idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy()
    idx_o, w_o, lg, sc, ch = oracle.router(c.x, c.Wr, c.b, k, c.r, want=True)
    check_routing(ig, wg, idx_o, w_o, ch)
    loads = np.bincount(ig.ravel(), minlength=E)
    print("expert loads: max %d, empty %d, top-8 share %.3f" % (
        loads.max(), int((loads == 0).sum()), np.sort(loads)[::-1][:8].sum() / loads.sum()))
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(T, 128, replace=False))
    cols = np.sort(rng.choice(H, 128, replace=False)).astype(np.int32)
    _, _, out_o = oracle_rows_parallel(
        lambda xs: oracle.layer(xs, c.Wr, c.b, c.distinct, c.shared, k, c.r, c.g, out_rows=cols,
                                expert_map=c.emap), c.x, toks)
    e, exact = check_out(og[toks][:, cols], out_o)
    print("GLM prefill, 128 tokens x 128 columns: max rel err %.3g, bit-exact %.5f" % (e, exact))
    lay.close()
