"""GPU parity of the router, the int4 x int8 projections and the whole layer
(GEMV kernels), through the C ABI, against the oracle."""
import numpy as np
import pytest

import oracle
from quantized_expert_ffn_topk_amd import abi, synth
from tests.gpu_common import (Case, check_bf16_out, check_out, check_routing,
                               oracle_rows_parallel, rel_err)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _sync():
    torch.cuda.synchronize()


def _proj_case(seed, H, F, g, unit):
    ex = synth.expert_int4(seed, 0, H, F, g)
    if unit:
        for k in ("s_gate", "s_up", "s_down"):
            ex[k] = np.full_like(ex[k], 0x3C00)          # fp16 1.0
    c = Case(seed, 1, H, F, 4, 2, 0, g)
    c.distinct = [ex]
    c.emap = [0] * 4
    return c, ex


@pytest.mark.parametrize("T", [1, 3, 8, 11])
@pytest.mark.parametrize("part", [0, 1, 2])
def test_project_unit_scales_equal_integer_dots(T, part):
    # Unit scales and s_in = 1 expose the int32 accumulators: exact integers.
    H, F, g = 512, 256, 32
    c, ex = _proj_case(1, H, F, g, unit=True)
    lay = c.layer(max_tokens=16, path=abi.PATH_GEMV)
    K = F if part == 2 else H
    N = H if part == 2 else F
    r = np.random.default_rng(T * 10 + part)
    q = r.integers(-127, 128, size=(T, K)).astype(np.int8)
    qd = torch.from_numpy(q).cuda()
    sd = torch.ones(T, dtype=torch.float32, device="cuda")
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    abi.moe_debug_project(lay.ctx, lay.blobs[0], part, qd, sd, T, y)
    _sync()
    W = ex[("q_gate", "q_up", "q_down")[part]].astype(np.int64)
    ref = q.astype(np.int64) @ W.T
    assert np.array_equal(y.cpu().numpy().astype(np.int64), ref)
    lay.close()


@pytest.mark.parametrize("g", [32, 64])
def test_project_real_scales_bit_exact(g):
    H, F = 768, 512
    c, ex = _proj_case(2, H, F, g, unit=False)
    lay = c.layer(max_tokens=8, path=abi.PATH_GEMV)
    r = np.random.default_rng(g)
    T = 5
    for part in range(3):
        K = F if part == 2 else H
        q = r.integers(-127, 128, size=(T, K)).astype(np.int8)
        s = r.uniform(1e-3, 1e-1, size=T).astype(np.float32)
        N = H if part == 2 else F
        y = torch.empty((T, N), dtype=torch.float32, device="cuda")
        abi.moe_debug_project(lay.ctx, lay.blobs[0], part, torch.from_numpy(q).cuda(),
                              torch.from_numpy(s).cuda(), T, y)
        _sync()
        yg = y.cpu().numpy()
        W = ex[("q_gate", "q_up", "q_down")[part]]
        S = ex[("s_gate", "s_up", "s_down")[part]]
        for t in range(T):
            ref = oracle.proj_i4i8(q[t], s[t], W, S, g)
            assert np.array_equal(yg[t].view(np.uint32), ref.view(np.uint32)), (part, t)
    lay.close()


def test_router_tiny_layer():
    # 16 tokens, hidden 2048, 64 experts, top-8, bias N(0, 0.01)
    c = Case(0, 16, 2048, 1024, 64, 8, 0, n_distinct=1)
    lay = c.layer()
    xd = lay.x_tensor(c.x)
    idx, w = lay.router(xd)
    _sync()
    idx_o, w_o, lg_o, sc_o, ch_o = c.oracle_router()
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
    lg = lay.debug_read(2, (16, 64), torch.float64).cpu().numpy()
    np.testing.assert_allclose(lg, lg_o, rtol=1e-12, atol=1e-13)
    lay.close()


def test_layer_tiny_full_parity():
    # OLMoE-like tiny layer: H 2048, 64 experts, F 1024, top-8, no shared, 16 tokens
    c = Case(0, 16, 2048, 1024, 64, 8, 0)
    lay = c.layer()
    xd = lay.x_tensor(c.x)
    idx, w, out = lay.forward(xd)
    _sync()
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch_o = c.oracle_router()
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
    e, exact = check_out(out.cpu().numpy(), out_o)
    print("tiny layer: max rel err %.3g, bit-exact fraction %.6f" % (e, exact))
    # intermediates: token codes exact; h and its codes per (token, rank)
    qa = lay.debug_read(0, (16, 2048), torch.int8).cpu().numpy()
    xf = synth.bf16_bits_to_f32(c.x)
    q_o, s_o = oracle.quant_rows(xf)
    assert np.array_equal(qa, q_o)
    S = c.k
    h = lay.debug_read(3, (16, S, 1024), torch.float32).cpu().numpy()
    qh = lay.debug_read(4, (16, S, 1024), torch.int8).cpu().numpy()
    idx_g = idx.cpu().numpy()
    for t in (0, 7, 15):
        for i in range(c.k):
            ex = c.distinct[c.emap[idx_g[t, i]]]
            ro = oracle.expert(q_o[t], s_o[t], ex, c.g)
            assert np.array_equal(h[t, i].view(np.uint32), ro["h"].view(np.uint32))
            assert np.array_equal(qh[t, i], ro["qh"])
    lay.close()


@pytest.mark.parametrize("T", [1, 5, 17])
@pytest.mark.parametrize("g", [32, 64])
def test_layer_shared_expert(T, g):
    c = Case(3, T, 512, 256, 16, 4, 1, g=g, r=2.5)
    lay = c.layer(max_tokens=32)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    _sync()
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch_o = c.oracle_router()
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
    check_out(out.cpu().numpy(), out_o)
    lay.close()


@pytest.mark.parametrize("T,H,E", [(9, 2048, 300), (3, 8192, 40), (20, 1024, 600)])
def test_layer_token_codes_from_topk_launch(T, H, E):
    # Two tokens and more: the top-k launch (4, 8 or 16 waves for up to 256,
    # 512 or 1024 experts) also quantises the tokens.  Its codes and scales
    # equal the oracle's bit for bit, and the layer output matches.
    c = Case(60 + T, T, H, 256, E, 4, 1, r=2.5, n_distinct=4)
    lay = c.layer(max_tokens=32)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    _sync()
    q_o, s_o = oracle.quant_rows(synth.bf16_bits_to_f32(c.x))
    q = lay.debug_read(0, (T, H), torch.int8).cpu().numpy()
    s = lay.debug_read(1, (T,), torch.float32).cpu().numpy()
    assert np.array_equal(q, np.asarray(q_o, np.int8))
    assert np.array_equal(s.view(np.uint32), np.asarray(s_o, np.float32).view(np.uint32))
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch_o = c.oracle_router()
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
    check_out(out.cpu().numpy(), out_o)
    lay.close()


def test_layer_bf16_output():
    c = Case(4, 6, 512, 256, 8, 2, 1, r=1.0)
    lay = c.layer(out_dtype=abi.DT_BF16)
    _, _, out = lay.forward(lay.x_tensor(c.x))
    _sync()
    _, _, out_o = c.oracle_layer()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    # bf16 output is the fp32 result rounded to nearest even: equal to the
    # oracle rounded the same way except next to a midpoint, max rel <= 2e-3
    e, same = check_bf16_out(got, out_o)
    assert same >= 0.999
    lay.close()


def test_layer_deterministic_and_expert_ffn_with_given_routing():
    c = Case(5, 9, 512, 256, 16, 4, 1, r=2.5)
    lay = c.layer()
    xd = lay.x_tensor(c.x)
    idx, w, out1 = lay.forward(xd)
    _, _, out2 = lay.forward(xd)
    out3 = lay.ffn(xd, idx, w)
    _sync()
    assert torch.equal(out1.view(torch.int32), out2.view(torch.int32))
    assert torch.equal(out1.view(torch.int32), out3.view(torch.int32))
    lay.close()


def test_edge_cases_zero_token_ties_and_empty_call():
    H, F, E, k = 512, 256, 12, 3
    x = synth.activations(6, 4, H)
    x[2] = 0                                       # zero token: output exactly 0
    c = Case(6, 4, H, F, E, k, 1, x=x)
    c.Wr[9] = c.Wr[4]                              # duplicated router rows ...
    c.b[:] = -1.0
    c.b[4] = c.b[9] = 0.5                          # ... with tied bias: 4 ranks before 9
    lay = c.layer()
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    _sync()
    idx_o, w_o, out_o = c.oracle_layer()
    ig = idx.cpu().numpy()
    assert np.array_equal(ig, idx_o)
    assert np.all(ig[:, 0] == 4) and np.all(ig[:, 1] == 9)
    og = out.cpu().numpy()
    check_out(og, out_o)
    assert not og[2].any() or np.array_equal(og[2], out_o[2])
    # T == 0 enqueues nothing and succeeds
    abi.moe_layer_forward(lay.ctx, None, 0, lay.weights, None, 0, None, None, None)
    with pytest.raises(abi.MoEError):
        abi.moe_layer_forward(lay.ctx, lay.x_tensor(c.x), 5, lay.weights, None, 0, None, None, out)
    lay.close()


def test_all_experts_selected():
    # k == E: every expert runs for every token
    c = Case(7, 3, 256, 256, 4, 4, 0, r=1.0)
    lay = c.layer()
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    _sync()
    idx_o, w_o, out_o = c.oracle_layer()
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    check_out(out.cpu().numpy(), out_o)
    lay.close()


def test_glm_decode_full_size():
    # GLM-shaped decode layer: hidden 6144, 256 routed + 1 shared, F 2048,
    # group 32, top-8, routed scale 2.5, one token per step.  Routing is
    # checked in full every step; the first step's output on all 6144 columns,
    # the next two on 96 sampled columns (7 distinct weight sets behind a
    # seeded random map of the 256 experts).
    H, F, E, k = 6144, 2048, 256, 8
    c = Case(0, 1, H, F, E, k, 1, r=2.5, n_distinct=7)
    lay = c.layer(max_tokens=1)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(H, 96, replace=False)).astype(np.int32)
    for step in range(3):
        c.x = synth.activations(100 + step, 1, H)
        idx, w, out = lay.forward(lay.x_tensor(c.x))
        _sync()
        idx_o, w_o, out_o = c.oracle_layer(out_rows=None if step == 0 else rows)
        _, _, _, _, ch_o = c.oracle_router()
        check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
        og = out.cpu().numpy()
        e, exact = check_out(og if step == 0 else og[:, rows], out_o)
        if step == 0:
            print("GLM decode, all 6144 outputs: max rel err %.3g, bit-exact %.5f" % (e, exact))
    lay.close()



@pytest.mark.parametrize("H,g", [(1536, 32), (2048, 64), (4096, 32), (6144, 64), (8192, 32)])
def test_one_token_half_tile_kernels(H, g):
    # One token, F 2048, 8 routed + 1 shared expert: the down projection runs
    # over half tiles (H/2048 of them per block up to 3, two for H = 8192, one
    # when H is not a multiple of 2048) and, for H a multiple of 1024, the
    # shared expert's gate/up over
    # half tile pairs inside the top-k launch.  Full outputs, the SwiGLU rows
    # and their codes of every slot are compared with the oracle.
    F, E, k = 2048, 16, 8
    c = Case(40 + H // 512, 1, H, F, E, k, 1, g=g, r=2.5, n_distinct=4)
    lay = c.layer(max_tokens=1)
    for step in range(2):
        c.x = synth.activations(200 + step, 1, H)
        idx, w, out = lay.forward(lay.x_tensor(c.x))
        _sync()
        idx_o, w_o, out_o = c.oracle_layer()
        _, _, _, _, ch_o = c.oracle_router()
        check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
        check_out(out.cpu().numpy(), out_o)
        xf = synth.bf16_bits_to_f32(c.x)
        q_o, s_o = oracle.quant_rows(xf)
        h = lay.debug_read(3, (1, k + 1, F), torch.float32).cpu().numpy()
        qh = lay.debug_read(4, (1, k + 1, F), torch.int8).cpu().numpy()
        idx_g = idx.cpu().numpy()
        for i in range(k + 1):
            ex = c.shared if i == k else c.distinct[c.emap[idx_g[0, i]]]
            ro = oracle.expert(q_o[0], s_o[0], ex, g)
            assert np.array_equal(h[0, i].view(np.uint32), ro["h"].view(np.uint32)), (step, i)
            assert np.array_equal(qh[0, i], ro["qh"]), (step, i)
    lay.close()


def test_kernel_timing_ring_counts_every_launch():
    # Profiling on: 300 one-token steps back to back (more than the 256 event
    # pairs per kind, so the ring drains while the steps run); every launch is
    # counted once with a positive duration, and the outputs equal those of
    # the same steps without profiling.
    c = Case(12, 1, 512, 256, 16, 4, 1, r=2.5)
    lay = c.layer(max_tokens=1)
    n = 300
    xs = lay.x_tensor(synth.activations(13, n, 512))
    outs = [lay._outs(1) for _ in range(2)]
    ref = []
    for i in range(n):
        lay.forward(xs[i:i + 1], outs=outs[0])
        ref.append(outs[0][2].clone())
    _sync()
    abi.moe_ctx_profile(lay.ctx, True)
    abi.moe_ctx_profile_read(lay.ctx)
    got = []
    for i in range(n):
        lay.forward(xs[i:i + 1], outs=outs[1])
        got.append(outs[1][2].clone())
    prof = abi.moe_ctx_profile_read(lay.ctx)
    abi.moe_ctx_profile(lay.ctx, False)
    _sync()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    used = {k: v for k, v in prof.items() if v[1]}
    assert used, prof
    for k, (ms, cnt) in used.items():
        assert cnt == n, (k, cnt)
        assert ms > 0.0, k
    # nothing left over for the next read
    again = abi.moe_ctx_profile_read(lay.ctx)
    assert all(v[1] == 0 for v in again.values())
    lay.close()


@pytest.mark.parametrize("F,E,k", [(4096, 16, 4), (512, 32, 16)])
def test_one_token_gemv_fallback(F, E, k):
    # One token where the one-token kernels do not apply (F above 2048, or
    # k + shared above 16 slots): routing, quantisation and lists in one
    # launch and the GEMV projections with requant and combine fused into
    # their tails.  Two steps, full outputs and routing against the oracle.
    c = Case(70 + k, 1, 512, F, E, k, 1, r=2.5, n_distinct=5)
    lay = c.layer(max_tokens=1)
    for step in range(2):
        c.x = synth.activations(300 + step, 1, 512)
        idx, w, out = lay.forward(lay.x_tensor(c.x))
        _sync()
        idx_o, w_o, out_o = c.oracle_layer()
        _, _, _, _, ch_o = c.oracle_router()
        check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
        check_out(out.cpu().numpy(), out_o)
    lay.close()

def test_graph_replay_matches_eager():
    # Three layer steps captured as one HIP graph, replayed three times with
    # eager work and synchronisations in between; every replay must equal the
    # eager results bit for bit.
    c = Case(8, 1, 512, 256, 16, 4, 1, r=2.5)
    lay = c.layer(max_tokens=1)
    xs = lay.x_tensor(synth.activations(9, 3, 512))
    s = torch.cuda.Stream()
    outs = [lay._outs(1) for _ in range(3)]
    with torch.cuda.stream(s):
        for i in range(3):
            lay.forward(xs[i:i + 1], stream=s, outs=outs[i])
    s.synchronize()
    eager = [o[2].clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(3):
            lay.forward(xs[i:i + 1], stream=s, outs=outs[i])
    for rep in range(3):
        for o in outs:
            o[2].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(outs[i][2].view(torch.int32), eager[i].view(torch.int32)), (rep, i)
        # eager work in between replays
        lay.forward(xs[rep:rep + 1])
        torch.cuda.synchronize()
    del g
    lay.close()


@pytest.mark.parametrize("T,E", [(17, 40), (100, 64), (300, 256), (1100, 48), (5, 300), (40, 513),
                                 (20, 1024), (2, 1024), (16, 7)])
def test_router_logits_many_tokens(T, E):
    # the router GEMV (up to 16 tokens) and the fp64 MFMA router (more), E not
    # a multiple of 16 included, and the block top-k with 4, 8 and 16 waves
    # (E up to 256, 512 and 1024)
    c = Case(30 + T, T, 1024, 256, E, 6, 0, n_distinct=1)
    lay = c.layer()
    idx, w = lay.router(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, lg_o, sc_o, ch_o = c.oracle_router()
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
    lg = lay.debug_read(2, (T, E), torch.float64).cpu().numpy()
    np.testing.assert_allclose(lg, lg_o, rtol=1e-12, atol=1e-13)
    lay.close()


@pytest.mark.parametrize("T", [1, 5, 40])
def test_router_nan_bias_ranks_last(T):
    # NaN biased scores rank as -inf on every router path (one token, the
    # few-token GEMV router and the MFMA router), as the oracle ranks them
    c = Case(12, T, 512, 256, 24, 6, 1, n_distinct=2)
    c.b = c.b.copy()
    c.b[[1, 9, 17]] = np.nan
    c.b[4] = 3.0
    c.b[5] = np.nan
    lay = c.layer(max_tokens=T)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    _sync()
    idx_o, w_o, _, _, ch_o = c.oracle_router()
    ig = idx.cpu().numpy()
    assert not np.isin(ig, [1, 5, 9, 17]).any()
    check_routing(ig, w.cpu().numpy(), idx_o, w_o, ch_o)
    lay.close()
