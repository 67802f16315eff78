"""GPU parity at more than 16 routed experts per token (top_k up to
min(E, 32)): the block top-k keeping 32 candidates per wave with 4, 8 and 16
waves, the permutation, the GEMV and MFMA projections and the 33-slot combine,
against the oracle."""
import numpy as np
import pytest

from quantized_expert_ffn_topk_amd import abi
from tests.gpu_common import Case, check_out, check_routing

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("T,k,path", [(1, 32, abi.PATH_AUTO), (5, 32, abi.PATH_AUTO),
                                      (70, 32, abi.PATH_AUTO), (9, 17, abi.PATH_GEMV),
                                      (66, 24, abi.PATH_MFMA)])
def test_layer_topk_above_16(T, k, path):
    H, F, E = 512, 256, 64
    c = Case(110 + k + T, T, H, F, E, k, 1, r=2.5, n_distinct=9)
    lay = c.layer(max_tokens=T, path=path)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, out_o = c.oracle_layer()
    _, _, _, _, ch_o = c.oracle_router()
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
    check_out(out.cpu().numpy(), out_o)
    lay.close()


def test_all_32_experts_selected():
    # k == E == 32, no shared expert: every expert runs for every token
    c = Case(120, 4, 256, 256, 32, 32, 0, r=1.0, n_distinct=6)
    lay = c.layer(max_tokens=4)
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, out_o = c.oracle_layer()
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    check_out(out.cpu().numpy(), out_o)
    lay.close()


@pytest.mark.parametrize("T,E,k", [(3, 300, 32), (20, 600, 32), (40, 1024, 25), (2, 200, 31)])
def test_router_topk_above_16_many_experts(T, E, k):
    # 4, 8 and 16 waves with 32 candidates kept per wave: routing and weights
    c = Case(130 + T, T, 1024, 256, E, k, 0, n_distinct=1)
    lay = c.layer(max_tokens=T)
    idx, w = lay.router(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, _, _, ch_o = c.oracle_router()
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch_o)
    lay.close()


def test_mxfp4_topk_above_16():
    from tests.test_gpu_mx import MxCase, _check_mx_out
    c = MxCase(140, 6, 512, 256, 40, 20, 1, r=1.5, n_distinct=7)
    lay = c.layer()
    idx, w, out = lay.forward(lay.x_tensor(c.x))
    torch.cuda.synchronize()
    idx_o, w_o, out_o = c.oracle_layer()
    from oracle import router
    _, _, _, _, ch = router(c.x, c.Wr, c.b, c.k, c.r, want=True)
    check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch)
    _check_mx_out(out.cpu().numpy(), out_o)
    lay.close()
