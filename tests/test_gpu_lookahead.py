"""GPU parity of the router lookahead on a small stack of MoE layers: the
experts predicted for layer l+1 (layer l+1's router on layer l's input, run
through moe_router_topk) equal the oracle's prediction, each layer's routing
and output equal the oracle's, and the residual composition between layers
(bf16(x + gamma*y)) gives the oracle's bits."""
import numpy as np
import pytest

import oracle
from quantized_expert_ffn_topk_amd import abi, synth
from quantized_expert_ffn_topk_amd.layer import Layer, make_desc
from tests.gpu_common import check_out, check_routing

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NL, H, F, E, K = 3, 512, 256, 16, 4


@pytest.mark.parametrize("T,gamma", [(1, 0.25), (6, 0.5)])
def test_lookahead_prediction_matches_oracle(T, gamma):
    experts = [[synth.expert_int4(200 + l, e, H, F, 32) for e in range(E)] for l in range(NL)]
    shared = [synth.expert_int4(200 + l, -1, H, F, 32) for l in range(NL)]
    Wr = [synth.router_weights(200 + l, E, H)[0] for l in range(NL)]
    b = [synth.zipf_bias(300 + l, E) for l in range(NL)]
    desc = make_desc(H, F, E, K, 1, 32, 2.5)
    lays = [Layer(desc, Wr[l], b[l], experts[l], shared[l], max_tokens=T) for l in range(NL)]
    x = synth.activations(77, T, H)
    xd = lays[0].x_tensor(x)
    hits = 0
    try:
        for l in range(NL):
            lay = lays[l]
            if l + 1 < NL:
                pi, _ = lays[l + 1].router(xd)          # next router on this state
            idx, w, out = lay.forward(xd)
            torch.cuda.synchronize()
            xh = xd.cpu().numpy().view(np.uint16)
            idx_o, w_o, out_o = oracle.layer(xh, Wr[l], b[l], experts[l], shared[l], K, 2.5, 32)
            _, _, _, _, ch = oracle.router(xh, Wr[l], b[l], K, 2.5, want=True)
            check_routing(idx.cpu().numpy(), w.cpu().numpy(), idx_o, w_o, ch)
            check_out(out.cpu().numpy(), out_o)
            if l + 1 < NL:
                pred_o = oracle.lookahead(xh, Wr[l + 1], b[l + 1], K)
                _, _, _, _, ch1 = oracle.router(xh, Wr[l + 1], b[l + 1], K, 1.0, want=True)
                wp = np.ones((T, K), np.float32)
                check_routing(pi.cpu().numpy(), wp, pred_o, wp, ch1)
            # the residual composition on the GPU against the oracle's, from
            # the same (GPU) layer output
            xn = (xd.view(torch.bfloat16).float() + out * gamma).to(torch.bfloat16)
            torch.cuda.synchronize()
            want = oracle.residual_bf16(xh, out.cpu().numpy(), gamma)
            assert np.array_equal(xn.view(torch.int16).cpu().numpy().view(np.uint16), want)
            if l > 0:
                hits += sum(len(set(a) & set(p)) for a, p in zip(idx.cpu().numpy().tolist(),
                                                                   prev_pred))
            prev_pred = pi.cpu().numpy().tolist() if l + 1 < NL else None
            xd = xn.view(torch.int16)
    finally:
        for lay in lays:
            lay.close()
    print("lookahead precision on this stack: %.3f" % (hits / ((NL - 1) * T * K)))
