"""GPU test of moe_layer_forward_noalloc (the allocation-free layer forward):
its outputs equal those of moe_layer_forward on a context, bit for bit, over
calls in a row on the one scratch array of the GPU, each call smaller than the
one before, on every kernel path; a call too large for the array is rejected
before anything is enqueued."""
import numpy as np
import pytest

from quantized_expert_ffn_topk_amd import abi, synth
from tests.gpu_common import Case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _noalloc(lay, x, T):
    idx, w, out = lay._outs(T)
    for t in (idx, w, out):
        t.fill_(-3)
    abi.moe_layer_forward_noalloc(lay.desc, x, T, lay.weights, idx, w, out)
    return idx, w, out


def _same(a, b):
    return all(torch.equal(p.view(torch.int32), q.view(torch.int32)) for p, q in zip(a, b))


@pytest.mark.parametrize("shape", ["int4", "int4_bf16", "mxfp4"])
def test_noalloc_equals_context_forward_on_calls_in_a_row(shape):
    # MFMA path (70 tokens), few-token GEMV path (5), one-token kernels (1):
    # each call reuses the array the one before left behind
    H, F, E, k = 512, 256, 16, 4
    if shape == "mxfp4":
        from tests.test_gpu_mx import MxCase
        c = MxCase(81, 70, H, F, E, k, 1, r=1.5, n_distinct=5)
        lay = c.layer(max_tokens=70)
        sizes = (70, 5, 1)
    else:
        dt = abi.DT_BF16 if shape == "int4_bf16" else abi.DT_F32
        c = Case(80, 70, H, F, E, k, 1, r=2.5, n_distinct=5)
        lay = c.layer(max_tokens=70, out_dtype=dt)
        sizes = (70, 5, 1)
    x = lay.x_tensor(c.x)
    for T in sizes:
        want = lay.forward(x[:T])
        got = _noalloc(lay, x[:T], T)
        torch.cuda.synchronize()
        assert _same(got, want), (shape, T)
    lay.close()


def test_noalloc_glm_decode_two_steps_and_the_size_limit():
    # GLM-shaped layer (hidden 6144, 256 routed + 1 shared, F 2048, top-8):
    # 16 tokens then 1 token against the context forward, then a call whose
    # workspace exceeds the array is refused and writes nothing
    H, F, E, k = 6144, 2048, 256, 8
    c = Case(0, 16, H, F, E, k, 1, r=2.5, n_distinct=4)
    lay = c.layer(max_tokens=16)
    x = lay.x_tensor(c.x)
    for T in (16, 1):
        want = lay.forward(x[:T])
        got = _noalloc(lay, x[:T], T)
        torch.cuda.synchronize()
        assert _same(got, want), T
    big = 256
    xb = lay.x_tensor(synth.activations(3, big, H))
    idx, w, out = lay._outs(big)
    out.fill_(-3)
    with pytest.raises(abi.MoEError) as ei:
        abi.moe_layer_forward_noalloc(lay.desc, xb, big, lay.weights, idx, w, out)
    assert ei.value.status == abi.E_INVAL
    torch.cuda.synchronize()
    assert bool((out == -3).all())
    lay.close()
