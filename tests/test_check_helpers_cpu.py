"""CPU tests of the parity helpers used by the GPU tests: the routing check
accepts exactly the near-tie of the router-precision reading and nothing
else."""
import numpy as np
import pytest

from tests.gpu_common import check_routing


def _case():
    # one token, 6 experts, k = 3; choice values with a near-tie between
    # rank 3 (expert 4) and rank 4 (expert 1)
    c = np.array([[0.10, 0.5 - 1e-14, 0.9, 0.2, 0.5, 0.7]])
    idx_o = np.array([[2, 5, 4]], np.int32)
    w_o = np.array([[0.4, 0.35, 0.25]], np.float32)
    return c, idx_o, w_o


def test_identical_routing_passes():
    c, idx_o, w_o = _case()
    check_routing(idx_o.copy(), w_o.copy(), idx_o, w_o, c)


def test_boundary_near_tie_is_accepted():
    c, idx_o, w_o = _case()
    check_routing(np.array([[2, 5, 1]], np.int32), np.array([[0.4, 0.35, 0.25]], np.float32),
                  idx_o, w_o, c, r=1.0)


def test_swap_before_the_tied_run_fails():
    c, idx_o, w_o = _case()
    with pytest.raises(AssertionError):
        check_routing(np.array([[5, 2, 1]], np.int32), w_o.copy(), idx_o, w_o, c)


def test_expert_outside_the_tied_run_fails():
    c, idx_o, w_o = _case()
    with pytest.raises(AssertionError):
        check_routing(np.array([[2, 5, 3]], np.int32), w_o.copy(), idx_o, w_o, c)


def test_no_exemption_without_a_boundary_tie():
    # a near-tie between ranks 1 and 2 does not excuse a different selection
    c = np.array([[0.9, 0.9 - 1e-14, 0.5, 0.1]])
    idx_o = np.array([[0, 1]], np.int32)
    w_o = np.array([[0.5, 0.5]], np.float32)
    with pytest.raises(AssertionError):
        check_routing(np.array([[1, 0]], np.int32), w_o.copy(), idx_o, w_o, c)
    with pytest.raises(AssertionError):
        check_routing(np.array([[0, 2]], np.int32), w_o.copy(), idx_o, w_o, c)


def test_weights_of_matching_tokens_are_compared():
    c, idx_o, w_o = _case()
    with pytest.raises(AssertionError):
        check_routing(idx_o.copy(), w_o * 1.001, idx_o, w_o, c)


def test_bf16_check_accepts_rounding_and_catches_a_wrong_step():
    from quantized_expert_ffn_topk_amd import synth
    from tests.gpu_common import check_bf16_out
    r = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    bits = synth.f32_to_bf16_bits(r)
    e, same = check_bf16_out(bits, r)
    assert same == 1.0 and e == 0.0
    planted = bits.copy()
    planted[5] += 1                       # one step off, away from a midpoint
    with pytest.raises(AssertionError):
        check_bf16_out(planted, r)
    # a value sitting on a midpoint may round either way
    mid = np.array([1.0 + 2 ** -8, 2.0], np.float32)
    up = synth.f32_to_bf16_bits(np.array([1.0 + 2 ** -7, 2.0], np.float32))
    check_bf16_out(up, mid)


def test_bf16_check_without_same_rounding_keeps_the_bar():
    from quantized_expert_ffn_topk_amd import synth
    from tests.gpu_common import check_bf16_out
    r = np.random.default_rng(1).standard_normal(1000).astype(np.float32)
    # sums off by 1e-4 of the largest output round to other bf16 values: fine
    # without same_rounding, caught with it
    near = r + np.float32(1e-4) * np.abs(r).max()
    bits = synth.f32_to_bf16_bits(near)
    with pytest.raises(AssertionError):
        check_bf16_out(bits, r)
    e, _ = check_bf16_out(bits, r, same_rounding=False)
    assert e <= 1.1e-4
    # 3e-3 of the largest output away: outside the bar either way
    far = synth.f32_to_bf16_bits(r + np.float32(3e-3) * np.abs(r).max())
    with pytest.raises(AssertionError):
        check_bf16_out(far, r, same_rounding=False)
