"""The parity checker itself (no GPU): the per-unit bar catches a wrong region
too small to move the whole-tensor error ratio, and holds near-zero units to
the tensor's typical scale rather than to their own."""
import numpy as np
import pytest

from _util import TOL, check, ratio, unit_ratios


def noisy(shape, rel=0.003, seed=0):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal(shape)
    return ref, ref * (1.0 + rel * rng.standard_normal(shape))


def test_one_wrong_token_of_a_long_sequence_fails():
    ref, x = noisy((1, 65536, 1, 128))
    x[0, 40000, 0] = 0.0
    assert ratio(x, ref) <= TOL            # invisible to the whole-tensor ratio
    worst = max(unit_ratios(x, ref, "tok"), key=lambda t: t[1])
    assert worst[0] == (0, 40000 // 64, 0) and worst[1] > 0.1
    with pytest.raises(AssertionError):
        check("o", x, ref, "tok")


def test_one_wrong_token_of_a_packed_sequence_fails():
    ref, x = noisy((1, 300, 2, 4))
    cu = np.array([0, 10, 11, 300])
    x[0, 10, 1] += 0.5 * np.abs(ref[0, 10, 1]).max() + 0.5   # the 1-token sequence
    worst = max(unit_ratios(x, ref, "tok", cu), key=lambda t: t[1])
    assert worst[0] == (1, 0, 1) and worst[1] > TOL


def test_wrong_state_row_fails():
    ref, x = noisy((8, 4, 16, 16))
    x[5, 2] *= -1.0
    with pytest.raises(AssertionError):
        check("final_state", x, ref, "state")


def test_near_zero_unit_is_held_to_the_typical_scale():
    # a unit whose exact values are 1/50 of the typical magnitude, computed
    # with an absolute error at the rounding level of typical values: a
    # 5 % relative error of its own, but 0.001 of a typical unit
    ref, x = noisy((1, 640, 1, 8))
    ref[0, 64:128] *= 0.02
    x[0, 64:128] = ref[0, 64:128] + 0.001 * np.sign(ref[0, 64:128])
    units = dict(unit_ratios(x, ref, "tok"))
    assert units[(0, 1, 0)] <= TOL
    check("dbeta", x, ref, "tok")
    # the same absolute error on a typical unit is its own relative error
    x2 = ref.copy()
    x2[0, 0:64] = 0.0
    assert dict(unit_ratios(x2, ref, "tok"))[(0, 0, 0)] > 0.5


def test_all_zero_reference_units_need_all_zero_results():
    ref = np.zeros((1, 128, 1, 4))
    ref[0, :64] = 1.0
    x = ref.copy()
    x[0, 100] = 0.5     # a wrong value where the exact result is 0
    worst = max(unit_ratios(x, ref, "tok"), key=lambda t: t[1])
    assert worst[0] == (0, 1, 0) and worst[1] > TOL
