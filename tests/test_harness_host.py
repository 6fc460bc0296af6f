"""Host logic of the GPU parity harness, on the CPU: the acceptance rule for
bf16 roundings of h that differ from the oracle's (tests/gpu_harness.py,
validate_h) accepts a rounding of a value within the fp32 error bound of the
exact one -- the other neighbour near a midpoint, several steps where the
dot products cancel -- and rejects the rest, and a large share of
differing elements."""
import numpy as np
import pytest

from tests import gpu_harness as gh


def _pre(h_exact, g=2.0, gabs=1.0, uabs=1.0):
    silu = g / (1.0 + np.exp(-g))
    u = h_exact / silu
    one = lambda v: np.array([[v]], dtype=np.float64)  # noqa: E731
    return lambda rows, cols: dict(g=one(g), u=one(u), h=one(h_exact), gabs=one(gabs),
                                   uabs=one(uabs))


K = 4096          # the bound is K 2^-24 sum|x w| through the SwiGLU, about 2.4e-4 here
ONE, ONE_UP, ONE_UP2 = 0x3F80, 0x3F81, 0x3F82   # 1, 1 + 2^-7, 1 + 2^-6
MID = 1.0 + 2.0 ** -8


def test_identical_roundings_need_no_bound():
    h = np.array([[ONE]], np.uint16)
    rep = gh.validate_h(h, h.copy(), _pre(1.0), 7.0, K)
    assert rep["flips"] == 0


def test_other_neighbour_near_a_midpoint_is_accepted():
    # exact value just below the midpoint: the oracle rounds down to 1, the
    # GPU (its fp32 value a little above) up to 1 + 2^-7: both correct
    rep = gh.validate_h(np.array([[ONE_UP]], np.uint16), np.array([[ONE]], np.uint16),
                        _pre(MID - 1e-6), 7.0, K)
    assert rep["flips"] == 1 and rep["flip_max_over_bound"] <= 1.0


def test_flip_far_from_a_midpoint_is_rejected():
    with pytest.raises(AssertionError):
        gh.validate_h(np.array([[ONE_UP]], np.uint16), np.array([[ONE]], np.uint16),
                      _pre(1.0001), 7.0, K)


def test_two_steps_away_is_rejected_when_the_bound_is_tight():
    with pytest.raises(AssertionError):
        gh.validate_h(np.array([[ONE_UP2]], np.uint16), np.array([[ONE]], np.uint16),
                      _pre(MID - 1e-6), 7.0, K)


def test_several_steps_are_accepted_where_the_dot_products_cancel():
    # sum|x w| far above the result: the fp32 value may lie several bf16
    # steps from the exact one (2^-6 away here, bound about 2.4e-2)
    rep = gh.validate_h(np.array([[ONE_UP2]], np.uint16), np.array([[ONE]], np.uint16),
                        _pre(1.0, gabs=100.0, uabs=100.0), 7.0, K)
    assert rep["flips"] == 1 and rep["flip_max_over_bound"] <= 1.0


def test_neighbour_on_the_same_side_is_rejected():
    # exact value above 1 + 2^-7 by more than the bound: only 1 + 2^-7 is a
    # correct rounding, 1 is not
    with pytest.raises(AssertionError):
        gh.validate_h(np.array([[ONE]], np.uint16), np.array([[ONE_UP]], np.uint16),
                      _pre(1.0 + 2.0 ** -7 + 1e-3), 7.0, K)


def test_a_large_share_of_differences_is_rejected():
    n = 2000
    h_ora = np.full((1, n), ONE, np.uint16)
    h_gpu = h_ora.copy()
    h_gpu[0, :100] = ONE_UP      # 5 % of the elements
    with pytest.raises(AssertionError):
        gh.validate_h(h_gpu, h_ora, _pre(MID - 1e-6), 7.0, K)
