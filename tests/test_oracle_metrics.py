"""Pins of the oracle's comparison function (CPU only).

Every parity check compares a GPU result with its fp64 reference through
``oracle.metrics``: rel-L2 = |x - ref|_2 / |ref|_2, max-abs = max |x - ref| and
the finiteness of x.  These values are computed here by hand, so that a wrong
norm, a silent broadcast or a swallowed NaN cannot make the GPU checks vacuous.
"""

import math

import numpy as np
import pytest

from oracle import metrics


def test_hand_computed_vector():
    # d = x - ref = [0, 0, -2]: |d| = 2, |ref| = sqrt(1 + 4 + 25) = sqrt(30)
    m = metrics(np.array([1.0, 2.0, 3.0]), np.array([1.0, 2.0, 5.0]))
    assert m["rel_l2"] == pytest.approx(2.0 / math.sqrt(30.0), rel=1e-15)
    assert m["max_abs"] == 2.0
    assert m["finite"] is True


def test_hand_computed_matrix_and_sign():
    ref = np.array([[1.0, -2.0], [3.0, 0.5]])
    x = np.array([[1.5, -2.0], [2.0, 0.5]])
    # d = [[0.5, 0], [-1, 0]]: |d| = sqrt(1.25), |ref| = sqrt(1 + 4 + 9 + 0.25)
    m = metrics(x, ref)
    assert m["rel_l2"] == pytest.approx(math.sqrt(1.25) / math.sqrt(14.25), rel=1e-15)
    assert m["max_abs"] == 1.0


def test_identical_is_zero_and_transposed_is_not():
    ref = np.arange(12, dtype=np.float64).reshape(3, 4) - 5.0
    m = metrics(ref.copy(), ref)
    assert m["rel_l2"] == 0.0 and m["max_abs"] == 0.0
    sq = np.arange(16, dtype=np.float64).reshape(4, 4)
    assert metrics(sq.T, sq)["rel_l2"] > 0.5


def test_zero_reference_reports_the_absolute_norm():
    x = np.array([[1.0, -1.0], [0.0, 2.0]])
    m = metrics(x, np.zeros((2, 2)))
    assert m["rel_l2"] == pytest.approx(math.sqrt(6.0), rel=1e-15)
    assert m["max_abs"] == 2.0
    assert metrics(np.zeros(3), np.zeros(3))["rel_l2"] == 0.0


def test_non_finite_result_fails_every_bar():
    for bad in (np.nan, np.inf, -np.inf):
        m = metrics(np.array([1.0, bad, 3.0]), np.array([1.0, 2.0, 3.0]))
        assert m["finite"] is False
        assert m["rel_l2"] == float("inf") and m["max_abs"] == float("inf")


def test_shape_mismatch_raises_instead_of_broadcasting():
    with pytest.raises(ValueError):
        metrics(np.zeros(3), np.zeros((3, 1)))
    with pytest.raises(ValueError):
        metrics(np.zeros((2, 3)), np.zeros((3, 2)))
    with pytest.raises(ValueError):
        metrics(np.zeros(1), np.zeros(4))  # would broadcast without the check


def test_non_finite_reference_raises():
    with pytest.raises(ValueError):
        metrics(np.zeros(3), np.array([0.0, np.nan, 1.0]))


def test_empty_tensors():
    m = metrics(np.zeros((0, 4)), np.zeros((0, 4)))
    assert m == {"rel_l2": 0.0, "max_abs": 0.0, "finite": True}
