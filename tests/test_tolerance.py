"""The per-element gradient bound (oracle.tolerance) behaves as stated."""
import numpy as np
import pytest

from oracle.tolerance import GRAD_ABS, GRAD_REL, grad_excess, grad_ok, max_abs_err


def test_per_element_not_tensor_wide():
    ref = np.array([10.0, 0.01])
    # the large element may be off by 2e-2 + 10/256; the small one only by ~2e-2
    assert grad_ok(ref + np.array([GRAD_ABS + 10 * GRAD_REL - 1e-6, 0.0]), ref)
    assert not grad_ok(ref + np.array([0.0, 0.03]), ref)          # a tensor-wide bound would pass this
    assert not grad_ok(ref + np.array([GRAD_ABS + 10 * GRAD_REL + 1e-6, 0.0]), ref)


def test_excess_value_and_shapes():
    ref = np.array([[1.0, -2.0], [0.0, 4.0]])
    got = ref + np.array([[0.0, 0.0], [0.01, -0.05]])
    assert grad_excess(got, ref) == pytest.approx(0.05 - 4 * GRAD_REL)
    assert max_abs_err(got, ref) == pytest.approx(0.05)
    assert grad_excess(np.zeros(0), np.zeros(0)) == float("-inf")
    with pytest.raises(ValueError):
        grad_excess(np.zeros(3), np.zeros(4))
