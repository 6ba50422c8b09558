"""CPU checks of the GPU tests' tolerance helpers."""
import numpy as np
import torch

import _tol


def test_ulp_and_rounding():
    assert _tol.ulp(1.0, torch.bfloat16) == 2.0 ** -7
    assert _tol.ulp(1.999, torch.bfloat16) == 2.0 ** -7
    assert _tol.ulp(0.75, torch.float16) == 2.0 ** -11
    assert _tol.rne(np.array([1.0 + 2.0 ** -8]), torch.bfloat16)[0] == 1.0          # tie to even
    assert _tol.rne(np.array([1.0 + 3 * 2.0 ** -8]), torch.bfloat16)[0] == 1.0 + 2.0 ** -6


def test_tmp_budget_one_partition_is_half_an_ulp():
    o = np.array([[0.3, 1.5, -3.0]])
    b = _tol.tmp_rounding_budget([2.0], [7.0], o, torch.bfloat16)
    assert np.allclose(b, 0.5 * _tol.ulp(o[0], torch.bfloat16))


def test_tmp_budget_weights_partitions():
    # equal weights (same m_p and l_p): the budget is the mean of the half-ulps;
    # a partition with m_p = -inf-like weight contributes nothing
    o = np.array([[1.5], [0.1]])
    b = _tol.tmp_rounding_budget([1.0, 1.0], [4.0, 4.0], o, torch.bfloat16)
    assert np.isclose(b[0], 0.5 * (0.5 * 2.0 ** -7 + 0.5 * 2.0 ** -11))
    b = _tol.tmp_rounding_budget([0.0, -800.0], [4.0, 4.0], o, torch.bfloat16)
    assert np.isclose(b[0], 0.5 * 2.0 ** -7)


def test_check_catches_drift_the_rounded_check_allows():
    ref = np.array([1.0 + 2.0 ** -8 - 1e-6])       # just below a bf16 rounding midpoint
    got = np.array([1.0 + 2.0 ** -7])              # one ulp up: allowed by the rounded check alone
    _tol.check(got, ref, torch.bfloat16, 2e-3 + 2.0 ** -8, "budget covers it")
    try:
        _tol.check(np.array([1.0 + 2.0 ** -6]), ref, torch.bfloat16, 2e-3, "two ulps")
    except AssertionError:
        pass
    else:
        raise AssertionError("two ulps of drift passed")
