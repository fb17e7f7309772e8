"""The tolerance check of the GPU parity tests, tested on the CPU: it must reject outputs that are off by more
than the bar (relative Frobenius error 4e-3, elementwise 1e-2 of max|ref|), accept outputs within it, and
reject non-finite outputs."""
import numpy as np
import pytest

import _parity


def _ref(seed=5, shape=(64, 96)):
    return np.random.default_rng(seed).standard_normal(shape)


def test_uniform_relative_perturbation_of_1e3_passes():
    R = _ref()
    rel, mx = _parity.assert_close(R * (1 + 1e-3), R)
    assert abs(rel - 1e-3) < 1e-9


def test_uniform_relative_perturbation_of_5e3_fails():
    R = _ref()
    with pytest.raises(AssertionError):
        _parity.assert_close(R * (1 + 5e-3), R)


def test_one_element_beyond_the_elementwise_bar_fails():
    # a single element off by 2% of max|ref|: tiny Frobenius error, caught by the elementwise bound
    R = _ref()
    G = R.copy()
    G[7, 11] += 0.02 * np.abs(R).max()
    rel, mx = _parity.compare(G, R)
    assert rel < 4e-3 and mx > 1e-2
    with pytest.raises(AssertionError):
        _parity.assert_close(G, R)


def test_bf16_rounding_of_the_reference_passes():
    # the output rounding alone (the expected GPU error) is inside the bar
    import oracle
    R = _ref()
    G = _parity.widen_bits(oracle.round_bf16(R))
    rel, mx = _parity.assert_close(G, R)
    assert 5e-4 < rel < 3e-3


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_output_fails(bad):
    R = _ref()
    G = R.copy()
    G[3, 4] = bad
    with pytest.raises(AssertionError):
        _parity.assert_close(G, R)


def test_non_finite_reference_fails():
    R = _ref()
    G = R.copy()
    R[0, 0] = np.nan
    with pytest.raises(AssertionError):
        _parity.assert_close(G, R)


def test_shape_mismatch_fails():
    R = _ref()
    with pytest.raises(AssertionError):
        _parity.assert_close(R[:, :-1], R)
