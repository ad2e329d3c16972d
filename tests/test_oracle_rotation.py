"""Pins for the oracle's rotation: the normalised Walsh-Hadamard matrix
(ResidualQuant, newx.sg page, AI Summary: the residual rotation is orthogonal)."""
import numpy as np
import pytest
import scipy.linalg

import oracle


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_matches_scipy_sylvester(d):
    # scipy builds the same Sylvester-order matrix independently
    np.testing.assert_array_equal(oracle.hadamard(d) * np.sqrt(d), scipy.linalg.hadamard(d))


@pytest.mark.parametrize("d", [32, 64, 128])
def test_orthogonal_symmetric_involutory(d):
    h = oracle.hadamard(d)
    np.testing.assert_allclose(h @ h.T, np.eye(d), atol=1e-15)
    np.testing.assert_array_equal(h, h.T)
    np.testing.assert_allclose(h @ h, np.eye(d), atol=1e-15)


def _butterfly(x):
    """In-place fast Walsh-Hadamard transform (natural order), written
    independently of the dense matrix as a cross-check."""
    x = np.array(x, dtype=np.float64, copy=True)
    n = x.shape[-1]
    span = 1
    while span < n:
        for start in range(0, n, 2 * span):
            a = x[..., start:start + span].copy()
            b = x[..., start + span:start + 2 * span].copy()
            x[..., start:start + span] = a + b
            x[..., start + span:start + 2 * span] = a - b
        span *= 2
    return x / np.sqrt(n)


@pytest.mark.parametrize("d", [64, 128])
def test_rotate_equals_butterfly_and_preserves_norm(d):
    r = np.random.default_rng(1).standard_normal((50, d))
    y = oracle.rotate(r)
    np.testing.assert_allclose(y, _butterfly(r), atol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(r, axis=-1), rtol=1e-14)


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.hadamard(48)
