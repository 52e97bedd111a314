"""Pins of the oracle's Hadamard rotation (rndamp article on KVarN, "How It
Works", item 1: a Hadamard transform along the channel dimension; reading
SC-1: Sylvester order, scaled by 1/sqrt(D), no random signs)."""
import numpy as np
import pytest
import scipy.linalg

from golden_io import rotate_cases


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_rotate_matches_scipy_hadamard(oracle, d):
    # Library routine: scipy builds the Sylvester Hadamard matrix itself.
    got = oracle.rotate(np.eye(d))
    want = scipy.linalg.hadamard(d) / np.sqrt(d) if d > 1 else np.ones((1, 1))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_rotate_golden_h4(oracle):
    for x, y in rotate_cases():
        np.testing.assert_allclose(oracle.rotate(x[None])[0], y, atol=1e-15)


def test_rotate_orthogonal_and_involution(oracle):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 128)) * np.exp(rng.standard_normal((64, 1)))
    y = oracle.rotate(x)
    # norm preservation row by row (closed form of an orthogonal map)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1),
                               rtol=1e-13)
    # H H = D I: rotating twice is the identity
    np.testing.assert_allclose(oracle.rotate(y), x, rtol=0, atol=1e-12)
    # inner products preserved (H^T H / D = I)
    np.testing.assert_allclose(y @ y.T, x @ x.T, rtol=1e-12, atol=1e-10)


def test_rotate_constant_and_basis(oracle):
    d = 128
    y = oracle.rotate(np.ones((1, d)))[0]
    want = np.zeros(d)
    want[0] = np.sqrt(d)
    np.testing.assert_allclose(y, want, atol=1e-13)
    # e_k maps to row k of H / sqrt(d): entries (-1)^popcount(k & j) / sqrt(d)
    for k in (0, 1, 5, 77, 127):
        e = np.zeros((1, d))
        e[0, k] = 1.0
        row = oracle.rotate(e)[0] * np.sqrt(d)
        want = np.array([(-1) ** bin(k & j).count("1") for j in range(d)], float)
        np.testing.assert_array_equal(row, want)


def test_rotate_rejects_bad_dim(oracle):
    with pytest.raises(oracle.OracleError):
        oracle.rotate(np.ones((2, 6)))
