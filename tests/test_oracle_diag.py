"""Pins of the oracle's per-token magnitude/direction error (kvo_token_error):
closed forms (scaling, plane rotations, opposite and orthogonal vectors), the
degenerate tokens, the law-of-cosines identity linking both numbers to the
squared error, and invariance under an orthogonal rotation and a common scale
(the property that lets the device compare in the rotated basis)."""
import numpy as np
import pytest
import scipy.linalg

import oracle


def test_scaling_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 128))
    for a in (0.25, 1.0, 3.5):
        ratio, cosine = oracle.token_error(x, a * x)
        np.testing.assert_allclose(ratio, a, rtol=1e-14)
        np.testing.assert_allclose(cosine, 1.0, rtol=1e-14)
    ratio, cosine = oracle.token_error(x, -2.0 * x)
    np.testing.assert_allclose(ratio, 2.0, rtol=1e-14)
    np.testing.assert_allclose(cosine, -1.0, rtol=1e-14)


@pytest.mark.parametrize("theta", [0.1, 0.7, np.pi / 2, 2.5])
def test_plane_rotation_closed_form(theta):
    """xhat = x turned by theta inside the plane of x and a unit vector
    orthogonal to it: ratio 1, cosine cos(theta)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(64)
    u = rng.standard_normal(64)
    u -= (u @ x) / (x @ x) * x
    u /= np.linalg.norm(u)
    xhat = np.cos(theta) * x + np.sin(theta) * np.linalg.norm(x) * u
    ratio, cosine = oracle.token_error(x[None], xhat[None])
    assert abs(ratio[0] - 1.0) < 1e-13
    assert abs(cosine[0] - np.cos(theta)) < 1e-13


def test_degenerate_tokens():
    z = np.zeros(8)
    e = np.eye(8)[2]
    ratio, cosine = oracle.token_error(np.stack([z, z, e]), np.stack([z, e, z]))
    assert ratio[0] == 1.0 and cosine[0] == 1.0
    assert np.isinf(ratio[1]) and cosine[1] == 0.0
    assert ratio[2] == 0.0 and cosine[2] == 0.0


def test_law_of_cosines():
    """||xhat - x||^2 = ||x||^2 (ratio^2 + 1 - 2 ratio cos): a dropped term or
    a wrong sign in either number breaks it."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 128)) * rng.lognormal(0, 1, (50, 1))
    xhat = x * rng.uniform(0.5, 1.5, (50, 1)) + 0.3 * rng.standard_normal((50, 128))
    ratio, cosine = oracle.token_error(x, xhat)
    nx2 = np.einsum("ij,ij->i", x, x)
    lhs = np.einsum("ij,ij->i", xhat - x, xhat - x)
    np.testing.assert_allclose(lhs, nx2 * (ratio ** 2 + 1 - 2 * ratio * cosine), rtol=1e-10)


def test_rotation_and_scale_invariance():
    rng = np.random.default_rng(3)
    H = scipy.linalg.hadamard(128) / np.sqrt(128)
    x = rng.standard_normal((20, 128))
    xhat = x + 0.2 * rng.standard_normal((20, 128))
    r0, c0 = oracle.token_error(x, xhat)
    r1, c1 = oracle.token_error(x @ H, xhat @ H)
    r2, c2 = oracle.token_error(7.0 * x, 7.0 * xhat)
    np.testing.assert_allclose(r1, r0, rtol=1e-12)
    np.testing.assert_allclose(c1, c0, rtol=1e-12)
    np.testing.assert_allclose(r2, r0, rtol=1e-12)
    np.testing.assert_allclose(c2, c0, rtol=1e-12)


def test_cache_token_error_matches_reconstruction():
    """On a quantized block the cache form is the plain form on the oracle's
    own reconstruction; with iters = 0 and with iters = 4 both numbers stay
    in range (ratio > 0, |cos| <= 1)."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((128, 128)) * rng.lognormal(0, 0.5, (128, 1))
    for iters in (0, 4):
        q = oracle.quantize_block(x, iters=iters)
        ratio, cosine = oracle.cache_token_error(x, q["codes"], q["rp"], q["c"][None])
        r2, c2 = oracle.token_error(x, oracle.dequant(q["codes"], q["rp"], q["c"][None]))
        np.testing.assert_array_equal(ratio, r2)
        np.testing.assert_array_equal(cosine, c2)
        assert np.all(ratio > 0) and np.all(np.abs(cosine) <= 1 + 1e-12)
