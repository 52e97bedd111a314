"""Pins of the oracle's dual-scaling variance normalization (rndamp article on
KVarN, "How It Works", item 2; abstract of arXiv 2606.03458: scaling on both
axes of K and V). Readings SC-4 (uncentred mean of squares) and SC-5 (c
starts at 1; an iteration is a row step then a column step; 4 iterations)."""
import numpy as np
import pytest
import scipy.linalg
import torch

import kvgen
from golden_io import keyed

TAU = 1e-3  # row-uniformity tolerance after 4 iterations (SC-5)


def _rank1(rng, T, D):
    a = np.exp(rng.standard_normal(T))
    b = np.exp(rng.standard_normal(D))
    s = rng.choice([-1.0, 1.0], size=(T, D))
    return a, b, s * np.sqrt(np.outer(a, b))


@pytest.mark.parametrize("T,D", [(2, 4), (16, 8), (128, 128), (256, 128)])
def test_rank_one_closed_form(oracle, T, D):
    rng = np.random.default_rng(T * 1000 + D)
    a, b, y = _rank1(rng, T, D)
    for iters in (1, 2, 4):
        r, c, eps = oracle.balance(y, iters)
        np.testing.assert_allclose(r, np.sqrt(a * b.mean()), rtol=1e-12)
        np.testing.assert_allclose(c, np.sqrt(b / b.mean()), rtol=1e-12)
        assert np.all(eps < 1e-12)


def test_golden_rank1_block(oracle):
    g = keyed("rank1_block.txt")
    x = np.array(g["x"])
    out = oracle.quantize_block(x, int(g["iters"][0][0]))
    np.testing.assert_allclose(out["c"], g["c"][0], rtol=1e-14)
    np.testing.assert_allclose(out["rp"], g["rprime"][0], rtol=1e-14)
    np.testing.assert_array_equal(out["codes"], np.array(g["codes"], np.uint8))
    r, c, _ = oracle.balance(oracle.rotate(x), 4)
    np.testing.assert_allclose(r, g["r"][0], rtol=1e-14)


def _gen_blocks(n_blocks=4):
    """Blocks from the synthetic generator for every workload's value
    distribution (fp64 copies of the exact values the device would read)."""
    for wl in kvgen.WORKLOADS:
        for tensor in (kvgen.K, kvgen.V):
            x = kvgen.kv_tensor(wl.seed, 0, tensor, 1, n_blocks, 128, wl.sigma,
                                dtype=wl.dtype)
            for h in range(n_blocks):
                yield wl.name, x[0, h].double().numpy()


def test_balance_tolerance_and_invariants(oracle):
    for name, x in _gen_blocks():
        y = oracle.rotate(x)
        r, c, eps = oracle.balance(y, 4)
        assert eps[-1] <= TAU, (name, eps)
        assert eps[-1] <= eps[0], (name, eps)
        z2 = (y / (r[:, None] * c[None, :])) ** 2
        # after a column step every column has mean square exactly 1
        np.testing.assert_allclose(z2.mean(axis=0), 1.0, atol=1e-12)
        # rows are uniform to eps (recomputed independently here)
        assert np.max(np.abs(z2.mean(axis=1) - 1.0)) == pytest.approx(eps[-1],
                                                                        rel=1e-9)


def test_each_iteration_column_step_exact(oracle):
    rng = np.random.default_rng(3)
    y = rng.standard_normal((128, 128)) * np.exp(rng.standard_normal((128, 1)))
    for k in (1, 2, 3, 4, 7):
        r, c, _ = oracle.balance(y, k)
        z2 = (y / (r[:, None] * c[None, :])) ** 2
        np.testing.assert_allclose(z2.mean(axis=0), 1.0, atol=1e-12)


def test_token_scaling_equivariance(oracle):
    """Scaling token i by beta > 0 leaves c and all codes unchanged and
    scales only r'_i by beta (the row step absorbs it before any column step
    sees it). A column-first order or a transposed operand breaks this."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((128, 128)) * np.exp(0.5 * rng.standard_normal((128, 1)))
    base = oracle.quantize_block(x, 4)
    beta = np.exp(rng.standard_normal(128))
    beta[::7] = 2.0 ** rng.integers(-6, 7, size=beta[::7].shape)
    got = oracle.quantize_block(x * beta[:, None], 4)
    np.testing.assert_allclose(got["c"], base["c"], rtol=1e-12)
    np.testing.assert_allclose(got["rp"], base["rp"] * beta, rtol=1e-12)
    ok = ~oracle.boundary_mask(base["u"], 1e-9)
    np.testing.assert_array_equal(got["codes"][ok], base["codes"][ok])
    # power-of-two scaling is exact in binary floating point
    p2 = beta.copy()
    p2[:] = 2.0 ** rng.integers(-6, 7, size=128)
    got2 = oracle.quantize_block(x * p2[:, None], 4)
    np.testing.assert_array_equal(got2["c"], base["c"])
    np.testing.assert_array_equal(got2["rp"], base["rp"] * p2)
    np.testing.assert_array_equal(got2["codes"], base["codes"])


def test_token_permutation_equivariance(oracle):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((128, 128)) * np.exp(0.5 * rng.standard_normal((128, 1)))
    base = oracle.quantize_block(x, 4)
    perm = rng.permutation(128)
    got = oracle.quantize_block(x[perm], 4)
    np.testing.assert_allclose(got["c"], base["c"], rtol=1e-12)
    np.testing.assert_allclose(got["rp"], base["rp"][perm], rtol=1e-12)
    ok = ~oracle.boundary_mask(base["u"][perm], 1e-9)
    np.testing.assert_array_equal(got["codes"][ok], base["codes"][perm][ok])


def test_zero_rows_and_columns(oracle):
    y = np.zeros((8, 4))
    y[:4, :2] = np.arange(1, 9).reshape(4, 2)
    r, c, eps = oracle.balance(y, 3)
    assert np.all(r[4:] == 1.0)       # zero rows keep r = 1 (SC-9)
    assert np.all(c[2:] == 1.0)       # zero columns keep c = 1 (SC-9)
    out = oracle.quantize_block(oracle.rotate(y), 3)
    np.testing.assert_array_equal(out["rp"][4:], 0.0)
    np.testing.assert_array_equal(out["codes"][4:], 2)


def test_iters_zero_is_rotation_only(oracle):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 128))
    out = oracle.quantize_block(x, 0)
    np.testing.assert_array_equal(out["c"], 1.0)
    y = x @ scipy.linalg.hadamard(128) / np.sqrt(128)
    np.testing.assert_allclose(out["rp"], np.abs(y).max(axis=1) / 2, rtol=1e-13)


def test_nonfinite_input_raises(oracle):
    x = np.ones((4, 8))
    x[1, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.quantize_block(x, 4)
