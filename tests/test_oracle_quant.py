"""Pins of the oracle's range step, 2-bit codes and packing (abstract of arXiv
2606.03458: 2-bit KV cache; rndamp article, "Numbers": two scales fused into
the dequantization). Readings SC-6 (mid-rise grid), SC-7 (per-token range step
folded into the row scale), SC-8 (ties up), SC-10 (packed layout)."""
import itertools

import numpy as np
import pytest
import scipy.linalg

import kvgen
from golden_io import keyed, lines

LEVELS = np.array([-1.5, -0.5, 0.5, 1.5])


def _blocks():
    rng = np.random.default_rng(11)
    yield rng.standard_normal((128, 128)) * np.exp(0.5 * rng.standard_normal((128, 1)))
    for wl in (kvgen.WORKLOADS[0], kvgen.WORKLOADS[4]):
        x = kvgen.kv_tensor(wl.seed, 0, kvgen.K, 1, 2, 128, wl.sigma, dtype=wl.dtype)
        yield x[0, 1].double().numpy()


def test_half_step_bound_and_range_use(oracle):
    for x in _blocks():
        out = oracle.quantize_block(x, 4)
        u, codes = out["u"], out["codes"].astype(float)
        # every value lies within half a step of its level
        assert np.all(np.abs((codes - 1.5) - u) <= 0.5 + 1e-12)
        # the range step is used fully: each row reaches |u| = 2 exactly once
        np.testing.assert_allclose(np.abs(u).max(axis=1), 2.0, rtol=1e-14)
        at_max = np.abs(np.abs(u) - 2.0) < 1e-12
        assert np.all(np.isin(out["codes"][at_max], [0, 3]))
        # minimality: a step one part in 1e9 smaller pushes some |u| past 2
        y = oracle.rotate(x)
        shrunk = np.abs(y / (out["rp"][:, None] * (1 - 1e-9) * out["c"][None, :]))
        assert np.all(shrunk.max(axis=1) > 2.0)


def test_dequant_error_bound_original_basis(oracle):
    """|Zhat - Z| <= step/2 elementwise in the rotated basis implies
    ||Xhat - X||_F^2 <= sum_ij (r'_i c_j / 2)^2 in the original one."""
    for x in _blocks():
        out = oracle.quantize_block(x, 4)
        xh = oracle.dequant(out["codes"], out["rp"], out["c"][None, :])
        bound = np.sum((out["rp"][:, None] * out["c"][None, :] / 2) ** 2, axis=1)
        assert np.all(np.sum((xh - x) ** 2, axis=1) <= bound * (1 + 1e-12))


@pytest.mark.parametrize("T,D", [(1, 2), (2, 2), (4, 2), (1, 4), (2, 4), (1, 8)])
def test_brute_force_codes(oracle, T, D):
    """With the oracle's scales fixed, its codes minimise the reconstruction
    error in the ORIGINAL basis over all 4^(T*D) code assignments (the
    rotation is orthogonal, so the error separates per element). Uses scipy's
    Hadamard matrix for the reconstruction, independent of the oracle."""
    rng = np.random.default_rng(T * 10 + D)
    Hs = scipy.linalg.hadamard(D) / np.sqrt(D)
    allc = np.array(list(itertools.product(range(4), repeat=T * D)), np.uint8)
    for trial in range(6):
        x = rng.standard_normal((T, D)) * np.exp(rng.standard_normal((T, 1)))
        out = oracle.quantize_block(x, 4 if T > 1 else 2)
        step = out["rp"][:, None] * out["c"][None, :]
        yh = (allc.reshape(-1, T, D) - 1.5) * step[None]
        xh = yh @ Hs                                 # back to the original basis
        err = ((xh - x[None]) ** 2).sum(axis=(1, 2))
        best = np.flatnonzero(err <= err.min() * (1 + 1e-12) + 1e-300)
        assert len(best) == 1, "unexpected tie on random data"
        np.testing.assert_array_equal(allc[best[0]].reshape(T, D), out["codes"])


def test_brute_force_tie_picks_upper(oracle):
    g = keyed("tie_block.txt")
    x = np.array(g["x"])
    out = oracle.quantize_block(x, int(g["iters"][0][0]))
    np.testing.assert_allclose(out["rp"], g["rprime"][0], rtol=0, atol=0)
    np.testing.assert_array_equal(out["u"], np.array(g["u"]))
    np.testing.assert_array_equal(out["codes"], np.array(g["codes"], np.uint8))
    # brute force: the tied elements have two minimisers; the oracle takes the
    # upper one and is a minimiser
    step = out["rp"][:, None] * out["c"][None, :]
    u = np.array(g["u"])[0]
    for j, uj in enumerate(u):
        d = np.abs(LEVELS - uj)
        mins = np.flatnonzero(d == d.min())
        assert out["codes"][0, j] == mins.max()
    assert step.shape == (1, 4)


def _golden_pack():
    for ln in lines("pack_bytes.txt"):
        tok = ln.split()
        chunk, dim, kind = int(tok[1]), int(tok[3]), tok[5]
        rest = " ".join(tok[6:])
        if rest.startswith("codes"):
            cpart, bpart = rest[len("codes"):].split("bytes")
            codes = np.array([[int(v) for v in row.split()]
                              for row in cpart.split("x")], np.uint8)
        else:
            bpart = rest[len("bytes"):]
            t = np.arange(chunk)[:, None]
            j = np.arange(dim)[None, :]
            codes = ((t + 2 * j) % 4).astype(np.uint8)
        yield chunk, dim, (0 if kind == "K" else 1), codes, np.array(
            bpart.split(), np.uint8)


def test_pack_golden_bytes(oracle):
    n = 0
    for chunk, dim, kind, codes, want in _golden_pack():
        got = oracle.pack(codes[None, None], chunk=chunk, kind=kind).reshape(-1)
        np.testing.assert_array_equal(got, want)
        back = oracle.unpack(got.reshape(1, 1, 1, -1), D=dim, chunk=chunk, kind=kind)
        np.testing.assert_array_equal(back[0, 0], codes)
        n += 1
    assert n == 3


@pytest.mark.parametrize("kind", [0, 1])
def test_pack_round_trip(oracle, kind):
    rng = np.random.default_rng(kind)
    codes = rng.integers(0, 4, size=(2, 3, 256, 128), dtype=np.uint8)
    packed = oracle.pack(codes, kind=kind)
    assert packed.shape == (2, 3, 2, 4096)
    np.testing.assert_array_equal(oracle.unpack(packed, kind=kind), codes)


def test_quantize_tensor_equals_blocks(oracle):
    """Chunking (SC-3): a tensor is quantized as independent 128-token blocks."""
    x = kvgen.kv_tensor(0, 0, kvgen.V, 2, 2, 256, 0.5, dtype=kvgen.torch.float32)
    x = x.double().numpy()
    out = oracle.quantize_tensor(x, threads=2)
    for b in range(2):
        for h in range(2):
            for k in range(2):
                blk = oracle.quantize_block(x[b, h, 128 * k:128 * (k + 1)], 4)
                np.testing.assert_array_equal(
                    out["codes"][b, h, 128 * k:128 * (k + 1)], blk["codes"])
                np.testing.assert_array_equal(out["c"][b, h, k], blk["c"])
                np.testing.assert_array_equal(
                    out["rp"][b, h, 128 * k:128 * (k + 1)], blk["rp"])
