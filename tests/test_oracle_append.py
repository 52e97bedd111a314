"""Pins of the oracle's one-token append (rndamp article on KVarN, "The
Problem": the cache grows one token per decoding step and errors carry into
later steps). Reading SC-11: the token is coded at once against its chunk's
column scales; a token that opens a chunk copies the previous chunk's column
scales (or 1 for the first chunk); its row scale is its own range step."""
import numpy as np
import scipy.linalg
import torch

import kvgen


def test_append_closed_form(oracle):
    B, H, D, cap = 2, 3, 128, 384
    codes = np.zeros((B, H, cap, D), np.uint8)
    rp = np.zeros((B, H, cap))
    c = np.zeros((B, H, cap // 128, D))
    rng = np.random.default_rng(0)
    c[:, :, 0] = np.exp(0.3 * rng.standard_normal((B, H, D)))
    x = kvgen.new_tokens(0, 0, kvgen.K, B, H, 0.5, dtype=torch.float32).double().numpy()
    pos = np.array([5, 77])
    u = oracle.append(x, pos, codes, rp, c)
    Hs = scipy.linalg.hadamard(D) / np.sqrt(D)
    for b in range(B):
        for h in range(H):
            y = x[b, h] @ Hs
            m = np.max(np.abs(y / c[b, h, 0]))
            assert rp[b, h, pos[b]] == np.float64(m / 2) or np.isclose(
                rp[b, h, pos[b]], m / 2, rtol=1e-14)
            want_u = y / (m / 2 * c[b, h, 0])
            np.testing.assert_allclose(u[b, h], want_u, rtol=1e-12, atol=1e-14)
            want = np.clip(np.floor(want_u + 2), 0, 3)
            ok = np.min(np.abs(want_u[:, None] - [-1, 0, 1]), axis=1) > 1e-9
            np.testing.assert_array_equal(codes[b, h, pos[b]][ok], want[ok])
            assert np.all(np.abs(codes[b, h, pos[b]] - 1.5 - u[b, h]) <= 0.5 + 1e-12)
    # untouched slots stay zero
    assert rp[0, :, 6:].sum() == 0 and codes[1, :, :77].sum() == 0


def test_append_opens_chunk(oracle):
    B, H, D, cap = 1, 2, 128, 384
    codes = np.zeros((B, H, cap, D), np.uint8)
    rp = np.zeros((B, H, cap))
    c = np.full((B, H, cap // 128, D), -7.0)      # sentinel: must be overwritten
    x = kvgen.new_tokens(1, 0, kvgen.V, B, H, 0.5, dtype=torch.float32).double().numpy()
    oracle.append(x, [0], codes, rp, c)
    np.testing.assert_array_equal(c[0, :, 0], 1.0)   # first chunk: c = 1
    c[0, :, 0] = np.linspace(0.5, 2.0, D)
    oracle.append(x, [128], codes, rp, c)
    np.testing.assert_array_equal(c[0, :, 1], c[0, :, 0])   # copied forward
    np.testing.assert_array_equal(c[0, :, 2], -7.0)          # later chunk untouched
    # a position outside [0, cap) is skipped
    before = codes.copy()
    oracle.append(x, [cap], codes, rp, c)
    np.testing.assert_array_equal(codes, before)


def test_append_equals_block_quantizer_with_fixed_c(oracle):
    """Appending every token of a chunk one by one with the chunk's c preset
    gives the same codes and row scales as the block quantizer, whose c the
    appends reuse (the block quantizer's codes depend on r only through c)."""
    x = kvgen.kv_tensor(2, 0, kvgen.K, 1, 1, 128, 0.5, dtype=torch.float32)
    x = x.double().numpy()
    blk = oracle.quantize_block(x[0, 0], 4)
    codes = np.zeros((1, 1, 256, 128), np.uint8)
    rp = np.zeros((1, 1, 256))
    c = np.zeros((1, 1, 2, 128))
    c[0, 0, 0] = blk["c"]
    for t in range(1, 128):
        oracle.append(x[:, :, t], [t], codes, rp, c)
    ok = ~oracle.boundary_mask(blk["u"][1:], 1e-9)
    np.testing.assert_array_equal(codes[0, 0, 1:128][ok], blk["codes"][1:][ok])
    np.testing.assert_allclose(rp[0, 0, 1:128], blk["rp"][1:], rtol=1e-13)
