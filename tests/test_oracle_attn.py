"""Pins of the oracle's decode attention over the reconstructed cache
(rndamp article on KVarN, "Numbers": both scales enter the dequantization;
reading SC-12: plain softmax attention, scale 1/sqrt(128), grouped-query
heads h -> h // (Hq/Hkv), lengths [0, len))."""
import numpy as np
import pytest
import scipy.linalg
import torch

import kvgen


def _cache(oracle, B, Hkv, T, seed=0, sigma=0.5):
    k = kvgen.kv_tensor(seed, 0, kvgen.K, B, Hkv, T, sigma, dtype=torch.float32)
    v = kvgen.kv_tensor(seed, 0, kvgen.V, B, Hkv, T, sigma, dtype=torch.float32)
    qk = oracle.quantize_tensor(k.double().numpy(), want_u=False)
    qv = oracle.quantize_tensor(v.double().numpy(), want_u=False)
    return qk, qv


def _deq_scipy(codes, rp, c, n, chunk=128):
    """Independent reconstruction with scipy's Hadamard matrix."""
    D = codes.shape[-1]
    cc = np.repeat(c, chunk, axis=0)[:n]
    yh = (codes[:n].astype(float) - 1.5) * rp[:n, None] * cc
    return yh @ (scipy.linalg.hadamard(D) / np.sqrt(D))


def test_dequant_matches_scipy(oracle):
    qk, _ = _cache(oracle, 1, 1, 256)
    for n in (1, 100, 256):
        got = oracle.dequant(qk["codes"][0, 0, :n], qk["rp"][0, 0], qk["c"][0, 0])
        want = _deq_scipy(qk["codes"][0, 0], qk["rp"][0, 0], qk["c"][0, 0], n)
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_attention_matches_torch_sdpa(oracle):
    B, Hkv, Hq, T = 2, 2, 8, 384
    qk, qv = _cache(oracle, B, Hkv, T, seed=3)
    q = kvgen.queries(3, 0, B, Hq, dtype=torch.float32).double().numpy()
    lens = np.array([384, 130], np.int32)
    got = oracle.decode_attn(q, qk["codes"], qk["rp"], qk["c"], qv["codes"],
                             qv["rp"], qv["c"], lens)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            n = lens[b]
            kh = _deq_scipy(qk["codes"][b, h // g], qk["rp"][b, h // g],
                            qk["c"][b, h // g], n)
            vh = _deq_scipy(qv["codes"][b, h // g], qv["rp"][b, h // g],
                            qv["c"][b, h // g], n)
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h])[None, None, None],
                torch.from_numpy(kh)[None, None], torch.from_numpy(vh)[None, None])
            np.testing.assert_allclose(got[b, h], o.numpy().reshape(-1),
                                       rtol=1e-10, atol=1e-12)


def test_rotated_domain_scores(oracle):
    """q . Xhat_t equals (H q / sqrt D) . Yhat_t (orthogonality): the identity
    that lets a kernel fold the rotation into q and the output."""
    qk, _ = _cache(oracle, 1, 1, 128, seed=4)
    q = np.random.default_rng(0).standard_normal(128)
    xh = oracle.dequant(qk["codes"][0, 0], qk["rp"][0, 0], qk["c"][0, 0])
    yh = (qk["codes"][0, 0] - 1.5) * qk["rp"][0, 0][:, None] * qk["c"][0, 0, 0][None]
    np.testing.assert_allclose(xh @ q, yh @ oracle.rotate(q[None])[0], rtol=1e-11,
                               atol=1e-11)


def test_special_cases(oracle):
    B, Hkv, Hq, T = 1, 1, 4, 128
    qk, qv = _cache(oracle, B, Hkv, T, seed=5)
    q = kvgen.queries(5, 0, B, Hq, dtype=torch.float32).double().numpy()
    args = (qk["codes"], qk["rp"], qk["c"], qv["codes"], qv["rp"], qv["c"])
    # a one-token cache returns that token's reconstructed V
    o1 = oracle.decode_attn(q, *args, lens=[1])
    v0 = oracle.dequant(qv["codes"][0, 0, :1], qv["rp"][0, 0], qv["c"][0, 0])[0]
    for h in range(Hq):
        np.testing.assert_allclose(o1[0, h], v0, rtol=1e-12, atol=1e-12)
    # length 0 (and length > capacity) give zero rows
    assert np.all(oracle.decode_attn(q, *args, lens=[0]) == 0)
    assert np.all(oracle.decode_attn(q, *args, lens=[T + 1]) == 0)
    # identical K rows -> uniform weights -> the mean of the V rows
    kc = qk["codes"].copy()
    kc[0, 0, :] = kc[0, 0, 0]
    krp = qk["rp"].copy()
    krp[0, 0, :] = krp[0, 0, 0]
    o = oracle.decode_attn(q, kc, krp, qk["c"], qv["codes"], qv["rp"], qv["c"],
                           lens=[T])
    vh = oracle.dequant(qv["codes"][0, 0], qv["rp"][0, 0], qv["c"][0, 0])
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], vh.mean(axis=0), rtol=1e-11, atol=1e-12)


def test_softmax_split_merge(oracle):
    """Splitting the tokens and merging the partial results by log-sum-exp
    (the flash-decoding recombination) reproduces the unsplit result."""
    qk, qv = _cache(oracle, 1, 1, 512, seed=6)
    q = kvgen.queries(6, 0, 1, 4, dtype=torch.float32).double().numpy()
    kh = oracle.dequant(qk["codes"][0, 0], qk["rp"][0, 0], qk["c"][0, 0])
    vh = oracle.dequant(qv["codes"][0, 0], qv["rp"][0, 0], qv["c"][0, 0])
    full = oracle.decode_attn(q, qk["codes"], qk["rp"], qk["c"], qv["codes"],
                              qv["rp"], qv["c"], lens=[512])
    for h in range(4):
        s = kh @ q[0, h] / np.sqrt(128)
        parts = []
        for lo, hi in ((0, 100), (100, 333), (333, 512)):
            m = s[lo:hi].max()
            p = np.exp(s[lo:hi] - m)
            parts.append((m, p.sum(), p @ vh[lo:hi]))
        M = max(p[0] for p in parts)
        num = sum(np.exp(m - M) * acc for m, _, acc in parts)
        den = sum(np.exp(m - M) * l for m, l, _ in parts)
        np.testing.assert_allclose(num / den, full[0, h], rtol=1e-12, atol=1e-13)


def test_gqa_head_mapping(oracle):
    """Query head h reads kv-head h // (Hq/Hkv): permuting kv-heads permutes
    the output groups."""
    qk, qv = _cache(oracle, 1, 2, 128, seed=7)
    q = kvgen.queries(7, 0, 1, 8, dtype=torch.float32).double().numpy()
    o = oracle.decode_attn(q, qk["codes"], qk["rp"], qk["c"], qv["codes"],
                           qv["rp"], qv["c"], lens=[128])
    sw = [a[:, ::-1].copy() for a in (qk["codes"], qk["rp"], qk["c"], qv["codes"],
                                      qv["rp"], qv["c"])]
    q2 = np.concatenate([q[:, 4:], q[:, :4]], axis=1)
    o2 = oracle.decode_attn(q2, *sw, lens=[128])
    np.testing.assert_allclose(o2[:, :4], o[:, 4:], rtol=1e-13)
    np.testing.assert_allclose(o2[:, 4:], o[:, :4], rtol=1e-13)
