"""GPU parity of the flag variants of the C ABI against the oracle:
KVARN_FLAG_NO_ROTATE (rotation absorbed into the model's weights: the caller
passes rotated K/V/q and receives the rotated output) and KVARN_FLAG_ONE_SCALE
(decode with the column scales taken as 1, the ablation of the second scale).
"""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import ATTN_RL2, SCALE_RTOL, assert_quant_parity, log, rel_l2

pytestmark = pytest.mark.gpu


def _rotated(oracle, x):
    """x . H_128 / sqrt(128) computed by the oracle in fp64, rounded to fp32."""
    return torch.from_numpy(oracle.rotate(x.double().cpu().numpy())).float()


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_quantize_no_rotate(kvarn, oracle, kind):
    """Quantizing pre-rotated input with the rotation skipped matches the
    oracle's quantizer of the unrotated input."""
    x = kvgen.kv_tensor(41, 0, kind, 2, 3, 384, 0.5, dtype=torch.float32)
    xr = _rotated(oracle, x).cuda()
    cache = kvarn.Cache.empty(2, 3, 384, kind, device="cuda")
    kvarn.quantize(xr, cache, flags=kvarn.FLAG_NO_ROTATE)
    torch.cuda.synchronize()
    ora = oracle.quantize_tensor(x.double().numpy())
    g = oracle.unpack(cache.codes.cpu().numpy(), kind=kind)
    st = assert_quant_parity(oracle, ora, g, cache.row_scale.cpu().numpy(),
                             cache.col_scale.cpu().numpy(), "no-rotate")
    log(f"[test] quantize no-rotate kind={kind}: {st}")


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_append_no_rotate(kvarn, oracle, kind):
    """Appending a pre-rotated token with the rotation skipped matches the
    oracle's append of the unrotated token (opening chunk 1 and inside it)."""
    B, H, cap = 2, 2, 256
    ck, rk, colk = kvgen.random_cache(42 + kind, B, H, cap)
    cache = kvarn.Cache(ck.cuda(), rk.cuda(), colk.cuda(), kind)
    codes = oracle.unpack(ck.numpy(), kind=kind)
    rp, c = rk.double().numpy().copy(), colk.double().numpy().copy()
    for step, p in enumerate((128, 129, 133)):
        x = kvgen.new_tokens(43, 0, kind, B, H, 0.5, step=step, dtype=torch.float32)
        pos = torch.full((B,), p, dtype=torch.int32)
        kvarn.append(_rotated(oracle, x).cuda(), pos.cuda(), cache, flags=kvarn.FLAG_NO_ROTATE)
        oracle.append(x.double().numpy(), pos.numpy(), codes, rp, c)
    torch.cuda.synchronize()
    g = oracle.unpack(cache.codes.cpu().numpy(), kind=kind)
    np.testing.assert_allclose(cache.row_scale.cpu().numpy()[:, :, 128:134],
                               rp[:, :, 128:134], rtol=SCALE_RTOL, atol=0)
    np.testing.assert_allclose(cache.col_scale.cpu().numpy(), c, rtol=SCALE_RTOL, atol=0)
    # codes away from rounding boundaries (u of the appended tokens in fp64)
    mism = g != codes
    for p in (128, 129, 133):
        for b in range(B):
            for h in range(H):
                if mism[b, h, p].any():
                    y = oracle.rotate(kvgen.new_tokens(
                        43, 0, kind, B, H, 0.5, step=(128, 129, 133).index(p),
                        dtype=torch.float32)[b, h].double().numpy())
                    u = y / (rp[b, h, p] * c[b, h, 1])
                    assert oracle.boundary_mask(u)[mism[b, h, p]].all()
    mism[:, :, [128, 129, 133]] = False
    if kind == kvgen.V:
        # the token at 128 starts a byte: its later slots were written fresh
        # (code 0) and only 129 has been appended since
        assert np.all(g[:, :, [130, 131]] == 0)
        mism[:, :, [130, 131]] = False
    assert not mism.any()


def _rotated_bf16(oracle, x):
    """x . H_128 / sqrt(128) in fp64, rounded to bf16: what a model with the
    rotation absorbed into its weights hands over. Returned with the oracle
    input that reproduces exactly those values: the scaled rotation is its
    own inverse, so rotate(xr) rotated again is xr up to fp64 rounding."""
    xr = torch.from_numpy(oracle.rotate(x.double().cpu().numpy())).to(torch.bfloat16)
    return xr, oracle.rotate(xr.double().numpy())


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
@pytest.mark.parametrize("iters", [4, 0])
def test_quantize_no_rotate_bf16(kvarn, oracle, kind, iters):
    """bf16 pre-rotated K/V with the rotation skipped (the identity-tile MFMAs
    and the first row step without the factor 128) against the oracle fed the
    exact values the GPU read."""
    x = kvgen.kv_tensor(51, 0, kind, 2, 3, 384, 0.5, dtype=torch.float32)
    xr, x_eq = _rotated_bf16(oracle, x)
    cache = kvarn.Cache.empty(2, 3, 384, kind, device="cuda")
    kvarn.quantize(xr.cuda(), cache, iters=iters, flags=kvarn.FLAG_NO_ROTATE)
    torch.cuda.synchronize()
    ora = oracle.quantize_tensor(x_eq, iters=iters)
    g = oracle.unpack(cache.codes.cpu().numpy(), kind=kind)
    st = assert_quant_parity(oracle, ora, g, cache.row_scale.cpu().numpy(),
                             cache.col_scale.cpu().numpy(), "no-rotate bf16")
    log(f"[test] quantize no-rotate bf16 kind={kind} iters={iters}: {st}")


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_append_no_rotate_bf16(kvarn, oracle, kind):
    """bf16 pre-rotated tokens appended with the rotation skipped: opening
    chunk 1 (column scales copied from chunk 0) and inside it."""
    B, H, cap = 2, 2, 256
    ck, rk, colk = kvgen.random_cache(52 + kind, B, H, cap)
    cache = kvarn.Cache(ck.cuda(), rk.cuda(), colk.cuda(), kind)
    codes = oracle.unpack(ck.numpy(), kind=kind)
    rp, c = rk.double().numpy().copy(), colk.double().numpy().copy()
    ys = {}
    for step, p in enumerate((128, 129, 133)):
        x = kvgen.new_tokens(53, 0, kind, B, H, 0.5, step=step, dtype=torch.float32)
        xr, x_eq = _rotated_bf16(oracle, x)
        ys[p] = xr.double().numpy()
        pos = torch.full((B,), p, dtype=torch.int32)
        kvarn.append(xr.cuda(), pos.cuda(), cache, flags=kvarn.FLAG_NO_ROTATE)
        oracle.append(x_eq, pos.numpy(), codes, rp, c)
    torch.cuda.synchronize()
    g = oracle.unpack(cache.codes.cpu().numpy(), kind=kind)
    np.testing.assert_allclose(cache.row_scale.cpu().numpy()[:, :, 128:134],
                               rp[:, :, 128:134], rtol=SCALE_RTOL, atol=0)
    np.testing.assert_allclose(cache.col_scale.cpu().numpy(), c, rtol=SCALE_RTOL, atol=0)
    mism = g != codes
    for p in (128, 129, 133):
        for b in range(B):
            for h in range(H):
                if mism[b, h, p].any():
                    u = ys[p][b, h] / (rp[b, h, p] * c[b, h, 1])
                    assert oracle.boundary_mask(u)[mism[b, h, p]].all()
    mism[:, :, [128, 129, 133]] = False
    if kind == kvgen.V:
        assert np.all(g[:, :, [130, 131]] == 0)
        mism[:, :, [130, 131]] = False
    assert not mism.any()


def _random_caches(kv, B, Hkv, cap, seed):
    ck, rk, colk = kvgen.random_cache(seed, B, Hkv, cap)
    cv, rv, colv = kvgen.random_cache(seed + 1000, B, Hkv, cap)
    return (kv.Cache(ck.cuda(), rk.cuda(), colk.cuda(), kv.K),
            kv.Cache(cv.cuda(), rv.cuda(), colv.cuda(), kv.V), (ck, rk, colk), (cv, rv, colv))


def _oracle_decode(oracle, q, hk, hv, lens, ones_c=False):
    ck, rk, colk = hk
    cv, rv, colv = hv
    ck_c = np.ones_like(colk.double().numpy()) if ones_c else colk.double().numpy()
    cv_c = np.ones_like(colv.double().numpy()) if ones_c else colv.double().numpy()
    return oracle.decode_attn(q.double().cpu().numpy(), oracle.unpack(ck.numpy(), kind=0),
                              rk.double().numpy(), ck_c, oracle.unpack(cv.numpy(), kind=1),
                              rv.double().numpy(), cv_c, lens)


def test_decode_no_rotate(kvarn, oracle):
    """Rotated query in, rotated output out: rotating the output back gives
    the oracle's attention on the same cache."""
    B, Hkv, G, cap = 2, 2, 4, 512
    kc, vc, hk, hv = _random_caches(kvarn, B, Hkv, cap, seed=44)
    q = kvgen.queries(45, 0, B, Hkv * G, dtype=torch.float32)
    lens = [512, 300]
    out_r = kvarn.decode_attn(_rotated(oracle, q).cuda(), kc, vc,
                              torch.tensor(lens, dtype=torch.int32).cuda(),
                              flags=kvarn.FLAG_NO_ROTATE)
    torch.cuda.synchronize()
    got = oracle.rotate(out_r.double().cpu().numpy())
    err = rel_l2(got, _oracle_decode(oracle, q, hk, hv, lens))
    log(f"[test] decode no-rotate: rel L2 {err:.3e}")
    assert err <= ATTN_RL2


@pytest.mark.parametrize("G", [4, 8])
def test_decode_one_scale(kvarn, oracle, G):
    """Column scales taken as 1: matches the oracle fed c = 1."""
    B, Hkv, cap = 2, 2, 512
    kc, vc, hk, hv = _random_caches(kvarn, B, Hkv, cap, seed=46)
    q = kvgen.queries(47, 0, B, Hkv * G, dtype=torch.bfloat16)
    lens = [512, 129]
    out = kvarn.decode_attn(q.cuda(), kc, vc, torch.tensor(lens, dtype=torch.int32).cuda(),
                            flags=kvarn.FLAG_ONE_SCALE)
    torch.cuda.synchronize()
    err = rel_l2(out.cpu().numpy(), _oracle_decode(oracle, q, hk, hv, lens, ones_c=True))
    log(f"[test] decode one-scale G={G}: rel L2 {err:.3e}")
    assert err <= ATTN_RL2


def test_one_scale_equals_two_scales_when_c_is_one(kvarn):
    """On a cache quantized with iters = 0 every column scale is exactly 1:
    the one-scale kernel and the two-scale kernel give identical outputs."""
    B, Hkv, T = 2, 2, 1024
    caches = []
    for kind in (kvgen.K, kvgen.V):
        x = kvgen.kv_tensor(48, 0, kind, B, Hkv, T, 0.5, device="cuda")
        c = kvarn.Cache.empty(B, Hkv, T, kind, device="cuda")
        kvarn.quantize(x, c, iters=0)
        caches.append(c)
    torch.cuda.synchronize()
    assert torch.all(caches[1].col_scale == 1)
    q = kvgen.queries(49, 0, B, Hkv * 4, device="cuda")
    lens = torch.tensor([1024, 700], dtype=torch.int32, device="cuda")
    a = kvarn.decode_attn(q, caches[0], caches[1], lens)
    b = kvarn.decode_attn(q, caches[0], caches[1], lens, flags=kvarn.FLAG_ONE_SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
