"""GPU parity of the per-token magnitude/direction diagnostic
(kvarn_token_error) against the oracle's definition, on caches written by the
device quantizer (with and without balancing), on random caches over ragged
token ranges, with the rotation absorbed, and on zero tokens."""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import log

pytestmark = pytest.mark.gpu

RATIO_RTOL = 1e-5   # fp32 sums of 128 squares against fp64
COS_ATOL = 1e-5


def _oracle_errors(oracle, x, cache, kind, token_offset, tokens):
    """x [B,H,tokens,128] (host fp64) against the cache's slots
    [token_offset, token_offset + tokens), per (b, h) through the oracle."""
    codes = oracle.unpack(cache.codes.cpu().numpy(), kind=kind)
    rp = cache.row_scale.double().cpu().numpy()
    c = cache.col_scale.double().cpu().numpy()
    B, H = x.shape[:2]
    ratio = np.empty((B, H, tokens))
    cosine = np.empty((B, H, tokens))
    sl = slice(token_offset, token_offset + tokens)
    for b in range(B):
        for h in range(H):
            xh = oracle.dequant(codes[b, h], rp[b, h], c[b, h])[sl]
            ratio[b, h], cosine[b, h] = oracle.token_error(x[b, h], xh)
    return ratio, cosine


def _compare(got, want, what):
    gr, gc = (t.double().cpu().numpy() for t in got)
    wr, wc = want
    np.testing.assert_allclose(gr, wr, rtol=RATIO_RTOL, atol=0, err_msg=f"{what}: ratio")
    np.testing.assert_allclose(gc, wc, rtol=0, atol=COS_ATOL, err_msg=f"{what}: cosine")
    log(f"[test] {what}: ratio mean {gr.mean():.4f}, cos mean {gc.mean():.5f}, "
        f"max |d ratio| {np.abs(gr - wr).max():.2e}, max |d cos| {np.abs(gc - wc).max():.2e}")


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
@pytest.mark.parametrize("iters", [0, 4])
def test_after_quantize(kvarn, oracle, kind, iters):
    B, H, T = 2, 3, 384
    x = kvgen.kv_tensor(51, 0, kind, B, H, T, 0.5, dtype=torch.bfloat16, device="cuda")
    cache = kvarn.Cache.empty(B, H, T, kind, device="cuda")
    kvarn.quantize(x, cache, iters=iters)
    got = kvarn.token_error(x, cache)
    torch.cuda.synchronize()
    want = _oracle_errors(oracle, x.double().cpu().numpy(), cache, kind, 0, T)
    _compare(got, want, f"quantize iters={iters} kind={kind}")


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_random_cache_ragged_range(kvarn, oracle, kind):
    """A random cache and fp32 input over slots [77, 77 + 301): token ranges
    neither chunk- nor byte-aligned, and a strided x (a slice of a larger
    tensor)."""
    B, H, cap = 2, 2, 512
    ck, rk, colk = kvgen.random_cache(52 + kind, B, H, cap)
    cache = kvarn.Cache(ck.cuda(), rk.cuda(), colk.cuda(), kind)
    big = torch.randn(B, H, 320, 128, generator=torch.Generator().manual_seed(53),
                      dtype=torch.float32)
    x = big.cuda()[:, :, 5:306]
    assert not x.is_contiguous() and x.stride(2) == 128
    got = kvarn.token_error(x, cache, token_offset=77)
    torch.cuda.synchronize()
    want = _oracle_errors(oracle, x.double().cpu().numpy(), cache, kind, 77, 301)
    _compare(got, want, f"random cache kind={kind}")


def test_no_rotate(kvarn, oracle):
    """Rotated input with the rotation absorbed gives the same numbers as the
    unrotated input (the rotation preserves norms and inner products)."""
    B, H, T = 2, 2, 256
    x = kvgen.kv_tensor(54, 0, kvgen.K, B, H, T, 0.5, dtype=torch.float32)
    xr = torch.from_numpy(oracle.rotate(x.double().numpy())).float().cuda()
    cache = kvarn.Cache.empty(B, H, T, kvgen.K, device="cuda")
    kvarn.quantize(x.cuda(), cache)
    a = kvarn.token_error(x.cuda(), cache)
    b = kvarn.token_error(xr, cache, flags=kvarn.FLAG_NO_ROTATE)
    torch.cuda.synchronize()
    np.testing.assert_allclose(b[0].cpu().numpy(), a[0].cpu().numpy(), rtol=1e-5)
    np.testing.assert_allclose(b[1].cpu().numpy(), a[1].cpu().numpy(), atol=1e-5)
    want = _oracle_errors(oracle, x.double().numpy(), cache, kvgen.K, 0, T)
    _compare(b, want, "no-rotate")


def test_zero_tokens(kvarn):
    """Zero tokens quantize to r' = 0 (SC-9): both norms are zero -> (1, 1);
    a zero token against a nonzero cache row -> (+inf, 0)."""
    B, H, T = 1, 2, 128
    x = torch.zeros(B, H, T, 128, dtype=torch.bfloat16, device="cuda")
    x[0, 1, 5:] = 1.0
    cache = kvarn.Cache.empty(B, H, T, kvgen.K, device="cuda")
    kvarn.quantize(x, cache)
    r, c = kvarn.token_error(x, cache)
    torch.cuda.synchronize()
    assert torch.all(r[0, 0] == 1) and torch.all(c[0, 0] == 1)
    assert torch.all(r[0, 1, :5] == 1) and torch.all(c[0, 1, :5] == 1)
    x2 = x.clone()
    x2[0, 1, 7] = 0.0
    r2, c2 = kvarn.token_error(x2, cache)
    torch.cuda.synchronize()
    assert torch.isinf(r2[0, 1, 7]) and c2[0, 1, 7] == 0


def test_appended_tokens(kvarn, oracle):
    """The error of tokens written by the append path (frozen column scales,
    SC-11) is read the same way; the oracle recomputes it from the cache."""
    B, H, T = 2, 2, 256
    cap = T + 128
    x = kvgen.kv_tensor(55, 0, kvgen.K, B, H, T, 0.5, dtype=torch.float32, device="cuda")
    cache = kvarn.Cache.empty(B, H, cap, kvgen.K, device="cuda")
    kvarn.quantize(x, cache)
    news = []
    for step in range(3):
        xn = kvgen.new_tokens(55, 0, kvgen.K, B, H, 0.5, step=step, dtype=torch.float32,
                              device="cuda")
        kvarn.append(xn, torch.full((B,), T + step, dtype=torch.int32, device="cuda"), cache)
        news.append(xn)
    xa = torch.stack(news, dim=2).contiguous()
    got = kvarn.token_error(xa, cache, token_offset=T)
    torch.cuda.synchronize()
    want = _oracle_errors(oracle, xa.double().cpu().numpy(), cache, kvgen.K, T, 3)
    _compare(got, want, "appended tokens")
