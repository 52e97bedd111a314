"""GPU parity for head sizes 64 and 256 (the Hadamard transform on the channel
dimension of other model families; rndamp article on KVarN, "How It Works",
item 1): quantize, append, append with re-balancing at chunk close, decode
attention, the per-token error and the allocation-free decode, each against
the oracle (which takes any power-of-two head size) at the bars of
gpu_util."""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import (ATTN_RL2, SCALE_RTOL, assert_quant_parity, cache_blocks, log, rel_l2,
                      sample_blocks, x_blocks)

pytestmark = pytest.mark.gpu

DIMS = [64, 256]


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
@pytest.mark.parametrize("dtype,iters", [(torch.bfloat16, 4), (torch.float32, 4),
                                         (torch.bfloat16, 0), (torch.float32, 7)])
def test_quantize_headdim(kvarn, oracle, D, kind, dtype, iters):
    B, H, T = 2, 3, 384
    x = kvgen.kv_tensor(81 + D, 0, kind, B, H, T, 0.5, dtype=dtype, head_dim=D)
    x[0, 1, 5] = 0  # a zero token
    cache = kvarn.Cache.empty(B, H, T + 128, kind, device="cuda", head_dim=D)
    kvarn.quantize(x.cuda(), cache, token_offset=128, iters=iters)
    torch.cuda.synchronize()
    ora = oracle.quantize_tensor(x.double().numpy(), iters=iters)
    g = oracle.unpack(cache.codes.cpu().numpy(), D=D, kind=kind)[:, :, 128:]
    st = assert_quant_parity(oracle, ora, g, cache.row_scale.cpu().numpy()[:, :, 128:],
                             cache.col_scale.cpu().numpy()[:, :, 1:], f"D={D}")
    assert np.all(cache.codes.cpu().numpy()[:, :, 0] == 0)  # chunk 0 untouched
    log(f"[test] quantize D={D} kind={kind} {dtype} iters={iters}: {st}")


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_quantize_headdim_many_blocks(kvarn, oracle, D, kind):
    """A launch of 2048 blocks (4 sequences x 8 kv-heads x 64 chunks, bf16):
    every resident workgroup walks several blocks, so the two-deep prefetch,
    the LDS input slice and the alternating V staging buffers all take part.
    Sampled blocks, the first and the last, against the oracle."""
    B, H, T = 4, 8, 8192
    x = kvgen.kv_tensor(31 + D, 0, kind, B, H, T, 0.5, device="cuda", head_dim=D)
    cache = kvarn.Cache.empty(B, H, T, kind, device="cuda", head_dim=D)
    kvarn.quantize(x, cache)
    torch.cuda.synchronize()
    sel = sample_blocks(np.random.default_rng(D + kind), B, H, T // 128, 48,
                        always=[(0, 0, 0), (B - 1, H - 1, T // 128 - 1)])
    ora = oracle.quantize_tensor(x_blocks(x, sel), threads=8)
    st = assert_quant_parity(oracle, ora, *cache_blocks(cache, kind, sel), f"many blocks D={D}")
    log(f"[test] quantize D={D} kind={kind} 2048 blocks, {len(sel)} sampled: {st}")


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_quantize_headdim_strided_offset(kvarn, oracle, D, kind):
    """x a strided view (token stride 2 D elements) written at token offset
    256 of a larger cache; the slots before and after stay untouched."""
    base = kvgen.kv_tensor(111 + D, 0, kind, 2, 3, 256, 0.5, dtype=torch.bfloat16,
                           device="cuda", head_dim=D)
    big = torch.zeros((2, 3, 256, 2 * D), dtype=torch.bfloat16, device="cuda")
    big[..., D // 2:D // 2 + D] = base
    x = big[..., D // 2:D // 2 + D]
    assert x.stride(2) == 2 * D
    cache = kvarn.Cache.empty(2, 3, 640, kind, device="cuda", head_dim=D)
    kvarn.quantize(x, cache, token_offset=256, iters=4)
    torch.cuda.synchronize()
    ora = oracle.quantize_tensor(base.double().cpu().numpy())
    g = oracle.unpack(cache.codes.cpu().numpy(), D=D, kind=kind)
    assert_quant_parity(oracle, ora, g[:, :, 256:512], cache.row_scale[:, :, 256:512].cpu(),
                        cache.col_scale[:, :, 2:4].cpu(), f"strided D={D}")
    assert cache.codes[:, :, :2].count_nonzero() == 0
    assert cache.codes[:, :, 4:].count_nonzero() == 0
    assert cache.row_scale[:, :, :256].count_nonzero() == 0
    assert cache.col_scale[:, :, 4:].count_nonzero() == 0


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_quantize_headdim_no_rotate(kvarn, oracle, D, kind):
    """bf16 pre-rotated input with the rotation skipped, against the oracle fed
    the exact values the GPU read (the scaled rotation is its own inverse)."""
    x = kvgen.kv_tensor(91, 0, kind, 2, 2, 256, 0.5, dtype=torch.float32, head_dim=D)
    xr = torch.from_numpy(oracle.rotate(x.double().numpy())).to(torch.bfloat16)
    cache = kvarn.Cache.empty(2, 2, 256, kind, device="cuda", head_dim=D)
    kvarn.quantize(xr.cuda(), cache, flags=kvarn.FLAG_NO_ROTATE)
    torch.cuda.synchronize()
    ora = oracle.quantize_tensor(oracle.rotate(xr.double().numpy()))
    g = oracle.unpack(cache.codes.cpu().numpy(), D=D, kind=kind)
    assert_quant_parity(oracle, ora, g, cache.row_scale.cpu().numpy(),
                        cache.col_scale.cpu().numpy(), f"D={D} no-rotate")


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_append_headdim(kvarn, oracle, D, kind, dtype):
    """Tokens appended into a random cache: chunk 1 opened (column scales
    copied from chunk 0), then further slots, one skipped sequence."""
    B, H, cap = 3, 2, 256
    ck, rk, colk = kvgen.random_cache(93 + kind, B, H, cap, head_dim=D)
    cache = kvarn.Cache(ck.cuda(), rk.cuda(), colk.cuda(), kind)
    codes = oracle.unpack(ck.numpy(), D=D, kind=kind)
    rp, c = rk.double().numpy().copy(), colk.double().numpy().copy()
    us = {}
    for step, p in enumerate((128, 129, 130, 133)):
        x = kvgen.new_tokens(94, 0, kind, B, H, 0.5, step=step, dtype=dtype, head_dim=D)
        pos = np.array([p, p, -1], np.int32)
        kvarn.append(x.cuda(), torch.from_numpy(pos).cuda(), cache)
        us[p] = oracle.append(x.double().numpy(), pos, codes, rp, c)
    torch.cuda.synchronize()
    g = oracle.unpack(cache.codes.cpu().numpy(), D=D, kind=kind)
    np.testing.assert_allclose(cache.row_scale.cpu().numpy(), rp, rtol=SCALE_RTOL, atol=0)
    np.testing.assert_allclose(cache.col_scale.cpu().numpy(), c, rtol=SCALE_RTOL, atol=0)
    mism = g != codes
    for p, u in us.items():
        for b in range(2):
            assert oracle.boundary_mask(u[b])[mism[b, :, p]].all()
        mism[:2, :, p] = False
    if kind == kvgen.V:
        # the token at 128 starts a byte: its later slot 131 was written fresh
        assert np.all(g[:2, :, 131] == 0)
        mism[:2, :, 131] = False
    assert not mism.any()


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_append_rebalance_headdim(kvarn, oracle, D, kind):
    """A chunk filled token by token and re-quantized at its close equals the
    oracle's block quantization of the appended tokens."""
    B, H, cap = 2, 2, 256
    cache = kvarn.Cache.empty(B, H, cap, kind, device="cuda", head_dim=D)
    window = kvarn.append_window(B, H, dtype=torch.bfloat16, head_dim=D)
    hist = []
    for step in range(130):
        x = kvgen.new_tokens(95, 0, kind, B, H, 0.5, step=step, head_dim=D, device="cuda")
        hist.append(x.double().cpu().numpy())
        pos = torch.full((B,), step, dtype=torch.int32, device="cuda")
        kvarn.append_rebalance(x, pos, cache, window)
    torch.cuda.synchronize()
    xs = np.stack(hist[:128], axis=2)  # [B, H, 128, D]
    ora = oracle.quantize_tensor(xs)
    g = oracle.unpack(cache.codes.cpu().numpy(), D=D, kind=kind)
    assert_quant_parity(oracle, ora, g[:, :, :128], cache.row_scale.cpu().numpy()[:, :, :128],
                        cache.col_scale.cpu().numpy()[:, :, :1], f"rebalance D={D}")
    # the next chunk opened with the re-balanced column scales
    np.testing.assert_allclose(cache.col_scale.cpu().numpy()[:, :, 1], ora["c"][:, :, 0],
                               rtol=SCALE_RTOL, atol=0)


def _caches(kv, B, Hkv, cap, D, seed):
    ck, rk, colk = kvgen.random_cache(seed, B, Hkv, cap, head_dim=D)
    cv, rv, colv = kvgen.random_cache(seed + 1000, B, Hkv, cap, head_dim=D)
    return (kv.Cache(ck.cuda(), rk.cuda(), colk.cuda(), kv.K),
            kv.Cache(cv.cuda(), rv.cuda(), colv.cuda(), kv.V), (ck, rk, colk), (cv, rv, colv))


def _oracle_decode(oracle, q, hk, hv, lens, D, ones_c=False):
    ck, rk, colk = hk
    cv, rv, colv = hv
    kc_ = np.ones_like(colk.double().numpy()) if ones_c else colk.double().numpy()
    vc_ = np.ones_like(colv.double().numpy()) if ones_c else colv.double().numpy()
    return oracle.decode_attn(q.double().cpu().numpy(), oracle.unpack(ck.numpy(), D=D, kind=0),
                              rk.double().numpy(), kc_, oracle.unpack(cv.numpy(), D=D, kind=1),
                              rv.double().numpy(), vc_, lens)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("B,Hkv,G,cap,lens,n_split", [
    (2, 2, 4, 512, [512, 300], 0),
    (3, 1, 1, 384, [1, 129, 384], 0),
    (1, 2, 8, 256, [200], 0),
    (2, 3, 3, 640, [640, 255], 1),
    (2, 2, 4, 2560, [2560, 700], 20),  # five workgroups per row: the last one merges
    (1, 4, 2, 1280, [1153], 0),
    (2, 2, 4, 4224, [4097, 3000], 48),  # twelve workgroups per row: one merge round (two at D = 256)
])
def test_decode_headdim(kvarn, oracle, D, B, Hkv, G, cap, lens, n_split):
    kc, vc, hk, hv = _caches(kvarn, B, Hkv, cap, D, seed=97 + B + G)
    q = kvgen.queries(98, 0, B, Hkv * G, dtype=torch.bfloat16, head_dim=D)
    L = torch.tensor(lens, dtype=torch.int32).cuda()
    out = kvarn.decode_attn(q.cuda(), kc, vc, L, n_split=n_split)
    torch.cuda.synchronize()
    err = rel_l2(out.cpu().numpy(), _oracle_decode(oracle, q, hk, hv, lens, D))
    log(f"[test] decode D={D} B={B} Hkv={Hkv} G={G} cap={cap} n_split={n_split}: rel L2 {err:.3e}")
    assert err <= ATTN_RL2


@pytest.mark.parametrize("D", DIMS)
def test_decode_headdim_splits_agree(kvarn, oracle, D):
    """One workgroup per row and 3, 10 and 20 (the last workgroup merging the
    row's partials in one, one and two rounds of 16 at head size 64, in one,
    two and three rounds of 8 at 256) agree with each other up to fp32
    reassociation, and with the oracle, over 80 chunks with a ragged last
    chunk."""
    cap = 80 * 128
    kc, vc, hk, hv = _caches(kvarn, 2, 1, cap, D, seed=123)
    q = kvgen.queries(124, 0, 2, 4, dtype=torch.bfloat16, head_dim=D)
    lens = [cap, cap - 77]
    L = torch.tensor(lens, dtype=torch.int32).cuda()
    outs = [kvarn.decode_attn(q.cuda(), kc, vc, L, n_split=n) for n in (1, 12, 40, 80)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert rel_l2(o.cpu().numpy(), outs[0].cpu().numpy()) < 1e-5
    err = rel_l2(outs[3].cpu().numpy(), _oracle_decode(oracle, q, hk, hv, lens, D))
    log(f"[test] decode D={D} split counts agree; 20 workgroups per row: rel L2 {err:.3e}")
    assert err <= ATTN_RL2


@pytest.mark.parametrize("D", DIMS)
def test_decode_headdim_invalid_lengths_give_zero(kvarn, oracle, D):
    """Lengths 0 and capacity + 1 give zero rows; a valid length beside them
    matches the oracle."""
    kc, vc, hk, hv = _caches(kvarn, 3, 1, 256, D, seed=113)
    q = kvgen.queries(114, 0, 3, 4, dtype=torch.bfloat16, head_dim=D)
    lens = [0, 257, 10]
    out = kvarn.decode_attn(q.cuda(), kc, vc, torch.tensor(lens, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(out[1] == 0)
    want = _oracle_decode(oracle, q[2:3], tuple(t[2:3] for t in hk), tuple(t[2:3] for t in hv),
                          [10], D)
    assert rel_l2(out[2:3].cpu().numpy(), want) <= ATTN_RL2


@pytest.mark.parametrize("D", DIMS)
def test_decode_headdim_flags(kvarn, oracle, D):
    """Absorbed rotation (rotated query in, rotated output out) and the
    one-scale ablation (column scales taken as 1)."""
    B, Hkv, G, cap = 2, 2, 4, 512
    kc, vc, hk, hv = _caches(kvarn, B, Hkv, cap, D, seed=99)
    q = kvgen.queries(100, 0, B, Hkv * G, dtype=torch.float32, head_dim=D)
    lens = [512, 333]
    L = torch.tensor(lens, dtype=torch.int32).cuda()
    qr = torch.from_numpy(oracle.rotate(q.double().numpy())).float().cuda()
    out_r = kvarn.decode_attn(qr, kc, vc, L, flags=kvarn.FLAG_NO_ROTATE)
    out_1 = kvarn.decode_attn(q.cuda(), kc, vc, L, flags=kvarn.FLAG_ONE_SCALE)
    torch.cuda.synchronize()
    e_r = rel_l2(oracle.rotate(out_r.double().cpu().numpy()),
                 _oracle_decode(oracle, q, hk, hv, lens, D))
    e_1 = rel_l2(out_1.cpu().numpy(), _oracle_decode(oracle, q, hk, hv, lens, D, ones_c=True))
    log(f"[test] decode D={D} flags: no-rotate {e_r:.3e}, one-scale {e_1:.3e}")
    assert e_r <= ATTN_RL2 and e_1 <= ATTN_RL2


@pytest.mark.parametrize("D", DIMS)
def test_pipeline_headdim(kvarn, oracle, D):
    """Quantize, append and decode of the synthetic K/V against the oracle's
    own pipeline, decode fed the GPU-produced cache."""
    B, Hkv, G, T = 2, 2, 4, 384
    caches, hosts = [], []
    for kind in (kvgen.K, kvgen.V):
        x = kvgen.kv_tensor(101, 0, kind, B, Hkv, T, 0.5, head_dim=D)
        c = kvarn.Cache.empty(B, Hkv, T + 128, kind, device="cuda", head_dim=D)
        kvarn.quantize(x.cuda(), c)
        n = kvgen.new_tokens(101, 0, kind, B, Hkv, 0.5, head_dim=D)
        kvarn.append(n.cuda(), torch.full((B,), T, dtype=torch.int32, device="cuda"), c)
        caches.append(c)
    torch.cuda.synchronize()
    q = kvgen.queries(102, 0, B, Hkv * G, head_dim=D)
    lens = [T + 1, 200]
    out = kvarn.decode_attn(q.cuda(), caches[0], caches[1],
                            torch.tensor(lens, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    for c, kind in zip(caches, (0, 1)):
        hosts.append((oracle.unpack(c.codes.cpu().numpy(), D=D, kind=kind),
                      c.row_scale.double().cpu().numpy(), c.col_scale.double().cpu().numpy()))
    want = oracle.decode_attn(q.double().numpy(), *hosts[0], *hosts[1], lens)
    err = rel_l2(out.cpu().numpy(), want)
    log(f"[test] pipeline D={D}: rel L2 {err:.3e}")
    assert err <= ATTN_RL2


@pytest.mark.parametrize("D", DIMS)
def test_token_error_headdim(kvarn, oracle, D):
    B, H, T = 2, 2, 256
    x = kvgen.kv_tensor(103, 0, kvgen.K, B, H, T, 0.5, dtype=torch.float32, head_dim=D)
    x[1, 0, 7] = 0
    for kind in (kvgen.K, kvgen.V):
        c = kvarn.Cache.empty(B, H, T, kind, device="cuda", head_dim=D)
        kvarn.quantize(x.cuda(), c)
        ratio, cosine = kvarn.token_error(x.cuda(), c)
        torch.cuda.synchronize()
        codes = oracle.unpack(c.codes.cpu().numpy(), D=D, kind=kind)
        rp, cs = c.row_scale.double().cpu().numpy(), c.col_scale.double().cpu().numpy()
        for b in range(B):
            for h in range(H):
                r_o, c_o = oracle.cache_token_error(x[b, h].double().numpy(), codes[b, h], rp[b, h],
                                                    cs[b, h])
                g_r, g_c = ratio[b, h].cpu().double().numpy(), cosine[b, h].cpu().double().numpy()
                fin = np.isfinite(r_o)
                np.testing.assert_allclose(g_r[fin], r_o[fin], rtol=1e-5, atol=0)
                assert np.array_equal(np.isinf(g_r), np.isinf(r_o))
                np.testing.assert_allclose(g_c, c_o, rtol=0, atol=1e-5)


def _token_errors(oracle, x, cache, kind, D, token_offset, tokens):
    """The oracle's ratio and cosine of x [B,H,tokens,D] (host fp64) against
    the cache's slots [token_offset, token_offset + tokens)."""
    codes = oracle.unpack(cache.codes.cpu().numpy(), D=D, kind=kind)
    rp, cs = cache.row_scale.double().cpu().numpy(), cache.col_scale.double().cpu().numpy()
    B, H = x.shape[:2]
    ratio, cosine = np.empty((B, H, tokens)), np.empty((B, H, tokens))
    sl = slice(token_offset, token_offset + tokens)
    for b in range(B):
        for h in range(H):
            xh = oracle.dequant(codes[b, h], rp[b, h], cs[b, h])[sl]
            ratio[b, h], cosine[b, h] = oracle.token_error(x[b, h], xh)
    return ratio, cosine


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_token_error_headdim_bf16_ragged_no_rotate(kvarn, oracle, D, kind):
    """bf16 input over all slots; fp32 strided input over the ragged slots
    [77, 77 + 301) of a random cache; and pre-rotated input with the rotation
    absorbed, which gives the unrotated numbers (the rotation keeps norms and
    inner products)."""
    B, H, T = 2, 2, 384
    x = kvgen.kv_tensor(107, 0, kind, B, H, T, 0.5, dtype=torch.bfloat16, head_dim=D)
    c = kvarn.Cache.empty(B, H, T, kind, device="cuda", head_dim=D)
    kvarn.quantize(x.cuda(), c)
    got = kvarn.token_error(x.cuda(), c)
    xr = torch.from_numpy(oracle.rotate(x.double().numpy())).float().cuda()
    got_r = kvarn.token_error(xr, c, flags=kvarn.FLAG_NO_ROTATE)
    ck, rk, colk = kvgen.random_cache(108 + kind, B, H, 512, head_dim=D)
    rc = kvarn.Cache(ck.cuda(), rk.cuda(), colk.cuda(), kind)
    big = torch.randn(B, H, 320, D, generator=torch.Generator().manual_seed(109),
                      dtype=torch.float32)
    xs = big.cuda()[:, :, 5:306]
    got_s = kvarn.token_error(xs, rc, token_offset=77)
    torch.cuda.synchronize()
    want = _token_errors(oracle, x.double().numpy(), c, kind, D, 0, T)
    want_s = _token_errors(oracle, xs.double().cpu().numpy(), rc, kind, D, 77, 301)
    for g, w, what in ((got, want, "bf16"), (got_r, want, "no-rotate"), (got_s, want_s, "ragged")):
        gr, gc = (t.double().cpu().numpy() for t in g)
        np.testing.assert_allclose(gr, w[0], rtol=1e-5, atol=0, err_msg=f"D={D} {what}: ratio")
        np.testing.assert_allclose(gc, w[1], rtol=0, atol=1e-5, err_msg=f"D={D} {what}: cosine")
    log(f"[test] token error D={D} kind={kind}: bf16, no-rotate and ragged range agree")


def test_noalloc_headdim(kvarn):
    """The allocation-free decode at head size 256 equals the workspace call."""
    D, B, Hkv, G, cap = 256, 2, 2, 4, 1024
    kc, vc, _, _ = _caches(kvarn, B, Hkv, cap, D, seed=105)
    q = kvgen.queries(106, 0, B, Hkv * G, head_dim=D, device="cuda")
    L = torch.tensor([1024, 500], dtype=torch.int32, device="cuda")
    for ns in (0, 12):
        ref = kvarn.decode_attn(q, kc, vc, L, n_split=ns)
        got = torch.full_like(ref, float("nan"))
        kvarn.decode_attn_noalloc(q, kc, vc, L, got, n_split=ns)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
