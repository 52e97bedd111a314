"""GPU parity of kvarn_quantize against the oracle (codes, row and column
scales), through the C ABI."""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import assert_quant_parity, cache_blocks, log, sample_blocks, x_blocks

pytestmark = pytest.mark.gpu


def _full(oracle, kv, x, kind, iters=4, token_offset=0, capacity=None):
    B, H, T, _ = x.shape
    cap = capacity or (T + token_offset)
    cache = kv.Cache.empty(B, H, cap, kind, device="cuda")
    kv.quantize(x.cuda() if not x.is_cuda else x, cache, token_offset=token_offset,
                iters=iters)
    torch.cuda.synchronize()
    return cache


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_tiny_fp32_full(kvarn, oracle, kind):
    """Tiny oracle case: 1 layer, 1 kv-head, 256 tokens x 128 channels fp32,
    4 iterations; every element compared."""
    wl = kvgen.WORKLOADS[0]
    log(f"[test] tiny fp32 kind={kind}")
    x = kvgen.kv_tensor(wl.seed, 0, kind, 1, 1, 256, wl.sigma, dtype=torch.float32)
    cache = _full(oracle, kvarn, x, kind)
    ora = oracle.quantize_tensor(x.double().numpy())
    g_codes = oracle.unpack(cache.codes.cpu().numpy(), kind=kind)
    st = assert_quant_parity(oracle, ora, g_codes, cache.row_scale.cpu().numpy(),
                             cache.col_scale.cpu().numpy(), "tiny")
    log(f"  {st}")
    # byte-level: packing the oracle's codes reproduces the GPU bytes wherever
    # no boundary element is involved
    if st["flipped"] == 0:
        np.testing.assert_array_equal(oracle.pack(ora["codes"], kind=kind),
                                      cache.codes.cpu().numpy())


@pytest.mark.parametrize("iters", [0, 1, 2, 7])
def test_iteration_counts(kvarn, oracle, iters):
    x = kvgen.kv_tensor(5, 0, kvgen.K, 2, 2, 256, 0.5, dtype=torch.bfloat16)
    cache = _full(oracle, kvarn, x, kvgen.K, iters=iters)
    ora = oracle.quantize_tensor(x.double().numpy(), iters=iters)
    g_codes = oracle.unpack(cache.codes.cpu().numpy(), kind=kvgen.K)
    assert_quant_parity(oracle, ora, g_codes, cache.row_scale.cpu().numpy(),
                        cache.col_scale.cpu().numpy(), f"iters={iters}")


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_qwen_layer_sampled(kvarn, oracle, kind):
    """One Qwen3-4B-shaped layer (batch 1, 8 kv-heads, 32768 tokens, bf16),
    quantized in one launch; 256 sampled blocks (incl. first and last)
    checked against the oracle."""
    wl = kvgen.WORKLOADS[1]
    log(f"[test] qwen layer kind={kind}")
    x = kvgen.kv_tensor(wl.seed, 0, kind, wl.batch, wl.kv_heads, wl.tokens, wl.sigma,
                        dtype=torch.bfloat16, device="cuda")
    cache = _full(oracle, kvarn, x, kind)
    nch = wl.tokens // 128
    sel = sample_blocks(np.random.default_rng(kind), wl.batch, wl.kv_heads, nch, 256,
                        always=[(0, 0, 0), (0, wl.kv_heads - 1, nch - 1)])
    ora = oracle.quantize_tensor(x_blocks(x, sel), threads=8)
    st = assert_quant_parity(oracle, ora, *cache_blocks(cache, kind, sel), "qwen layer")
    log(f"  {st}")


def test_strided_input_and_offset(kvarn, oracle):
    """x a strided view (token stride 256 elements, head stride padded) and
    written at token_offset 256 of a larger cache; other slots untouched."""
    base = kvgen.kv_tensor(6, 0, kvgen.V, 2, 3, 256, 0.5, dtype=torch.bfloat16,
                           device="cuda")
    big = torch.zeros((2, 3, 256, 256), dtype=torch.bfloat16, device="cuda")
    big[..., 64:192] = base
    x = big[..., 64:192]
    assert x.stride(2) == 256
    cache = kvarn.Cache.empty(2, 3, 640, kvgen.V, device="cuda")
    kvarn.quantize(x, cache, token_offset=256, iters=4)
    torch.cuda.synchronize()
    ora = oracle.quantize_tensor(base.double().cpu().numpy())
    g = oracle.unpack(cache.codes.cpu().numpy(), kind=kvgen.V)
    assert_quant_parity(oracle, ora, g[:, :, 256:512], cache.row_scale[:, :, 256:512].cpu(),
                        cache.col_scale[:, :, 2:4].cpu(), "strided")
    assert cache.codes[:, :, :2].count_nonzero() == 0
    assert cache.codes[:, :, 4:].count_nonzero() == 0
    assert cache.row_scale[:, :, :256].count_nonzero() == 0


def test_degenerate_blocks(kvarn, oracle):
    """Zero token rows (r' = 0, code 2) and zero channels after rotation
    (c = 1) handled like the oracle."""
    x = torch.randn((1, 2, 128, 128), dtype=torch.float32)
    x[0, 0, 5] = 0
    x[0, 0, 77] = 0
    x[0, 1] = 0          # an all-zero block
    cache = _full(oracle, kvarn, x, kvgen.K)
    ora = oracle.quantize_tensor(x.double().numpy())
    g = oracle.unpack(cache.codes.cpu().numpy(), kind=kvgen.K)
    assert_quant_parity(oracle, ora, g, cache.row_scale.cpu().numpy(),
                        cache.col_scale.cpu().numpy(), "degenerate")
    assert float(cache.row_scale[0, 0, 5]) == 0.0
    assert np.all(g[0, 1] == 2)


def test_power_of_two_token_scaling_is_bit_exact(kvarn):
    """Scaling a token by 2^k changes only its row scale, by exactly 2^k;
    codes and column scales stay bit-identical (the row step absorbs it)."""
    x = kvgen.kv_tensor(8, 0, kvgen.K, 1, 4, 512, 0.5, dtype=torch.float32, device="cuda")
    e = torch.randint(-5, 6, (1, 4, 512, 1), generator=torch.Generator().manual_seed(1))
    s = torch.pow(2.0, e.float()).cuda()
    c1 = kvarn.Cache.empty(1, 4, 512, kvgen.K, device="cuda")
    c2 = kvarn.Cache.empty(1, 4, 512, kvgen.K, device="cuda")
    kvarn.quantize(x, c1)
    kvarn.quantize((x * s).contiguous(), c2)
    torch.cuda.synchronize()
    assert torch.equal(c1.codes, c2.codes)
    assert torch.equal(c1.col_scale, c2.col_scale)
    assert torch.equal(c1.row_scale * s[..., 0], c2.row_scale)


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
@pytest.mark.parametrize("k", [-40, -20, 20, 40])
def test_power_of_two_tensor_scaling_is_bit_exact(kvarn, kind, k):
    """Scaling the whole input by 2^k, far from unit magnitudes, scales every
    row scale by exactly 2^k and leaves codes and column scales bit-identical:
    the fp32 sums stay normal and finite over this range (|x| up to about
    2^48, squared rotated values down to about 2^-110 here)."""
    log(f"[test] tensor scaling 2^{k} kind={kind}")
    x = kvgen.kv_tensor(21, 0, kind, 1, 2, 512, 0.5, dtype=torch.bfloat16, device="cuda")
    c1 = kvarn.Cache.empty(1, 2, 512, kind, device="cuda")
    c2 = kvarn.Cache.empty(1, 2, 512, kind, device="cuda")
    kvarn.quantize(x, c1)
    kvarn.quantize((x * 2.0 ** k).contiguous(), c2)
    torch.cuda.synchronize()
    assert torch.equal(c1.codes, c2.codes)
    assert torch.equal(c1.col_scale, c2.col_scale)
    assert torch.equal(c1.row_scale * 2.0 ** k, c2.row_scale)


def test_block_independence(kvarn):
    """Quantizing a subset of chunks gives the same bytes as the same chunks of
    a full run."""
    x = kvgen.kv_tensor(9, 0, kvgen.V, 2, 2, 1024, 0.5, dtype=torch.bfloat16, device="cuda")
    full = kvarn.Cache.empty(2, 2, 1024, kvgen.V, device="cuda")
    part = kvarn.Cache.empty(2, 2, 1024, kvgen.V, device="cuda")
    kvarn.quantize(x, full)
    kvarn.quantize(x[:, :, 384:768], part, token_offset=384)
    torch.cuda.synchronize()
    assert torch.equal(full.codes[:, :, 3:6], part.codes[:, :, 3:6])
    assert torch.equal(full.row_scale[:, :, 384:768], part.row_scale[:, :, 384:768])
    assert torch.equal(full.col_scale[:, :, 3:6], part.col_scale[:, :, 3:6])


def test_errors_raise(kvarn):
    cache = kvarn.Cache.empty(1, 1, 256, kvgen.K, device="cuda")
    x = torch.zeros((1, 1, 384, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvarn.KvarnError) as e:
        kvarn.quantize(x, cache)
    assert e.value.status == kvarn.ERR_CAPACITY
    with pytest.raises(kvarn.KvarnError):
        kvarn.quantize(x[:, :, :100].contiguous(), cache)
    kvarn.quantize(x[:, :, :0], cache)   # no-op
