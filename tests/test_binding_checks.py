"""The Python binding's argument checks, which need no GPU: host tensors,
mismatched shapes and wrong output buffers are refused with ValueError before
any pointer reaches the library (the kernels would otherwise read or write a
host address or out of bounds)."""
import pytest
import torch

import kv_cache_bit_kvarn_amd as kv


def _cache(kind=kv.K, B=2, H=2, cap=256):
    return kv.Cache.empty(B, H, cap, kind, device="cpu")


def test_host_cache_refused():
    c = _cache()
    with pytest.raises(ValueError, match="GPU"):
        c.desc()


def test_cache_layout_checked():
    c = _cache()
    bad = kv.Cache(c.codes, c.row_scale[:, :, :128].contiguous(), c.col_scale, kv.K)
    with pytest.raises(ValueError, match="row_scale"):
        bad.desc()
    bad = kv.Cache(c.codes, c.row_scale, c.col_scale.double(), kv.K)
    with pytest.raises(ValueError, match="fp32"):
        bad.desc()
    bad = kv.Cache(c.codes, c.row_scale, c.col_scale, 5)
    with pytest.raises(ValueError, match="kind"):
        bad.desc()


def test_quantize_host_tensors_refused():
    x = torch.zeros((2, 2, 256, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kv.quantize(x, _cache())


def test_append_host_positions_refused():
    x = torch.zeros((2, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kv.append(x, torch.zeros(2, dtype=torch.int32), _cache())
    with pytest.raises(ValueError, match="int32"):
        kv.append(x, torch.zeros(2, dtype=torch.int64), _cache())


def test_append_kv_checks():
    k, v = _cache(kv.K), _cache(kv.V)
    x = torch.zeros((2, 2, 128), dtype=torch.bfloat16)
    pos = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="K cache and a V cache"):
        kv.append_kv(x, x, pos, v, k)
    with pytest.raises(ValueError, match="shape"):
        kv.append_kv(x, x, pos, k, _cache(kv.V, cap=512))
    with pytest.raises(ValueError, match="matching"):
        kv.append_kv(x, torch.zeros((2, 2, 64), dtype=torch.bfloat16), pos, k, v)
    with pytest.raises(ValueError, match="one dtype"):
        kv.append_kv(x, x.float(), pos, k, v)
    with pytest.raises(ValueError, match="int32"):
        kv.append_kv(x, x, pos.long(), k, v)
    with pytest.raises(ValueError, match="GPU"):       # host tensors and caches
        kv.append_kv(x, x, pos, k, v)


def test_decode_checks():
    k, v = _cache(kv.K), _cache(kv.V)
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="batch"):
        kv.decode_attn(torch.zeros((3, 8, 128), dtype=torch.bfloat16), k, v, lens)
    with pytest.raises(ValueError, match="out"):
        kv.decode_attn(q, k, v, lens, out=torch.zeros((2, 8, 64), dtype=torch.float32))
    with pytest.raises(ValueError, match="out"):
        kv.decode_attn(q, k, v, lens, out=torch.zeros((2, 8, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out"):
        kv.decode_attn(q, k, v, lens, out=torch.zeros((2, 128, 8)).transpose(1, 2))
    with pytest.raises(ValueError, match="seq_lens"):
        kv.decode_attn(q, k, v, torch.ones(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        kv.decode_attn(q, k, v, lens)


def test_token_error_output_shapes():
    c = _cache()
    x = torch.zeros((2, 2, 256, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="ratio"):
        kv.token_error(x, c, ratio=torch.zeros((2, 2, 128)))
    with pytest.raises(ValueError, match="cosine"):
        kv.token_error(x, c, cosine=torch.zeros((2, 2, 256), dtype=torch.float64))


def test_cache_head_dim_checked():
    c = kv.Cache.empty(1, 1, 128, kv.K, device="cpu", head_dim=256)
    assert c.head_dim == 256 and c.codes.shape[3] == 32 * 256
    bad = kv.Cache.empty(1, 1, 128, kv.K, device="cpu", head_dim=96)
    with pytest.raises(ValueError, match="head_dim"):
        bad.desc()
    with pytest.raises(ValueError, match="D"):
        kv.quantize(torch.zeros((1, 1, 128, 128)), c)
    k2 = kv.Cache.empty(1, 1, 128, kv.K, device="cpu", head_dim=64)
    v2 = kv.Cache.empty(1, 1, 128, kv.V, device="cpu", head_dim=256)
    with pytest.raises(ValueError, match="head_dim"):
        kv.decode_attn(torch.zeros((1, 4, 64), dtype=torch.bfloat16), k2, v2,
                       torch.ones(1, dtype=torch.int32))
