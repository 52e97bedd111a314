"""Host-side checks of libkvarn.so that need no GPU: every function declared in
include/kvarn.h is exported, and invalid arguments are rejected on the host
with the documented status before any HIP call (fake device addresses are
never dereferenced because validation fails first)."""
import ctypes
import os
import re

import pytest

import kv_cache_bit_kvarn_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvarn.h")

A = 0x10000   # fake, 16-byte aligned "device" addresses (never touched)
B = 0x20000
C = 0x30000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvarn_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kv.LIB_PATH):
        import kv_cache_bit_kvarn_amd.build as b
        b.build()
    return kv.load()


def test_header_symbols_exported(lib):
    names = _declared()
    assert set(names) == set(kv.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def _cache(batch=2, heads=4, cap=512, kind=kv.K, codes=A, row=B, col=C):
    return kv.CacheDesc(codes, row, col, batch, heads, cap, kind)


def _q(lib, x=A, dtype=kv.DT_BF16, sb=4 * 512 * 128, sh=512 * 128, st=128, tokens=256,
       off=0, iters=4, cache=None):
    cache = cache or _cache()
    return lib.kvarn_quantize(x, dtype, sb, sh, st, tokens, off, iters, ctypes.byref(cache),
                              None)


def test_quantize_validation(lib):
    assert _q(lib, x=None) == kv.ERR_NULL
    assert _q(lib, x=None, tokens=0) == kv.OK
    assert lib.kvarn_quantize(A, 0, 0, 0, 128, 128, 0, 4, None, None) == kv.ERR_NULL
    assert _q(lib, cache=_cache(codes=None)) == kv.ERR_NULL
    assert _q(lib, cache=_cache(row=None)) == kv.ERR_NULL
    assert _q(lib, cache=_cache(col=None)) == kv.ERR_NULL
    assert _q(lib, dtype=7) == kv.ERR_DTYPE
    assert _q(lib, cache=_cache(kind=2)) == kv.ERR_DTYPE
    assert _q(lib, tokens=100) == kv.ERR_SHAPE
    assert _q(lib, off=64) == kv.ERR_SHAPE
    assert _q(lib, tokens=-128) == kv.ERR_SHAPE
    assert _q(lib, iters=-1) == kv.ERR_SHAPE
    assert _q(lib, iters=65) == kv.ERR_SHAPE
    assert _q(lib, st=64) == kv.ERR_SHAPE
    assert _q(lib, cache=_cache(cap=500)) == kv.ERR_SHAPE
    assert _q(lib, tokens=512, off=128) == kv.ERR_CAPACITY
    assert _q(lib, tokens=640) == kv.ERR_CAPACITY
    assert _q(lib, x=A + 8) == kv.ERR_ALIGN
    assert _q(lib, st=132) == kv.ERR_ALIGN          # 264 bytes: not a multiple of 16
    assert _q(lib, sh=128 * 128 + 4) == kv.ERR_ALIGN
    assert _q(lib, cache=_cache(codes=A + 4)) == kv.ERR_ALIGN
    assert _q(lib, cache=_cache(col=C + 8)) == kv.ERR_ALIGN
    # no-ops: nothing to launch, nothing touched
    assert _q(lib, tokens=0) == kv.OK
    assert _q(lib, cache=_cache(batch=0)) == kv.OK


def test_append_validation(lib):
    c = _cache()
    assert lib.kvarn_append(None, 0, B, ctypes.byref(c), None) == kv.ERR_NULL
    assert lib.kvarn_append(A, 0, None, ctypes.byref(c), None) == kv.ERR_NULL
    assert lib.kvarn_append(A, 0, B, None, None) == kv.ERR_NULL
    assert lib.kvarn_append(A, 3, B, ctypes.byref(c), None) == kv.ERR_DTYPE
    assert lib.kvarn_append(A + 2, 0, B, ctypes.byref(c), None) == kv.ERR_ALIGN
    bad = _cache(cap=130)
    assert lib.kvarn_append(A, 0, B, ctypes.byref(bad), None) == kv.ERR_SHAPE
    empty = _cache(batch=0)
    assert lib.kvarn_append(A, 0, B, ctypes.byref(empty), None) == kv.OK


def test_append_kv_validation(lib):
    k, v = _cache(kind=kv.K), _cache(kind=kv.V)

    def call(xk=A, xv=C, dtype=0, pos=B, flags=0, kc=k, vc=v):
        return lib.kvarn_append_kv(xk, xv, dtype, pos, flags,
                                   ctypes.byref(kc) if kc is not None else None,
                                   ctypes.byref(vc) if vc is not None else None, None)
    assert call(xk=None) == kv.ERR_NULL
    assert call(xv=None) == kv.ERR_NULL
    assert call(pos=None) == kv.ERR_NULL
    assert call(kc=None) == kv.ERR_NULL
    assert call(vc=None) == kv.ERR_NULL
    assert call(flags=kv.FLAG_ONE_SCALE) == kv.ERR_FLAGS
    assert call(dtype=3) == kv.ERR_DTYPE
    assert call(kc=v) == kv.ERR_DTYPE                  # a V cache where K goes
    assert call(vc=k) == kv.ERR_DTYPE
    assert call(vc=_cache(kind=kv.V, cap=256)) == kv.ERR_SHAPE
    assert call(vc=_cache(kind=kv.V, heads=2)) == kv.ERR_SHAPE
    assert call(xv=C + 8) == kv.ERR_ALIGN
    assert call(kc=_cache(kind=kv.K, batch=0), vc=_cache(kind=kv.V, batch=0)) == kv.OK


def test_workspace_bytes(lib):
    # one int32 counter per (sequence, query head) rounded up to 256 bytes, then
    # the partials of ceil(chunks / 4) four-split workgroups per row
    assert lib.kvarn_decode_workspace_bytes(8, 32, 32768) == 1024 + 8 * 32 * 64 * 130 * 4
    assert lib.kvarn_decode_workspace_bytes(1, 4, 256) == 256 + 1 * 4 * 1 * 130 * 4
    assert lib.kvarn_decode_workspace_bytes(1, 4, 640) == 256 + 1 * 4 * 2 * 130 * 4
    assert lib.kvarn_decode_workspace_bytes(1, 4, 100) == 0
    assert lib.kvarn_decode_workspace_bytes(-1, 4, 256) == 0


def _d(lib, q=A, qdt=kv.DT_BF16, hq=16, k=None, v=None, lens=B, out=C, nsplit=0,
       ws=0x40000, wsb=None, scale=0.088):
    k = k or _cache(kind=kv.K)
    v = v or _cache(kind=kv.V)
    if wsb is None:
        wsb = lib.kvarn_decode_workspace_bytes(k.batch, hq, k.capacity)
    return lib.kvarn_decode_attn(q, qdt, hq, ctypes.byref(k), ctypes.byref(v), lens, scale,
                                 out, nsplit, ws, wsb, None)


def test_decode_validation(lib):
    assert _d(lib, q=None) == kv.ERR_NULL
    assert _d(lib, lens=None) == kv.ERR_NULL
    assert _d(lib, out=None) == kv.ERR_NULL
    assert _d(lib, ws=None) == kv.ERR_NULL
    assert _d(lib, k=_cache(kind=kv.V)) == kv.ERR_DTYPE
    assert _d(lib, v=_cache(kind=kv.K)) == kv.ERR_DTYPE
    assert _d(lib, qdt=9) == kv.ERR_DTYPE
    assert _d(lib, hq=6) == kv.ERR_SHAPE                  # 6 % 4 kv-heads
    assert _d(lib, hq=0) == kv.ERR_SHAPE
    assert _d(lib, hq=36) == kv.ERR_SHAPE                 # group of 9 > 8
    assert _d(lib, v=_cache(kind=kv.V, cap=256)) == kv.ERR_SHAPE
    assert _d(lib, v=_cache(kind=kv.V, heads=2)) == kv.ERR_SHAPE
    assert _d(lib, nsplit=-1) == kv.ERR_SHAPE
    assert _d(lib, scale=float("nan")) == kv.ERR_SHAPE
    assert _d(lib, wsb=100) == kv.ERR_WORKSPACE
    assert _d(lib, out=C + 4) == kv.ERR_ALIGN
    assert _d(lib, q=A + 2) == kv.ERR_ALIGN
    assert _d(lib, ws=0x40008) == kv.ERR_ALIGN
    assert _d(lib, k=_cache(batch=0, kind=kv.K), v=_cache(batch=0, kind=kv.V)) == kv.OK


def test_flags_validation(lib):
    c = _cache()
    assert lib.kvarn_quantize_ex(A, 0, 4 * 512 * 128, 512 * 128, 128, 256, 0, 4, 4,
                                 ctypes.byref(c), None) == kv.ERR_FLAGS
    assert lib.kvarn_quantize_ex(A, 0, 4 * 512 * 128, 512 * 128, 128, 256, 0, 4,
                                 kv.FLAG_ONE_SCALE, ctypes.byref(c), None) == kv.ERR_FLAGS
    assert lib.kvarn_quantize_ex(None, 0, 0, 0, 128, 256, 0, 4, kv.FLAG_NO_ROTATE,
                                 ctypes.byref(c), None) == kv.ERR_NULL
    assert lib.kvarn_append_ex(A, 0, B, kv.FLAG_ONE_SCALE, ctypes.byref(c), None) == kv.ERR_FLAGS
    assert lib.kvarn_append_ex(None, 0, B, kv.FLAG_NO_ROTATE, ctypes.byref(c),
                               None) == kv.ERR_NULL
    k, v = _cache(kind=kv.K), _cache(kind=kv.V)
    wsb = lib.kvarn_decode_workspace_bytes(k.batch, 16, k.capacity)
    assert lib.kvarn_decode_attn_ex(A, 0, 16, ctypes.byref(k), ctypes.byref(v), B, 0.088, 8,
                                    C, 0, 0x40000, wsb, None) == kv.ERR_FLAGS
    assert lib.kvarn_decode_attn_ex(A, 0, 16, ctypes.byref(k), ctypes.byref(v), B, 0.088,
                                    kv.FLAG_NO_ROTATE | kv.FLAG_ONE_SCALE, C, 0, 0x40000, 100,
                                    None) == kv.ERR_WORKSPACE


def _te(lib, x=A, dtype=kv.DT_BF16, sb=4 * 512 * 128, sh=512 * 128, st=128, tokens=200, off=0,
        flags=0, cache=None, ratio=0x50000, cosine=0x60000):
    cache = cache or _cache()
    return lib.kvarn_token_error(x, dtype, sb, sh, st, tokens, off, flags, ctypes.byref(cache),
                                 ratio, cosine, None)


def test_token_error_validation(lib):
    assert _te(lib, flags=kv.FLAG_ONE_SCALE) == kv.ERR_FLAGS
    assert _te(lib, x=None) == kv.ERR_NULL
    assert _te(lib, ratio=None) == kv.ERR_NULL
    assert _te(lib, cosine=None) == kv.ERR_NULL
    assert _te(lib, x=None, tokens=0) == kv.OK
    assert _te(lib, cache=_cache(codes=None)) == kv.ERR_NULL
    assert _te(lib, dtype=3) == kv.ERR_DTYPE
    assert _te(lib, tokens=-1) == kv.ERR_SHAPE
    assert _te(lib, off=-128) == kv.ERR_SHAPE
    assert _te(lib, st=64) == kv.ERR_SHAPE
    assert _te(lib, tokens=200, off=400) == kv.ERR_CAPACITY
    assert _te(lib, x=A + 2) == kv.ERR_ALIGN
    assert _te(lib, st=132) == kv.ERR_ALIGN
    assert _te(lib, ratio=0x50002) == kv.ERR_ALIGN
    assert _te(lib, cache=_cache(batch=0)) == kv.OK


def test_append_rebalance_validation(lib):
    c = _cache()
    W = 0x70000
    assert lib.kvarn_append_rebalance(A, 0, B, W, 4, kv.FLAG_ONE_SCALE, ctypes.byref(c),
                                      None) == kv.ERR_FLAGS
    assert lib.kvarn_append_rebalance(None, 0, B, W, 4, 0, ctypes.byref(c), None) == kv.ERR_NULL
    assert lib.kvarn_append_rebalance(A, 0, None, W, 4, 0, ctypes.byref(c), None) == kv.ERR_NULL
    assert lib.kvarn_append_rebalance(A, 0, B, None, 4, 0, ctypes.byref(c), None) == kv.ERR_NULL
    assert lib.kvarn_append_rebalance(A, 0, B, W, 4, 0, None, None) == kv.ERR_NULL
    assert lib.kvarn_append_rebalance(A, 9, B, W, 4, 0, ctypes.byref(c), None) == kv.ERR_DTYPE
    assert lib.kvarn_append_rebalance(A, 0, B, W + 8, 4, 0, ctypes.byref(c), None) == kv.ERR_ALIGN
    assert lib.kvarn_append_rebalance(A + 2, 0, B, W, 4, 0, ctypes.byref(c), None) == kv.ERR_ALIGN
    assert lib.kvarn_append_rebalance(A, 0, B, W, 65, 0, ctypes.byref(c), None) == kv.ERR_SHAPE
    assert lib.kvarn_append_rebalance(A, 0, B, W, -1, 0, ctypes.byref(c), None) == kv.ERR_SHAPE
    z = _cache(batch=0)
    assert lib.kvarn_append_rebalance(A, 0, B, W, 4, 0, ctypes.byref(z), None) == kv.OK


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = kv.status_string(st)
        assert s and s != "unknown status"
    assert kv.status_string(-99) == "unknown status"


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib
    mod = importlib.import_module("kv_cache_bit_kvarn_amd")
    monkeypatch.setattr(mod, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        mod.load(str(tmp_path / "nope.so"))
