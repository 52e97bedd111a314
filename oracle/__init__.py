"""CPU oracle for the KVarN quantizer and its decode attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in
__graft_entry__.py and by the cpu_baseline leg of bench.py; never by the
product package kv_cache_bit_kvarn_amd, which shares no code with it.

This module is argument marshalling around kvarn_oracle.c (plain fp64 C,
built by gcc into liboracle_kvarn.so). Every arithmetic step of the method is
in that C file, each function citing the passage it follows. Unpinned parts:
none of the functions here is left without a pin (see tests/test_oracle_*.py);
what the pins cannot reach is that the pages' authors may have made other
choices where the pages are silent (the SC-n readings), so agreement with the
authors' own code is not claimed.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvarn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_kvarn.so")

CHUNK = 128

_dp = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_ip = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True) -> str:
    """Compile kvarn_oracle.c with gcc (strict IEEE fp64: no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
_lock = threading.Lock()


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            L = ctypes.CDLL(_LIB)
            L.kvo_hadamard_entry.restype = ctypes.c_double
            L.kvo_hadamard_entry.argtypes = [ctypes.c_int, ctypes.c_int]
            L.kvo_rotate.argtypes = [_dp, ctypes.c_int, ctypes.c_int, _dp]
            L.kvo_balance.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _dp, _dp, _dp]
            L.kvo_quantize_block.argtypes = [_dp, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, _u8p, _dp, _dp, _dp, _dp]
            L.kvo_quantize_tensor.argtypes = [_dp] + [ctypes.c_int] * 6 + [
                _u8p, _dp, _dp, _dp, _dp]
            L.kvo_append.argtypes = [_dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     _ip, _u8p, _dp, _dp, ctypes.c_int,
                                     ctypes.c_int, _dp]
            L.kvo_pack.argtypes = [_u8p] + [ctypes.c_int] * 6 + [_u8p]
            L.kvo_unpack.argtypes = [_u8p] + [ctypes.c_int] * 6 + [_u8p]
            L.kvo_dequant.argtypes = [_u8p, _dp, _dp, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, _dp]
            L.kvo_decode_attn.argtypes = [_dp] + [ctypes.c_int] * 4 + [
                _u8p, _dp, _dp, _u8p, _dp, _dp, ctypes.c_int, ctypes.c_int, _ip,
                ctypes.c_double, _dp]
            L.kvo_token_error.argtypes = [_dp, _dp, ctypes.c_int, ctypes.c_int, _dp, _dp]
            for name in ("kvo_rotate", "kvo_balance", "kvo_quantize_block",
                         "kvo_quantize_tensor", "kvo_append", "kvo_pack",
                         "kvo_unpack", "kvo_dequant", "kvo_decode_attn",
                         "kvo_token_error"):
                getattr(L, name).restype = ctypes.c_int
            _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _check(st: int, what: str):
    if st != 0:
        raise OracleError(f"{what} failed with status {st}"
                          + (" (non-finite input)" if st == -2 else ""))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def hadamard_entry(i: int, k: int) -> float:
    return lib().kvo_hadamard_entry(int(i), int(k))


def rotate(x) -> np.ndarray:
    """Rows of x[..., D] times H_D / sqrt(D) (own inverse)."""
    x = _f64(x)
    d = x.shape[-1]
    rows = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    y = np.empty_like(x)
    _check(lib().kvo_rotate(_ptr(x, _dp), rows, d, _ptr(y, _dp)), "rotate")
    return y


def balance(y, iters: int = 4):
    """Returns (r[T], c[D], eps[iters]) for one block y[T][D]."""
    y = _f64(y)
    T, D = y.shape
    r = np.empty(T)
    c = np.empty(D)
    eps = np.empty(max(iters, 1))
    _check(lib().kvo_balance(_ptr(y, _dp), T, D, iters, _ptr(r, _dp), _ptr(c, _dp),
                             _ptr(eps, _dp)), "balance")
    return r, c, eps[:iters]


def quantize_block(x, iters: int = 4):
    """One block x[T][D] -> dict(codes[T][D] u8, rp[T], c[D], u[T][D], eps)."""
    x = _f64(x)
    T, D = x.shape
    codes = np.empty((T, D), np.uint8)
    rp = np.empty(T)
    c = np.empty(D)
    u = np.empty((T, D))
    eps = np.empty(max(iters, 1))
    _check(lib().kvo_quantize_block(_ptr(x, _dp), T, D, iters, _ptr(codes, _u8p),
                                    _ptr(rp, _dp), _ptr(c, _dp), _ptr(u, _dp),
                                    _ptr(eps, _dp)), "quantize_block")
    return dict(codes=codes, rp=rp, c=c, u=u, eps=eps[:iters])


def quantize_tensor(x, chunk: int = CHUNK, iters: int = 4, want_u: bool = True,
                    threads: int = 1):
    """Dense x[B][H][T][D] -> unpacked codes/u [B,H,T,D], rp [B,H,T],
    c [B,H,T/chunk,D], eps [B,H,T/chunk,iters]. `threads` > 1 runs independent
    (b, h) slices on Python threads (the C call releases the GIL)."""
    x = _f64(x)
    B, H, T, D = x.shape
    nch = T // chunk
    codes = np.empty((B, H, T, D), np.uint8)
    rp = np.empty((B, H, T))
    c = np.empty((B, H, nch, D))
    u = np.empty((B, H, T, D)) if want_u else None
    eps = np.empty((B, H, nch, max(iters, 1)))

    def run(bh_lo: int, bh_hi: int):
        xs = x.reshape(B * H, T, D)[bh_lo:bh_hi]
        n = bh_hi - bh_lo
        cs = codes.reshape(B * H, T, D)[bh_lo:bh_hi]
        rs = rp.reshape(B * H, T)[bh_lo:bh_hi]
        ccs = c.reshape(B * H, nch, D)[bh_lo:bh_hi]
        us = u.reshape(B * H, T, D)[bh_lo:bh_hi] if u is not None else None
        es = eps.reshape(B * H, nch, -1)[bh_lo:bh_hi]
        _check(lib().kvo_quantize_tensor(
            _ptr(xs, _dp), 1, n, T, D, chunk, iters, _ptr(cs, _u8p), _ptr(rs, _dp),
            _ptr(ccs, _dp), _ptr(us, _dp) if us is not None else None,
            _ptr(es, _dp) if iters > 0 else None), "quantize_tensor")

    nbh = B * H
    if threads <= 1 or nbh <= 1:
        run(0, nbh)
    else:
        errs = []

        def worker(lo, hi):
            try:
                run(lo, hi)
            except Exception as e:  # pragma: no cover - surfaced below
                errs.append(e)
        bounds = np.linspace(0, nbh, min(threads, nbh) + 1).astype(int)
        ts = [threading.Thread(target=worker, args=(int(lo), int(hi)))
              for lo, hi in zip(bounds[:-1], bounds[1:]) if hi > lo]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        if errs:
            raise errs[0]
    return dict(codes=codes, rp=rp, c=c, u=u, eps=eps[..., :iters])


def append(x, pos, codes, rp, c, chunk: int = CHUNK):
    """In-place append of x[B][H][D] at pos[B] into unpacked cache arrays
    codes[B,H,cap,D] u8, rp[B,H,cap] f64, c[B,H,cap/chunk,D] f64.
    Returns u[B][H][D] (pre-rounding values)."""
    x = _f64(x)
    B, H, D = x.shape
    cap = codes.shape[2]
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int32))
    for a, dt in ((codes, np.uint8), (rp, np.float64), (c, np.float64)):
        if a.dtype != dt or not a.flags.c_contiguous:
            raise OracleError("cache arrays must be C-contiguous u8/f64/f64")
    u = np.zeros((B, H, D))
    _check(lib().kvo_append(_ptr(x, _dp), B, H, D, _ptr(pos, _ip), _ptr(codes, _u8p),
                            _ptr(rp, _dp), _ptr(c, _dp), cap, chunk, _ptr(u, _dp)),
           "append")
    return u


def pack(codes, chunk: int = CHUNK, kind: int = 0) -> np.ndarray:
    """codes[B,H,T,D] -> packed [B,H,T/chunk,chunk*D/4] (kind 0 = K, 1 = V)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    B, H, T, D = codes.shape
    out = np.empty((B, H, T // chunk, chunk * D // 4), np.uint8)
    _check(lib().kvo_pack(_ptr(codes, _u8p), B, H, T, D, chunk, kind,
                          _ptr(out, _u8p)), "pack")
    return out


def unpack(packed, D: int = 128, chunk: int = CHUNK, kind: int = 0) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    B, H, nch, per = packed.shape
    assert per == chunk * D // 4
    T = nch * chunk
    out = np.empty((B, H, T, D), np.uint8)
    _check(lib().kvo_unpack(_ptr(packed, _u8p), B, H, T, D, chunk, kind,
                            _ptr(out, _u8p)), "unpack")
    return out


def dequant(codes, rp, c, chunk: int = CHUNK) -> np.ndarray:
    """One (sequence, head): codes[n][D], rp[n], c[>=ceil(n/chunk)][D] ->
    reconstruction in the original basis [n][D]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rp = _f64(rp)
    c = _f64(c)
    n, D = codes.shape
    out = np.empty((n, D))
    _check(lib().kvo_dequant(_ptr(codes, _u8p), _ptr(rp, _dp), _ptr(c, _dp), n, D,
                             chunk, _ptr(out, _dp)), "dequant")
    return out


def decode_attn(q, k_codes, k_rp, k_c, v_codes, v_rp, v_c, lens, scale=None,
                chunk: int = CHUNK) -> np.ndarray:
    """q[B,Hq,D]; caches unpacked: codes[B,Hkv,cap,D], rp[B,Hkv,cap],
    c[B,Hkv,cap/chunk,D]; lens[B] -> out[B,Hq,D] (fp64)."""
    q = _f64(q)
    B, Hq, D = q.shape
    k_codes = np.ascontiguousarray(k_codes, dtype=np.uint8)
    v_codes = np.ascontiguousarray(v_codes, dtype=np.uint8)
    Hkv, cap = k_codes.shape[1], k_codes.shape[2]
    k_rp, k_c, v_rp, v_c = (_f64(a) for a in (k_rp, k_c, v_rp, v_c))
    lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D))
    _check(lib().kvo_decode_attn(
        _ptr(q, _dp), B, Hq, Hkv, D, _ptr(k_codes, _u8p), _ptr(k_rp, _dp),
        _ptr(k_c, _dp), _ptr(v_codes, _u8p), _ptr(v_rp, _dp), _ptr(v_c, _dp), cap,
        chunk, _ptr(lens, _ip), float(scale), _ptr(out, _dp)), "decode_attn")
    return out


def boundary_mask(u, tol: float = 1e-5) -> np.ndarray:
    """Elements whose pre-rounding value lies within `tol` of a rounding
    boundary (u in {-1, 0, +1}); their code may legitimately differ between
    an fp64 and an fp32 evaluation."""
    u = np.asarray(u, dtype=np.float64)
    return np.min(np.abs(u[..., None] - np.array([-1.0, 0.0, 1.0])), axis=-1) < tol


def token_error(x, xhat):
    """Per-token (||xhat|| / ||x||, cos(xhat, x)) over the last axis of
    x, xhat [..., D]; the magnitude and direction parts of the error
    (kvo_token_error). Returns two arrays of shape x.shape[:-1]."""
    x = _f64(x)
    xhat = _f64(xhat)
    if x.shape != xhat.shape:
        raise ValueError("x and xhat differ in shape")
    D = x.shape[-1]
    n = x.size // D if D else 0
    ratio = np.empty(x.shape[:-1])
    cosine = np.empty(x.shape[:-1])
    _check(lib().kvo_token_error(_ptr(x, _dp), _ptr(xhat, _dp), n, D, _ptr(ratio, _dp),
                                 _ptr(cosine, _dp)), "token_error")
    return ratio, cosine


def cache_token_error(x, codes, rp, c, chunk: int = CHUNK):
    """One (sequence, head): original tokens x[n][D] against the cache's
    reconstruction of the same n tokens (codes unpacked [n][D], rp[n],
    c[>=ceil(n/chunk)][D]) -> (ratio[n], cosine[n])."""
    return token_error(x, dequant(codes, rp, c, chunk))
