"""Python binding of libkvarn.so, the MI355X KVarN quantizer and 2-bit decode
attention (C ABI declared in include/kvarn.h).

Argument marshalling only: torch tensors are used for device memory and
streams; every step of the method runs in the library's HIP kernels. There is
no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvarn.so")

HEAD_DIM = 128
HEAD_DIMS = (64, 128, 256)   # supported head sizes (128: the tuned kernels)
CHUNK = 128
CHUNK_BYTES = 4096           # packed codes of one chunk at head size 128 (32 x head_dim)

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_CAPACITY, ERR_WORKSPACE, ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6, -7)
ERR_FLAGS = -8
FLAG_NO_ROTATE, FLAG_ONE_SCALE = 1, 2
DT_BF16, DT_F32 = 0, 1
K, V = 0, 1

EXPORTED = ("kvarn_quantize", "kvarn_quantize_ex", "kvarn_append", "kvarn_append_ex",
            "kvarn_append_kv",
            "kvarn_decode_workspace_bytes", "kvarn_decode_workspace_bytes_ex",
            "kvarn_decode_attn", "kvarn_decode_attn_ex",
            "kvarn_decode_attn_noalloc", "kvarn_append_rebalance", "kvarn_token_error",
            "kvarn_status_string")
NOALLOC_SCRATCH_BYTES = 16 << 20   # KVARN_NOALLOC_SCRATCH_BYTES


class KvarnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class CacheDesc(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("row_scale", ctypes.c_void_p),
                ("col_scale", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("kind", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


_lib = None


def load(path: str | None = None):
    """Load libkvarn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with kv_cache_bit_kvarn_amd/build.py "
                           "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    cd = ctypes.POINTER(CacheDesc)
    L.kvarn_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, i32, cd, vp]
    L.kvarn_quantize.restype = ctypes.c_int
    L.kvarn_append.argtypes = [vp, i32, vp, cd, vp]
    L.kvarn_append.restype = ctypes.c_int
    L.kvarn_decode_workspace_bytes.argtypes = [i32, i32, i32]
    L.kvarn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.kvarn_decode_workspace_bytes_ex.argtypes = [i32, i32, i32, i32]
    L.kvarn_decode_workspace_bytes_ex.restype = ctypes.c_size_t
    L.kvarn_decode_attn.argtypes = [vp, i32, i32, cd, cd, vp, ctypes.c_float, vp, i32,
                                    vp, ctypes.c_size_t, vp]
    L.kvarn_decode_attn.restype = ctypes.c_int
    u32 = ctypes.c_uint32
    L.kvarn_quantize_ex.argtypes = [vp, i32, i64, i64, i64, i32, i32, i32, u32, cd, vp]
    L.kvarn_quantize_ex.restype = ctypes.c_int
    L.kvarn_append_ex.argtypes = [vp, i32, vp, u32, cd, vp]
    L.kvarn_append_ex.restype = ctypes.c_int
    L.kvarn_append_kv.argtypes = [vp, vp, i32, vp, u32, cd, cd, vp]
    L.kvarn_append_kv.restype = ctypes.c_int
    L.kvarn_decode_attn_ex.argtypes = [vp, i32, i32, cd, cd, vp, ctypes.c_float, u32, vp, i32,
                                       vp, ctypes.c_size_t, vp]
    L.kvarn_decode_attn_ex.restype = ctypes.c_int
    L.kvarn_decode_attn_noalloc.argtypes = [vp, i32, i32, cd, cd, vp, ctypes.c_float, u32, vp,
                                            i32, vp]
    L.kvarn_decode_attn_noalloc.restype = ctypes.c_int
    L.kvarn_append_rebalance.argtypes = [vp, i32, vp, vp, i32, u32, cd, vp]
    L.kvarn_append_rebalance.restype = ctypes.c_int
    L.kvarn_token_error.argtypes = [vp, i32, i64, i64, i64, i32, i32, u32, cd, vp, vp, vp]
    L.kvarn_token_error.restype = ctypes.c_int
    L.kvarn_status_string.argtypes = [ctypes.c_int]
    L.kvarn_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().kvarn_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _on_device(what: str, *tensors) -> torch.device:
    """Every tensor argument must live on one GPU: the kernels dereference
    their data pointers on the device, so a host tensor would be read as a
    device address."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            where = t.device if isinstance(t, torch.Tensor) else type(t).__name__
            raise ValueError(f"{what}: every tensor argument must be on the GPU (got {where})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{what}: tensor arguments on different devices ({dev}, {t.device})")
    return dev


def _stream(stream, device=None) -> int | None:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _raise(st: int, what: str):
    if st != OK:
        raise KvarnError(st, what)


@dataclass
class Cache:
    """One layer's K or V cache: device tensors in the layout of kvarn.h
    (D = head_dim: 64, 128 or 256)."""
    codes: torch.Tensor      # uint8 [B, H, cap/128, 32 D]
    row_scale: torch.Tensor  # f32 [B, H, cap]
    col_scale: torch.Tensor  # f32 [B, H, cap/128, D]
    kind: int

    @staticmethod
    def empty(batch: int, kv_heads: int, capacity: int, kind: int, device="cuda",
              zero: bool = True, head_dim: int = HEAD_DIM) -> "Cache":
        nch = capacity // CHUNK
        f = torch.zeros if zero else torch.empty
        return Cache(f((batch, kv_heads, nch, 32 * head_dim), dtype=torch.uint8, device=device),
                     f((batch, kv_heads, capacity), dtype=torch.float32, device=device),
                     f((batch, kv_heads, nch, head_dim), dtype=torch.float32, device=device),
                     kind)

    @property
    def batch(self):
        return self.codes.shape[0]

    @property
    def kv_heads(self):
        return self.codes.shape[1]

    @property
    def capacity(self):
        return self.row_scale.shape[2]

    @property
    def head_dim(self):
        return self.col_scale.shape[3] if self.col_scale.dim() == 4 else HEAD_DIM

    def desc(self) -> CacheDesc:
        """The kvarn_cache descriptor, after checking dtypes, shapes and
        placement against the layout the kernels index."""
        for t in (self.codes, self.row_scale, self.col_scale):
            if not t.is_contiguous():
                raise ValueError("cache tensors must be contiguous")
        if self.codes.dtype != torch.uint8 or self.row_scale.dtype != torch.float32 or \
                self.col_scale.dtype != torch.float32:
            raise ValueError("cache tensors must be uint8 codes and fp32 scales")
        if self.codes.dim() != 4 or self.row_scale.dim() != 3 or self.col_scale.dim() != 4:
            raise ValueError("cache tensors must be codes [B,H,cap/128,32 D], row_scale "
                             "[B,H,cap], col_scale [B,H,cap/128,D]")
        B, H, nch = self.codes.shape[:3]
        D = self.col_scale.shape[3]
        if D not in HEAD_DIMS:
            raise ValueError(f"head_dim {D} not supported (64, 128 or 256)")
        if self.codes.shape[3] != 32 * D or \
                tuple(self.row_scale.shape) != (B, H, nch * CHUNK) or \
                tuple(self.col_scale.shape) != (B, H, nch, D):
            raise ValueError("cache tensors must be codes [B,H,cap/128,32 D], row_scale "
                             "[B,H,cap], col_scale [B,H,cap/128,D] with one B, H, cap and D")
        if self.kind not in (K, V):
            raise ValueError("cache kind must be K or V")
        _on_device("cache", self.codes, self.row_scale, self.col_scale)
        return CacheDesc(self.codes.data_ptr(), self.row_scale.data_ptr(),
                         self.col_scale.data_ptr(), self.batch, self.kv_heads,
                         self.capacity, self.kind, self.head_dim)


def quantize(x: torch.Tensor, cache: Cache, token_offset: int = 0, iters: int = 4,
             stream=None, flags: int = 0) -> None:
    """x [B, H, tokens, D] (bf16/fp32, channels contiguous) -> cache slots
    [token_offset, token_offset + tokens). flags: FLAG_NO_ROTATE."""
    if x.dim() != 4 or x.shape[3] != cache.head_dim or x.stride(3) != 1:
        raise ValueError("x must be [B, H, T, D] with contiguous channels, D the cache's "
                         "head_dim")
    if x.shape[0] != cache.batch or x.shape[1] != cache.kv_heads:
        raise ValueError("x batch/heads differ from the cache")
    d = cache.desc()
    dev = _on_device("quantize", x, cache.codes)
    st = load().kvarn_quantize_ex(x.data_ptr(), _dtype_code(x), x.stride(0), x.stride(1),
                                  x.stride(2), x.shape[2], token_offset, iters, flags,
                                  ctypes.byref(d), _stream(stream, dev))
    _raise(st, "kvarn_quantize")


def append(x: torch.Tensor, positions: torch.Tensor, cache: Cache, stream=None,
           flags: int = 0) -> None:
    """x [B, H, D] new tokens at positions [B] (int32, device). flags:
    FLAG_NO_ROTATE."""
    if x.dim() != 3 or tuple(x.shape) != (cache.batch, cache.kv_heads, cache.head_dim) or \
            not x.is_contiguous():
        raise ValueError("x must be contiguous [B, H, D] matching the cache")
    if positions.dtype != torch.int32 or positions.numel() != cache.batch or \
            not positions.is_contiguous():
        raise ValueError("positions must be contiguous int32 [B]")
    d = cache.desc()
    dev = _on_device("append", x, positions, cache.codes)
    st = load().kvarn_append_ex(x.data_ptr(), _dtype_code(x), positions.data_ptr(), flags,
                                ctypes.byref(d), _stream(stream, dev))
    _raise(st, "kvarn_append")


def append_kv(xk: torch.Tensor, xv: torch.Tensor, positions: torch.Tensor, k: Cache, v: Cache,
              stream=None, flags: int = 0) -> None:
    """append(xk, positions, k) and append(xv, positions, v) in one launch:
    xk, xv [B, H, D] of one dtype, k a K cache and v a V cache of one shape.
    flags: FLAG_NO_ROTATE."""
    if k.kind != K or v.kind != V:
        raise ValueError("append_kv takes a K cache and a V cache")
    if (k.batch, k.kv_heads, k.capacity, k.head_dim) != (v.batch, v.kv_heads, v.capacity,
                                                          v.head_dim):
        raise ValueError("append_kv: the K and V caches differ in shape")
    for x in (xk, xv):
        if x.dim() != 3 or tuple(x.shape) != (k.batch, k.kv_heads, k.head_dim) or \
                not x.is_contiguous():
            raise ValueError("xk and xv must be contiguous [B, H, D] matching the caches")
    if xk.dtype != xv.dtype:
        raise ValueError("xk and xv must have one dtype")
    if positions.dtype != torch.int32 or positions.numel() != k.batch or \
            not positions.is_contiguous():
        raise ValueError("positions must be contiguous int32 [B]")
    dk, dv = k.desc(), v.desc()
    dev = _on_device("append_kv", xk, xv, positions, k.codes, v.codes)
    st = load().kvarn_append_kv(xk.data_ptr(), xv.data_ptr(), _dtype_code(xk),
                                positions.data_ptr(), flags, ctypes.byref(dk), ctypes.byref(dv),
                                _stream(stream, dev))
    _raise(st, "kvarn_append_kv")


def append_window(batch: int, kv_heads: int, dtype=torch.bfloat16, device="cuda",
                  head_dim: int = HEAD_DIM) -> torch.Tensor:
    """A window for append_rebalance: [batch, kv_heads, 128, head_dim]."""
    return torch.zeros((batch, kv_heads, CHUNK, head_dim), dtype=dtype, device=device)


def append_rebalance(x: torch.Tensor, positions: torch.Tensor, cache: Cache,
                     window: torch.Tensor, iters: int = 4, stream=None, flags: int = 0) -> None:
    """append, plus the chunk re-quantized from `window` (same dtype as x,
    [B, H, 128, D], kept by the caller) when a token fills it. flags:
    FLAG_NO_ROTATE."""
    if x.dim() != 3 or tuple(x.shape) != (cache.batch, cache.kv_heads, cache.head_dim) or \
            not x.is_contiguous():
        raise ValueError("x must be contiguous [B, H, D] matching the cache")
    if positions.dtype != torch.int32 or positions.numel() != cache.batch or \
            not positions.is_contiguous():
        raise ValueError("positions must be contiguous int32 [B]")
    if tuple(window.shape) != (cache.batch, cache.kv_heads, CHUNK, cache.head_dim) or \
            window.dtype != x.dtype or not window.is_contiguous():
        raise ValueError("window must be contiguous [B, H, 128, D] of x's dtype")
    d = cache.desc()
    dev = _on_device("append_rebalance", x, positions, window, cache.codes)
    st = load().kvarn_append_rebalance(x.data_ptr(), _dtype_code(x), positions.data_ptr(),
                                       window.data_ptr(), iters, flags, ctypes.byref(d),
                                       _stream(stream, dev))
    _raise(st, "kvarn_append_rebalance")


def decode_workspace_bytes(batch: int, q_heads: int, capacity: int,
                           head_dim: int = HEAD_DIM) -> int:
    return int(load().kvarn_decode_workspace_bytes_ex(batch, q_heads, capacity, head_dim))


def decode_workspace(batch: int, q_heads: int, capacity: int, device="cuda",
                     head_dim: int = HEAD_DIM) -> torch.Tensor:
    """A decode workspace, zero-filled: its leading counters must be zero
    before the first call, and every call leaves them zero."""
    n = decode_workspace_bytes(batch, q_heads, capacity, head_dim)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def _decode_checks(what, q, k, v, seq_lens, out):
    D = k.head_dim
    if v.head_dim != D:
        raise ValueError(f"{what}: K and V caches differ in head_dim")
    if q.dim() != 3 or q.shape[2] != D or not q.is_contiguous():
        raise ValueError(f"{what}: q must be contiguous [B, Hq, D], D the caches' head_dim")
    if q.shape[0] != k.batch:
        raise ValueError(f"{what}: q's batch differs from the caches'")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != k.batch or \
            not seq_lens.is_contiguous():
        raise ValueError(f"{what}: seq_lens must be contiguous int32 [B]")
    if out is not None and (out.dtype != torch.float32 or not out.is_contiguous() or
                            tuple(out.shape) != (q.shape[0], q.shape[1], D)):
        raise ValueError(f"{what}: out must be contiguous fp32 [B, Hq, D]")
    return D


def decode_attn(q: torch.Tensor, k: Cache, v: Cache, seq_lens: torch.Tensor,
                out: torch.Tensor | None = None, softmax_scale: float | None = None,
                n_split: int = 0, workspace: torch.Tensor | None = None,
                stream=None, flags: int = 0) -> torch.Tensor:
    """q [B, Hq, D] -> out fp32 [B, Hq, D] (original basis; with
    FLAG_NO_ROTATE q and out are in the rotated basis). flags: FLAG_NO_ROTATE,
    FLAG_ONE_SCALE."""
    D = _decode_checks("decode_attn", q, k, v, seq_lens, out)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    B, Hq = q.shape[0], q.shape[1]
    kd, vd = k.desc(), v.desc()
    dev = _on_device("decode_attn", q, seq_lens, out, workspace, k.codes, v.codes)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = decode_workspace(B, Hq, k.capacity, dev, head_dim=D)
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    st = load().kvarn_decode_attn_ex(q.data_ptr(), _dtype_code(q), Hq, ctypes.byref(kd),
                                     ctypes.byref(vd), seq_lens.data_ptr(), softmax_scale,
                                     flags, out.data_ptr(), n_split, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(),
                                     _stream(stream, dev))
    _raise(st, "kvarn_decode_attn")
    return out


def decode_attn_noalloc(q: torch.Tensor, k: Cache, v: Cache, seq_lens: torch.Tensor,
                        out: torch.Tensor, softmax_scale: float | None = None, n_split: int = 0,
                        stream=None, flags: int = 0) -> torch.Tensor:
    """decode_attn without a workspace: the library keeps the split partials
    in its own fixed device array (NOALLOC_SCRATCH_BYTES per GPU) and the call
    allocates nothing, so `out` must be given. Calls that may overlap in time
    on one GPU race on that array."""
    if out is None:
        raise ValueError("decode_attn_noalloc: out must be given")
    D = _decode_checks("decode_attn_noalloc", q, k, v, seq_lens, out)
    Hq = q.shape[1]
    kd, vd = k.desc(), v.desc()
    dev = _on_device("decode_attn_noalloc", q, seq_lens, out, k.codes, v.codes)
    if softmax_scale is None:
        softmax_scale = D ** -0.5
    st = load().kvarn_decode_attn_noalloc(q.data_ptr(), _dtype_code(q), Hq, ctypes.byref(kd),
                                          ctypes.byref(vd), seq_lens.data_ptr(), softmax_scale,
                                          flags, out.data_ptr(), n_split, _stream(stream, dev))
    _raise(st, "kvarn_decode_attn_noalloc")
    return out


def token_error(x: torch.Tensor, cache: Cache, token_offset: int = 0, stream=None,
                flags: int = 0, ratio: torch.Tensor | None = None,
                cosine: torch.Tensor | None = None):
    """Per-token ||x_hat|| / ||x|| and cos(x_hat, x) of the cache's
    reconstruction of slots [token_offset, token_offset + T) against
    x [B, H, T, D] (bf16/fp32, channels contiguous). Returns (ratio,
    cosine), fp32 [B, H, T]. flags: FLAG_NO_ROTATE (x already rotated)."""
    if x.dim() != 4 or x.shape[3] != cache.head_dim or x.stride(3) != 1:
        raise ValueError("x must be [B, H, T, D] with contiguous channels, D the cache's "
                         "head_dim")
    if x.shape[0] != cache.batch or x.shape[1] != cache.kv_heads:
        raise ValueError("x batch/heads differ from the cache")
    shape = (x.shape[0], x.shape[1], x.shape[2])
    for name, t in (("ratio", ratio), ("cosine", cosine)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or
                              tuple(t.shape) != shape):
            raise ValueError(f"{name} must be contiguous fp32 [B, H, T] = {list(shape)}")
    d = cache.desc()
    dev = _on_device("token_error", x, ratio, cosine, cache.codes)
    if ratio is None:
        ratio = torch.empty(shape, dtype=torch.float32, device=dev)
    if cosine is None:
        cosine = torch.empty(shape, dtype=torch.float32, device=dev)
    st = load().kvarn_token_error(x.data_ptr(), _dtype_code(x), x.stride(0), x.stride(1),
                                  x.stride(2), x.shape[2], token_offset, flags, ctypes.byref(d),
                                  ratio.data_ptr(), cosine.data_ptr(), _stream(stream, dev))
    _raise(st, "kvarn_token_error")
    return ratio, cosine
