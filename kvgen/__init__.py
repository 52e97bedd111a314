"""Seeded synthetic K/V/Q inputs for the KVarN quantizer and its decode step.

This module only draws random numbers with the value structure the pages
describe; it holds none of the method's arithmetic and is shared by the
oracle-side and the GPU-side of every test (and by bench.py).

Value structure (stands in for the Qwen3-4B / Llama-3-8B K/V caches of the
pages' experiments, which need weights and datasets that are not used here):
  X[b,h,t,j] = s[b,h,t] * g[b,h,t,j] * (20 if j in O[layer,h,tensor] else 1)
  g ~ N(0,1) i.i.d.                  -- base values
  O = 4 channels drawn without replacement per (layer, kv-head, tensor),
      shared over batch and tokens   -- the channel outliers the rotation
                                        spreads out (rndamp article, "How It
                                        Works", item 1)
  s = exp(sigma * n), n ~ N(0,1) per (b, h, t)  -- token-scale spread that the
                                        dual scaling targets ("How It Works",
                                        item 2; "The Problem")
  Q ~ N(0,1).
Streams are keyed by (config seed, layer, tensor) so that every tensor is
reproducible on its own.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

HEAD_DIM = 128
CHUNK = 128
N_OUTLIERS = 4
OUTLIER_GAIN = 20.0


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    kv_heads: int
    q_heads: int
    tokens: int
    sigma: float
    dtype: torch.dtype
    seed: int
    head_dim: int = HEAD_DIM


# The five workloads, in order: tiny oracle case; one Qwen3-4B-shaped layer;
# Qwen3-4B-shaped full cache; Llama-3-8B-shaped decode (cache of 8192 tokens,
# then one appended token per step); long-horizon stress case.
WORKLOADS = [
    Workload("tiny-1L-1kvh-256tok-fp32", 1, 1, 1, 4, 256, 0.5, torch.float32, 0),
    Workload("qwen3-4b-1L-b1-32k", 1, 1, 8, 32, 32768, 0.5, torch.bfloat16, 1),
    Workload("qwen3-4b-36L-b8-32k", 36, 8, 8, 32, 32768, 0.5, torch.bfloat16, 2),
    Workload("llama3-8b-32L-b32-8k-append", 32, 32, 8, 32, 8192, 0.5,
             torch.bfloat16, 3),
    Workload("stress-1L-b64-128k-sigma1", 1, 64, 8, 32, 131072, 1.0,
             torch.bfloat16, 4),
]

K, V = 0, 1


def _stream_seed(seed: int, layer: int, tensor: int, salt: int = 0) -> int:
    return (seed * 1_000_003 + layer * 10_007 + tensor * 101 + salt * 7) & 0x7FFFFFFF


def outlier_channels(seed: int, layer: int, tensor: int, heads: int,
                     head_dim: int = HEAD_DIM) -> torch.Tensor:
    """[heads, N_OUTLIERS] channel indices (CPU generator, so identical on
    every device)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(_stream_seed(seed, layer, tensor, salt=1))
    return torch.stack([torch.randperm(head_dim, generator=g)[:N_OUTLIERS]
                        for _ in range(heads)])


def kv_tensor(seed: int, layer: int, tensor: int, batch: int, heads: int,
              tokens: int, sigma: float, dtype: torch.dtype = torch.bfloat16,
              device="cpu", head_dim: int = HEAD_DIM,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense [batch, heads, tokens, head_dim] K or V with the structure above.
    Generated one sequence at a time to bound temporary memory."""
    device = torch.device(device)
    if out is None:
        out = torch.empty((batch, heads, tokens, head_dim), dtype=dtype,
                          device=device)
    gain = torch.ones((heads, head_dim), dtype=torch.float32)
    idx = outlier_channels(seed, layer, tensor, heads, head_dim)
    gain.scatter_(1, idx, OUTLIER_GAIN)
    gain = gain.to(device)[:, None, :]
    g = torch.Generator(device=device)
    g.manual_seed(_stream_seed(seed, layer, tensor))
    for b in range(batch):
        base = torch.randn((heads, tokens, head_dim), generator=g, device=device,
                           dtype=torch.float32)
        n = torch.randn((heads, tokens, 1), generator=g, device=device,
                        dtype=torch.float32)
        base.mul_(torch.exp(sigma * n)).mul_(gain)
        out[b].copy_(base.to(dtype))
        del base, n
    return out


def queries(seed: int, layer: int, batch: int, q_heads: int,
            dtype: torch.dtype = torch.bfloat16, device="cpu",
            head_dim: int = HEAD_DIM, salt: int = 0) -> torch.Tensor:
    """[batch, q_heads, head_dim] ~ N(0,1)."""
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_stream_seed(seed, layer, 2, salt=3 + salt))
    return torch.randn((batch, q_heads, head_dim), generator=g,
                       device=torch.device(device), dtype=torch.float32).to(dtype)


def new_tokens(seed: int, layer: int, tensor: int, batch: int, heads: int,
               sigma: float, step: int = 0, dtype: torch.dtype = torch.bfloat16,
               device="cpu", head_dim: int = HEAD_DIM) -> torch.Tensor:
    """[batch, heads, head_dim]: one decoding step's new K or V (same value
    structure and outlier channels as the cache of that layer)."""
    device = torch.device(device)
    gain = torch.ones((heads, head_dim), dtype=torch.float32)
    gain.scatter_(1, outlier_channels(seed, layer, tensor, heads, head_dim),
                  OUTLIER_GAIN)
    g = torch.Generator(device=device)
    g.manual_seed(_stream_seed(seed, layer, tensor, salt=11 + step))
    base = torch.randn((batch, heads, head_dim), generator=g, device=device)
    n = torch.randn((batch, heads, 1), generator=g, device=device)
    return (base * torch.exp(sigma * n) * gain.to(device)).to(dtype)


def random_cache(seed: int, batch: int, heads: int, capacity: int,
                 device="cpu", head_dim: int = HEAD_DIM, chunk: int = CHUNK,
                 sigma: float = 0.5):
    """A synthetic packed cache with uniformly random code bytes, log-normal
    row scales and column scales around 1, for testing the decode step on its
    own. Returns (codes u8 [B,H,cap/chunk,chunk*D/4], row f32 [B,H,cap],
    col f32 [B,H,cap/chunk,D])."""
    g = torch.Generator(device="cpu")
    g.manual_seed(_stream_seed(seed, 0, 3, salt=5))
    nch = capacity // chunk
    codes = torch.randint(0, 256, (batch, heads, nch, chunk * head_dim // 4),
                          generator=g, dtype=torch.int32).to(torch.uint8)
    row = torch.exp(sigma * torch.randn((batch, heads, capacity), generator=g))
    col = torch.exp(0.25 * torch.randn((batch, heads, nch, head_dim), generator=g))
    dev = torch.device(device)
    return codes.to(dev), row.float().to(dev), col.float().to(dev)
