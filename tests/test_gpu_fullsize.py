"""Parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times: whole-tensor quantize launches, one-token
appends, and decode over the whole cache with the library's own split count.
Sampled blocks and sampled (sequence, kv-head) groups are recomputed by the
oracle; for attention and append the oracle is fed the GPU-produced cache, so
boundary-exempt code flips cannot leak into the comparison."""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import (ATTN_RL2, SCALE_RTOL, assert_quant_parity, cache_blocks, log, rel_l2,
                      sample_blocks, x_blocks)

pytestmark = pytest.mark.gpu

CH = 128


def _group_cache(oracle, cache, kind, b, g):
    """Unpacked codes [1,1,cap,D], rp [1,1,cap], c [1,1,cap/128,D] of one group."""
    codes = oracle.unpack(cache.codes[b:b + 1, g:g + 1].cpu().numpy(), kind=kind)
    rp = cache.row_scale[b:b + 1, g:g + 1].double().cpu().numpy()
    c = cache.col_scale[b:b + 1, g:g + 1].double().cpu().numpy()
    return codes, rp, c


def _check_decode_groups(oracle, q, kc, vc, lens, out, groups, G, what):
    for b, g in groups:
        k = _group_cache(oracle, kc, kvgen.K, b, g)
        v = _group_cache(oracle, vc, kvgen.V, b, g)
        want = oracle.decode_attn(q[b:b + 1, g * G:(g + 1) * G].double().cpu().numpy(), *k, *v,
                                  [int(lens[b])])
        err = rel_l2(out[b:b + 1, g * G:(g + 1) * G].cpu().numpy(), want)
        log(f"  {what} decode (b={b}, kv-head={g}, len={int(lens[b])}): rel L2 {err:.3e}")
        assert err <= ATTN_RL2


def _check_quant_sampled(oracle, x, cache, kind, n, seed, what):
    B, H, T, _ = x.shape
    nch = T // CH
    sel = sample_blocks(np.random.default_rng(seed), B, H, nch, n,
                        always=[(0, 0, 0), (B - 1, H - 1, nch - 1)])
    ora = oracle.quantize_tensor(x_blocks(x, sel), threads=8)
    st = assert_quant_parity(oracle, ora, *cache_blocks(cache, kind, sel), what)
    log(f"  {what}: {st}")


def _check_append(oracle, kvarn, x_new, cache_before, cache_after, kind, pos, groups, what):
    """The appended token (codes, r', and the chunk's c when it opens) against
    the oracle's append onto the GPU's cache state before the step."""
    for b, g in groups:
        codes, rp, c = cache_before
        codes, rp, c = (np.ascontiguousarray(a[b:b + 1, g:g + 1]) for a in (codes, rp, c))
        xo = x_new[b:b + 1, g:g + 1].double().cpu().numpy()
        oracle.append(xo, [pos], codes, rp, c)
        got_codes, got_rp, got_c = _group_cache(oracle, cache_after, kind, b, g)
        k = pos // CH
        np.testing.assert_allclose(got_c[0, 0, k], c[0, 0, k], rtol=SCALE_RTOL, atol=0,
                                   err_msg=f"{what}: chunk scales")
        np.testing.assert_allclose(got_rp[0, 0, pos], rp[0, 0, pos], rtol=SCALE_RTOL, atol=0,
                                   err_msg=f"{what}: row scale")
        # codes: exact away from rounding boundaries (u recomputed in fp64)
        y = oracle.rotate(xo[0, 0])
        u = y / (rp[0, 0, pos] * c[0, 0, k]) if rp[0, 0, pos] > 0 else np.zeros_like(y)
        ok = (got_codes[0, 0, pos] == codes[0, 0, pos]) | oracle.boundary_mask(u)
        assert ok.all(), f"{what}: appended codes differ at {np.flatnonzero(~ok)[:8]}"


def _host_state(cache, groups):
    """Host copies (all groups, unpacked lazily by the caller) of a cache."""
    return (cache.codes.clone(), cache.row_scale.clone(), cache.col_scale.clone())


def _unpacked(oracle, state, kind, groups):
    codes_p, rp, c = state
    B, H = codes_p.shape[:2]
    out_codes, out_rp, out_c = {}, {}, {}
    cap = codes_p.shape[2] * CH
    codes = np.zeros((B, H, cap, 128), np.uint8)
    rp_np = np.zeros((B, H, cap))
    c_np = np.zeros((B, H, codes_p.shape[2], 128))
    for b, g in groups:
        codes[b, g] = oracle.unpack(codes_p[b:b + 1, g:g + 1].cpu().numpy(), kind=kind)[0, 0]
        rp_np[b, g] = rp[b, g].double().cpu().numpy()
        c_np[b, g] = c[b, g].double().cpu().numpy()
    return codes, rp_np, c_np


def test_bench_default_layer(kvarn, oracle):
    """One layer of the default benchmark workload (batch 8, 8 kv-heads,
    32768 tokens, 32 query heads, capacity 32768 + 128): quantize K and V,
    append one token at position 32768, decode over 32769 tokens."""
    wl = kvgen.WORKLOADS[2]
    B, H, Hq, T = wl.batch, wl.kv_heads, wl.q_heads, wl.tokens
    G = Hq // H
    cap = T + CH
    log(f"[test] full-size {wl.name} layer 0")
    caches = {}
    for kind in (kvgen.K, kvgen.V):
        x = kvgen.kv_tensor(wl.seed, 0, kind, B, H, T, wl.sigma, device="cuda")
        cache = kvarn.Cache.empty(B, H, cap, kind, device="cuda")
        kvarn.quantize(x, cache)
        torch.cuda.synchronize()
        _check_quant_sampled(oracle, x, cache, kind, 96, 10 + kind, f"{wl.name} quantize")
        del x
        caches[kind] = cache
    groups = [(0, 0), (B - 1, H - 1), (3, 5)]
    pos = torch.full((B,), T, dtype=torch.int32, device="cuda")
    for kind in (kvgen.K, kvgen.V):
        x_new = kvgen.new_tokens(wl.seed, 0, kind, B, H, wl.sigma, device="cuda")
        before = _unpacked(oracle, _host_state(caches[kind], groups), kind, groups)
        kvarn.append(x_new, pos, caches[kind])
        torch.cuda.synchronize()
        _check_append(oracle, kvarn, x_new, before, caches[kind], kind, T, groups,
                      f"{wl.name} append kind={kind}")
    q = kvgen.queries(wl.seed, 0, B, Hq, device="cuda")
    lens = torch.full((B,), T + 1, dtype=torch.int32, device="cuda")
    out = kvarn.decode_attn(q, caches[kvgen.K], caches[kvgen.V], lens)
    torch.cuda.synchronize()
    _check_decode_groups(oracle, q, caches[kvgen.K], caches[kvgen.V], lens.cpu(), out, groups, G,
                         wl.name)


def test_llama_steady_state(kvarn, oracle):
    """The steady-state workload (batch 32, 8 kv-heads, 8192 tokens, 32
    query heads): quantize once, then three decoding steps of append + decode;
    the first append opens chunk 64 (column scales copied from chunk 63)."""
    wl = kvgen.WORKLOADS[3]
    B, H, Hq, T = wl.batch, wl.kv_heads, wl.q_heads, wl.tokens
    G = Hq // H
    cap = T + CH
    log(f"[test] full-size {wl.name}")
    caches = {}
    for kind in (kvgen.K, kvgen.V):
        x = kvgen.kv_tensor(wl.seed, 0, kind, B, H, T, wl.sigma, device="cuda")
        caches[kind] = kvarn.Cache.empty(B, H, cap, kind, device="cuda")
        kvarn.quantize(x, caches[kind])
        torch.cuda.synchronize()
        _check_quant_sampled(oracle, x, caches[kind], kind, 64, 20 + kind, f"{wl.name} quantize")
        del x
    groups = [(0, 0), (B - 1, H - 1), (17, 2)]
    q = kvgen.queries(wl.seed, 0, B, Hq, device="cuda")
    for step in range(3):
        p = T + step
        pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
        for kind in (kvgen.K, kvgen.V):
            x_new = kvgen.new_tokens(wl.seed, 0, kind, B, H, wl.sigma, step=step, device="cuda")
            before = _unpacked(oracle, _host_state(caches[kind], groups), kind, groups)
            kvarn.append(x_new, pos, caches[kind])
            torch.cuda.synchronize()
            _check_append(oracle, kvarn, x_new, before, caches[kind], kind, p, groups,
                          f"{wl.name} step {step} kind={kind}")
        lens = torch.full((B,), p + 1, dtype=torch.int32, device="cuda")
        out = kvarn.decode_attn(q, caches[kvgen.K], caches[kvgen.V], lens)
        torch.cuda.synchronize()
        _check_decode_groups(oracle, q, caches[kvgen.K], caches[kvgen.V], lens.cpu(), out,
                             groups, G, f"{wl.name} step {step}")


def test_long_horizon_stress(kvarn, oracle):
    """The stress workload (batch 64, 8 kv-heads, 131072 tokens, token scales
    log-normal with sigma 1.0): quantize both tensors in one launch each,
    decode over the whole cache with ragged lengths."""
    wl = kvgen.WORKLOADS[4]
    B, H, Hq, T = wl.batch, wl.kv_heads, wl.q_heads, wl.tokens
    G = Hq // H
    log(f"[test] full-size {wl.name}")
    caches = {}
    for kind in (kvgen.K, kvgen.V):
        x = kvgen.kv_tensor(wl.seed, 0, kind, B, H, T, wl.sigma, device="cuda")
        caches[kind] = kvarn.Cache.empty(B, H, T, kind, device="cuda")
        kvarn.quantize(x, caches[kind])
        torch.cuda.synchronize()
        _check_quant_sampled(oracle, x, caches[kind], kind, 64, 30 + kind, f"{wl.name} quantize")
        del x
        torch.cuda.empty_cache()
    q = kvgen.queries(wl.seed, 0, B, Hq, device="cuda")
    lens_h = torch.full((B,), T, dtype=torch.int32)
    lens_h[1] = 1
    lens_h[2] = T - 77
    lens_h[3] = 129
    out = kvarn.decode_attn(q, caches[kvgen.K], caches[kvgen.V], lens_h.cuda())
    torch.cuda.synchronize()
    _check_decode_groups(oracle, q, caches[kvgen.K], caches[kvgen.V], lens_h, out,
                         [(0, 0), (1, 3), (2, 7), (3, 1), (B - 1, H - 1)], G, wl.name)
