"""A seeded random sweep over combinations the listed cases do not spell out:
head size, K or V, input dtype, balancing iterations, batch, kv-heads, chunk
count and chunk offset for quantize; head size, group size, capacity,
per-sequence lengths, split count and query dtype for decode attention. Each
case is checked against the oracle at the same bars as the listed cases
(codes and scales: assert_quant_parity; attention: ATTN_RL2)."""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import ATTN_RL2, assert_quant_parity, log, rel_l2
from test_gpu_headdim import _caches, _oracle_decode

pytestmark = pytest.mark.gpu


def _quant_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128, 256]))
        kind = int(rng.integers(0, 2))
        f32 = bool(rng.integers(0, 2))
        iters = int(rng.integers(0, 6))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        T, off = 128 * int(rng.integers(1, 5)), 128 * int(rng.integers(0, 3))
        cases.append((i, D, kind, f32, iters, B, H, T, off))
    return cases


def _decode_cases(n=24, seed=4048):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128, 256]))
        B, Hkv, G = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 9))
        nch = int(rng.integers(1, 25))
        cap = 128 * nch
        lens = [int(rng.integers(1, cap + 1)) for _ in range(B)]
        if i % 3 == 0:
            lens[0] = cap
        n_split = 0 if i % 2 == 0 else int(rng.integers(1, 4 * nch + 9))
        f32 = bool(rng.integers(0, 2))
        cases.append((i, D, B, Hkv, G, cap, lens, n_split, f32))
    return cases


@pytest.mark.parametrize("case", _quant_cases(), ids=lambda c: f"q{c[0]}")
def test_quantize_random_sweep(kvarn, oracle, case):
    i, D, kind, f32, iters, B, H, T, off = case
    log(f"[test] sweep quantize i={i} D={D} kind={kind} f32={f32} iters={iters} "
        f"B={B} H={H} T={T} offset={off}")
    dtype = torch.float32 if f32 else torch.bfloat16
    x = kvgen.kv_tensor(500 + i, 0, kind, B, H, T, 0.5, dtype=dtype, head_dim=D)
    cache = kvarn.Cache.empty(B, H, T + off, kind, device="cuda", head_dim=D)
    kvarn.quantize(x.cuda(), cache, token_offset=off, iters=iters)
    torch.cuda.synchronize()
    ora = oracle.quantize_tensor(x.double().numpy(), iters=iters)
    g = oracle.unpack(cache.codes.cpu().numpy(), D=D, kind=kind)[:, :, off:]
    st = assert_quant_parity(oracle, ora, g, cache.row_scale.cpu().numpy()[:, :, off:],
                             cache.col_scale.cpu().numpy()[:, :, off // 128:], f"sweep q{i}")
    if off:
        assert np.all(cache.codes.cpu().numpy()[:, :, :off // 128] == 0)  # chunks before untouched
    log(f"  {st}")


@pytest.mark.parametrize("case", _decode_cases(), ids=lambda c: f"d{c[0]}")
def test_decode_random_sweep(kvarn, oracle, case):
    i, D, B, Hkv, G, cap, lens, n_split, f32 = case
    log(f"[test] sweep decode i={i} D={D} B={B} Hkv={Hkv} G={G} cap={cap} lens={lens} "
        f"n_split={n_split} f32={f32}")
    kc, vc, hk, hv = _caches(kvarn, B, Hkv, cap, D, seed=700 + i)
    q = kvgen.queries(701 + i, 0, B, Hkv * G, dtype=torch.float32 if f32 else torch.bfloat16,
                      head_dim=D)
    L = torch.tensor(lens, dtype=torch.int32).cuda()
    out = kvarn.decode_attn(q.cuda(), kc, vc, L, n_split=n_split)
    torch.cuda.synchronize()
    err = rel_l2(out.cpu().numpy(), _oracle_decode(oracle, q, hk, hv, lens, D))
    log(f"  rel L2 {err:.3e}")
    assert err <= ATTN_RL2
