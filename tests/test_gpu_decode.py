"""GPU parity of kvarn_decode_attn (and of the quantize -> decode pipeline)
against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import ATTN_RL2, log, rel_l2

pytestmark = pytest.mark.gpu


def _random_caches(kv, B, Hkv, cap, seed):
    ck, rk, colk = kvgen.random_cache(seed, B, Hkv, cap)
    cv, rv, colv = kvgen.random_cache(seed + 1000, B, Hkv, cap)
    kc = kv.Cache(ck.cuda(), rk.cuda(), colk.cuda(), kv.K)
    vc = kv.Cache(cv.cuda(), rv.cuda(), colv.cuda(), kv.V)
    return kc, vc, (ck, rk, colk), (cv, rv, colv)


def _oracle_on(oracle, q, host_k, host_v, lens, scale=None):
    ck, rk, colk = host_k
    cv, rv, colv = host_v
    return oracle.decode_attn(q.double().cpu().numpy(),
                              oracle.unpack(ck.numpy(), kind=0), rk.double().numpy(),
                              colk.double().numpy(), oracle.unpack(cv.numpy(), kind=1),
                              rv.double().numpy(), colv.double().numpy(), lens, scale)


@pytest.mark.parametrize("B,Hkv,G,cap,lens", [
    (2, 2, 4, 512, [512, 300]),
    (3, 1, 1, 384, [1, 129, 384]),
    (1, 2, 8, 256, [200]),
    (2, 3, 3, 256, [256, 255]),
])
def test_decode_random_cache(kvarn, oracle, B, Hkv, G, cap, lens):
    log(f"[test] decode random cache B={B} Hkv={Hkv} G={G} cap={cap} lens={lens}")
    kc, vc, hk, hv = _random_caches(kvarn, B, Hkv, cap, seed=B * 100 + G)
    q = kvgen.queries(11, 0, B, Hkv * G, dtype=torch.bfloat16)
    L = torch.tensor(lens, dtype=torch.int32)
    out = kvarn.decode_attn(q.cuda(), kc, vc, L.cuda())
    torch.cuda.synchronize()
    want = _oracle_on(oracle, q, hk, hv, lens)
    err = rel_l2(out.cpu().numpy(), want)
    log(f"  rel L2 {err:.3e}")
    assert err <= ATTN_RL2


def test_decode_splits_agree(kvarn):
    """Split-KV with one split and with many give the same result (log-sum-exp
    merge), up to fp32 reassociation."""
    kc, vc, _, _ = _random_caches(kvarn, 2, 2, 2048, seed=3)
    q = kvgen.queries(12, 0, 2, 8, device="cuda")
    L = torch.tensor([2048, 1000], dtype=torch.int32, device="cuda")
    outs = [kvarn.decode_attn(q, kc, vc, L, n_split=n) for n in (1, 3, 16, 0)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert rel_l2(o.cpu().numpy(), outs[0].cpu().numpy()) < 1e-5


def test_decode_many_splits_merge_in_rounds(kvarn, oracle):
    """Many workgroups per row: the last one merges the row's partials in
    rounds of 16 with a running maximum (n_split 33, 64, 68, 80: 9, 16, 17
    and 20 workgroups, one, one, two and two rounds, the second with one
    and with four partials). Every split count agrees with one split, and
    with the oracle, over a cache of 80 chunks with a ragged last chunk."""
    cap = 80 * 128
    kc, vc, hk, hv = _random_caches(kvarn, 2, 1, cap, seed=5)
    q = kvgen.queries(14, 0, 2, 4, dtype=torch.bfloat16)
    lens = [cap, cap - 77]
    L = torch.tensor(lens, dtype=torch.int32, device="cuda")
    outs = [kvarn.decode_attn(q.cuda(), kc, vc, L, n_split=n) for n in (1, 33, 64, 68, 80)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert rel_l2(o.cpu().numpy(), outs[0].cpu().numpy()) < 1e-5
    err = rel_l2(outs[2].cpu().numpy(), _oracle_on(oracle, q, hk, hv, lens))
    log(f"[test] decode 64 splits over 80 chunks: rel L2 {err:.3e}")
    assert err <= ATTN_RL2


def test_decode_invalid_lengths_give_zero(kvarn):
    kc, vc, _, _ = _random_caches(kvarn, 3, 1, 256, seed=4)
    q = kvgen.queries(13, 0, 3, 4, device="cuda")
    L = torch.tensor([0, 257, 10], dtype=torch.int32, device="cuda")
    out = kvarn.decode_attn(q, kc, vc, L)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.all(out[1] == 0)
    assert torch.all(torch.isfinite(out[2])) and out[2].abs().sum() > 0


def test_pipeline_tiny_fp32(kvarn, oracle):
    """Tiny oracle case end to end: quantize K and V (fp32, 256 tokens), one
    decode step with 4 query heads. GPU pipeline vs oracle pipeline; each side
    uses its own cache."""
    wl = kvgen.WORKLOADS[0]
    xk = kvgen.kv_tensor(wl.seed, 0, kvgen.K, 1, 1, 256, wl.sigma, dtype=torch.float32)
    xv = kvgen.kv_tensor(wl.seed, 0, kvgen.V, 1, 1, 256, wl.sigma, dtype=torch.float32)
    q = kvgen.queries(wl.seed, 0, 1, 4, dtype=torch.float32)
    kc = kvarn.Cache.empty(1, 1, 256, kvarn.K)
    vc = kvarn.Cache.empty(1, 1, 256, kvarn.V)
    kvarn.quantize(xk.cuda(), kc)
    kvarn.quantize(xv.cuda(), vc)
    for n in (256, 200, 1):
        L = torch.tensor([n], dtype=torch.int32)
        out = kvarn.decode_attn(q.cuda(), kc, vc, L.cuda())
        torch.cuda.synchronize()
        ok = oracle.quantize_tensor(xk.double().numpy(), want_u=False)
        ov = oracle.quantize_tensor(xv.double().numpy(), want_u=False)
        want = oracle.decode_attn(q.double().numpy(), ok["codes"], ok["rp"], ok["c"],
                                  ov["codes"], ov["rp"], ov["c"], [n])
        err = rel_l2(out.cpu().numpy(), want)
        log(f"[test] pipeline tiny len={n}: rel L2 {err:.3e}")
        assert err <= ATTN_RL2


def test_pipeline_qwen_layer_sampled_heads(kvarn, oracle):
    """One Qwen3-4B-shaped layer (batch 1, 8 kv-heads, 32 query heads, 32768
    tokens): GPU quantize + decode in the launch shapes of the benchmark;
    the oracle recomputes two kv-heads (8 query heads) from the same inputs."""
    wl = kvgen.WORKLOADS[1]
    xk = kvgen.kv_tensor(wl.seed, 0, kvgen.K, 1, 8, wl.tokens, wl.sigma, device="cuda")
    xv = kvgen.kv_tensor(wl.seed, 0, kvgen.V, 1, 8, wl.tokens, wl.sigma, device="cuda")
    q = kvgen.queries(wl.seed, 0, 1, 32, device="cuda")
    kc = kvarn.Cache.empty(1, 8, wl.tokens, kvarn.K)
    vc = kvarn.Cache.empty(1, 8, wl.tokens, kvarn.V)
    kvarn.quantize(xk, kc)
    kvarn.quantize(xv, vc)
    L = torch.tensor([wl.tokens], dtype=torch.int32, device="cuda")
    out = kvarn.decode_attn(q, kc, vc, L)
    torch.cuda.synchronize()
    for g in (0, 5):
        ok = oracle.quantize_tensor(xk[:, g:g + 1].double().cpu().numpy(), want_u=False,
                                    threads=8)
        ov = oracle.quantize_tensor(xv[:, g:g + 1].double().cpu().numpy(), want_u=False,
                                    threads=8)
        want = oracle.decode_attn(q[:, 4 * g:4 * g + 4].double().cpu().numpy(), ok["codes"],
                                  ok["rp"], ok["c"], ov["codes"], ov["rp"], ov["c"],
                                  [wl.tokens])
        err = rel_l2(out[:, 4 * g:4 * g + 4].cpu().numpy(), want)
        log(f"[test] qwen layer kv-head {g}: rel L2 {err:.3e}")
        assert err <= ATTN_RL2


def test_decode_last_workgroup_merge_resets_counters(kvarn, oracle):
    """Many workgroups per row: the workgroup that finishes a row last merges
    its partials (here 20 per row); it leaves the row's counter at zero, so a
    second call on the same workspace gives the same output."""
    B, Hkv, G, cap = 2, 2, 8, 128 * 80
    kc, vc, hk, hv = _random_caches(kvarn, B, Hkv, cap, seed=77)
    q = kvgen.queries(78, 0, B, Hkv * G, dtype=torch.bfloat16)
    lens = [cap, 5000]
    L = torch.tensor(lens, dtype=torch.int32).cuda()
    ws = kvarn.decode_workspace(B, Hkv * G, cap)
    a = kvarn.decode_attn(q.cuda(), kc, vc, L, n_split=80, workspace=ws).clone()
    b = kvarn.decode_attn(q.cuda(), kc, vc, L, n_split=80, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert int(ws[:B * Hkv * G * 4].view(torch.int32).abs().sum()) == 0
    err = rel_l2(a.cpu().numpy(), _oracle_on(oracle, q, hk, hv, lens))
    log(f"[test] decode 20 workgroups per row: rel L2 {err:.3e}")
    assert err <= ATTN_RL2
