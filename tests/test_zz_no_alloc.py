"""kvarn_decode_attn_noalloc (the allocation-free decode entry point, for
callers that cannot allocate device memory) against kvarn_decode_attn_ex on
the same inputs: bit-identical outputs, since both run the same kernels with
the same split count, on two calls in a row, the second with a smaller
input (the library's array keeps the first call's partials), plus the
oracle at the attention bar, and the size limit."""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import ATTN_RL2, log, rel_l2

pytestmark = pytest.mark.gpu


def _case(kv, oracle, B, Hkv, G, cap, lens, seed, n_split=0, flags=0):
    ck, rk, colk = kvgen.random_cache(seed, B, Hkv, cap)
    cv, rv, colv = kvgen.random_cache(seed + 1, B, Hkv, cap)
    kc = kv.Cache(ck.cuda(), rk.cuda(), colk.cuda(), kv.K)
    vc = kv.Cache(cv.cuda(), rv.cuda(), colv.cuda(), kv.V)
    q = kvgen.queries(seed + 2, 0, B, Hkv * G, device="cuda")
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ref = kv.decode_attn(q, kc, vc, ln, n_split=n_split, flags=flags)
    got = torch.full_like(ref, float("nan"))
    kv.decode_attn_noalloc(q, kc, vc, ln, got, n_split=n_split, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "noalloc output differs from the workspace entry point"
    if not flags:
        want = oracle.decode_attn(q.double().cpu().numpy(), oracle.unpack(ck.numpy(), kind=0),
                                  rk.double().numpy(), colk.double().numpy(),
                                  oracle.unpack(cv.numpy(), kind=1), rv.double().numpy(),
                                  colv.double().numpy(), lens)
        err = rel_l2(got.cpu().numpy(), want)
        log(f"[test] noalloc B={B} Hkv={Hkv} G={G} cap={cap}: rel L2 {err:.3e}")
        assert err <= ATTN_RL2
    return got


def test_noalloc_matches_workspace_call(kvarn, oracle):
    # a larger call, then a smaller one that reuses the array with fewer partials
    _case(kvarn, oracle, 4, 4, 4, 2048, [2048, 1, 777, 1500], seed=301)
    _case(kvarn, oracle, 2, 2, 8, 512, [300, 512], seed=311)
    # explicit split counts and the flag variants
    _case(kvarn, oracle, 3, 2, 4, 1024, [1024, 129, 0], seed=321, n_split=3)
    _case(kvarn, oracle, 2, 2, 4, 1024, [1000, 640], seed=331, flags=kvarn.FLAG_ONE_SCALE)


def test_noalloc_size_limit(kvarn):
    """Partials beyond the fixed array are refused before any launch."""
    B, Hkv, G, cap = 64, 8, 8, 128 * 64
    need = B * Hkv * G * 64 * 130 * 4
    assert need > kvarn.NOALLOC_SCRATCH_BYTES
    kc = kvarn.Cache.empty(B, Hkv, cap, kvarn.K, device="cuda")
    vc = kvarn.Cache.empty(B, Hkv, cap, kvarn.V, device="cuda")
    q = torch.zeros((B, Hkv * G, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B, Hkv * G, 128), dtype=torch.float32, device="cuda")
    ln = torch.full((B,), cap, dtype=torch.int32, device="cuda")
    with pytest.raises(kvarn.KvarnError) as e:
        kvarn.decode_attn_noalloc(q, kc, vc, ln, out, n_split=64)
    assert e.value.status == kvarn.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 0)
