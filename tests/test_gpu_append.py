"""GPU parity of kvarn_append against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import SCALE_RTOL, U_TOL, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
def test_append_on_random_cache(kvarn, oracle, kind):
    """Both sides start from the same synthetic cache; one token per sequence
    at positions that open chunks, sit inside bytes, and fall outside."""
    B, H, cap = 6, 3, 512
    pos = [0, 5, 128, 130, 383, 512]       # the last one is outside -> skipped
    codes, row, col = kvgen.random_cache(21 + kind, B, H, cap)
    x = kvgen.new_tokens(3, 0, kind, B, H, 0.5, dtype=torch.bfloat16)
    gc = kvarn.Cache(codes.cuda(), row.cuda(), col.cuda(), kind)
    P = torch.tensor(pos, dtype=torch.int32)
    kvarn.append(x.cuda(), P.cuda(), gc)
    torch.cuda.synchronize()

    o_codes = oracle.unpack(codes.numpy(), kind=kind)
    o_rp = row.double().numpy().copy()
    o_c = col.double().numpy().copy()
    u = oracle.append(x.double().numpy(), pos, o_codes, o_rp, o_c)
    g_codes = oracle.unpack(gc.codes.cpu().numpy(), kind=kind)
    g_rp = gc.row_scale.cpu().double().numpy()
    g_c = gc.col_scale.cpu().double().numpy()
    for b, p in enumerate(pos):
        if p >= cap:
            assert np.array_equal(g_codes[b], oracle.unpack(codes.numpy(), kind=kind)[b])
            continue
        k = p // 128
        np.testing.assert_allclose(g_c[b, :, k], o_c[b, :, k], rtol=0, atol=0)  # exact copy / 1
        np.testing.assert_allclose(g_rp[b, :, p], o_rp[b, :, p], rtol=SCALE_RTOL)
        mism = g_codes[b, :, p] != o_codes[b, :, p]
        exempt = oracle.boundary_mask(u[b], U_TOL)
        assert not (mism & ~exempt).any(), (b, p)
        # everything else of the cache is unchanged, except (V) the three later
        # slots of the token's byte when the token starts a byte
        other = np.ones(cap, bool)
        other[p] = False
        if kind == kvgen.V and p % 4 == 0:
            later = np.arange(p + 1, min(p + 4, cap))
            other[later] = False
            assert np.all(g_codes[b, :, later] == 0)
        assert np.array_equal(g_codes[b, :, other], o_codes[b, :, other])
    log(f"[test] append kind={kind} ok")


def test_append_after_quantize_pipeline(kvarn, oracle):
    """Quantize 256 tokens, then append tokens 256..260 one step at a time
    (the first opens chunk 2 and copies chunk 1's column scales). Each side
    runs its own pipeline from the same inputs."""
    B, H, cap = 2, 2, 384
    x = kvgen.kv_tensor(4, 0, kvgen.K, B, H, 256, 0.5, dtype=torch.bfloat16)
    gc = kvarn.Cache.empty(B, H, cap, kvarn.K)
    kvarn.quantize(x.cuda(), gc)
    ora = oracle.quantize_tensor(x.double().numpy())
    o_codes = np.zeros((B, H, cap, 128), np.uint8)
    o_codes[:, :, :256] = ora["codes"]
    o_rp = np.zeros((B, H, cap))
    o_rp[:, :, :256] = ora["rp"]
    o_c = np.zeros((B, H, 3, 128))
    o_c[:, :, :2] = ora["c"]
    us = {}
    for step in range(5):
        t = kvgen.new_tokens(4, 0, kvgen.K, B, H, 0.5, step=step, dtype=torch.bfloat16)
        P = [256 + step] * B
        kvarn.append(t.cuda(), torch.tensor(P, dtype=torch.int32).cuda(), gc)
        us[256 + step] = oracle.append(t.double().numpy(), P, o_codes, o_rp, o_c)
    torch.cuda.synchronize()
    g_codes = oracle.unpack(gc.codes.cpu().numpy(), kind=kvarn.K)
    np.testing.assert_allclose(gc.col_scale.cpu().double().numpy(), o_c, rtol=SCALE_RTOL)
    np.testing.assert_allclose(gc.row_scale.cpu().double().numpy()[:, :, :261],
                               o_rp[:, :, :261], rtol=SCALE_RTOL)
    u_all = np.zeros((B, H, cap, 128))
    u_all[:, :, :256] = ora["u"]
    for p, u in us.items():
        u_all[:, :, p] = u
    mism = g_codes != o_codes
    assert not (mism & ~oracle.boundary_mask(u_all, U_TOL)).any()


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype,flags", [(torch.bfloat16, 0), (torch.float32, 0),
                                         (torch.bfloat16, 1)])
def test_append_kv_equals_two_appends(kvarn, D, dtype, flags):
    """kvarn_append_kv (K and V in one launch) leaves both caches bit for bit
    as kvarn_append_ex on K and then on V does: chunk openings, tokens inside
    and at the start of V bytes, and positions outside the cache (skipped)."""
    B, H, cap = 7, 3, 512
    pos = torch.tensor([0, 5, 128, 130, 383, 512, -1], dtype=torch.int32, device="cuda")
    caches = []
    for rep in range(2):
        kv_pair = []
        for kind in (kvgen.K, kvgen.V):
            codes, row, col = kvgen.random_cache(31 + kind, B, H, cap, head_dim=D)
            kv_pair.append(kvarn.Cache(codes.cuda(), row.cuda(), col.cuda(), kind))
        caches.append(kv_pair)
    xk = kvgen.new_tokens(5, 0, kvgen.K, B, H, 0.5, dtype=dtype, device="cuda", head_dim=D)
    xv = kvgen.new_tokens(5, 0, kvgen.V, B, H, 0.5, dtype=dtype, device="cuda", head_dim=D)
    (k1, v1), (k2, v2) = caches
    kvarn.append(xk, pos, k1, flags=flags)
    kvarn.append(xv, pos, v1, flags=flags)
    kvarn.append_kv(xk, xv, pos, k2, v2, flags=flags)
    torch.cuda.synchronize()
    for a, b in ((k1, k2), (v1, v2)):
        assert torch.equal(a.codes, b.codes)
        assert torch.equal(a.row_scale, b.row_scale)
        assert torch.equal(a.col_scale, b.col_scale)
    log(f"[test] append_kv D={D} dtype={dtype} flags={flags} ok")
