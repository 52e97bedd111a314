"""Helpers shared by the GPU parity tests: run the library through its C ABI,
bring results to the host, compare with the oracle at the stated bars:
  codes   bit-exact except elements whose oracle pre-rounding value lies
          within 1e-5 of a rounding boundary (the decision is taken in fp64 by
          the oracle and in fp32 by the kernel);
  scales  within 1e-5 relative error (fp32 vs fp64);
  attention output within 2e-3 relative L2 over the whole output of a call.
"""
import sys

import numpy as np
import torch

U_TOL = 1e-5
SCALE_RTOL = 1e-5
ATTN_RL2 = 2e-3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_l2(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


def assert_quant_parity(oracle, ora, g_codes, g_rp, g_c, what=""):
    """ora: oracle.quantize_tensor output (unpacked codes, u, rp, c);
    g_codes: GPU codes unpacked by the oracle's unpack; g_rp, g_c: fp32."""
    mism = g_codes != ora["codes"]
    exempt = oracle.boundary_mask(ora["u"], U_TOL)
    bad = mism & ~exempt
    assert not bad.any(), (f"{what}: {int(bad.sum())} code mismatches away from a "
                           f"rounding boundary; first at {np.argwhere(bad)[:5].tolist()}")
    rp_o = ora["rp"]
    np.testing.assert_allclose(np.asarray(g_rp, np.float64), rp_o, rtol=SCALE_RTOL, atol=0,
                               err_msg=f"{what}: row scales")
    np.testing.assert_allclose(np.asarray(g_c, np.float64), ora["c"], rtol=SCALE_RTOL,
                               atol=0, err_msg=f"{what}: column scales")
    return dict(elements=int(mism.size), boundary=int(exempt.sum()), flipped=int(mism.sum()))


def cache_blocks(cache, kind, sel):
    """Selected blocks of a GPU cache as oracle-shaped arrays. sel: list of
    (b, h, chunk). Returns codes [1, n, 128, D] (unpacked by the oracle),
    rp [1, n, 128], c [1, n, 1, D] (D = the cache's head size)."""
    import oracle
    b = torch.tensor([s[0] for s in sel])
    h = torch.tensor([s[1] for s in sel])
    k = torch.tensor([s[2] for s in sel])
    dev = cache.codes.device
    packed = cache.codes[b.to(dev), h.to(dev), k.to(dev)].cpu().numpy()
    rows = cache.row_scale.view(cache.batch, cache.kv_heads, -1, 128)
    rp = rows[b.to(dev), h.to(dev), k.to(dev)].cpu().numpy()
    c = cache.col_scale[b.to(dev), h.to(dev), k.to(dev)].cpu().numpy()
    codes = oracle.unpack(packed[None, :, None, :], D=cache.head_dim, kind=kind)
    return codes, rp[None], c[None, :, None, :]


def x_blocks(x, sel):
    """Blocks of a [B, H, T, D] tensor as an oracle input [1, n, 128, D]."""
    dev = x.device
    b = torch.tensor([s[0] for s in sel], device=dev)
    h = torch.tensor([s[1] for s in sel], device=dev)
    k = torch.tensor([s[2] for s in sel], device=dev)
    xs = x.view(x.shape[0], x.shape[1], -1, 128, x.shape[3])[b, h, k]
    return xs.double().cpu().numpy()[None]


def sample_blocks(rng, B, H, nch, n, always=()):
    sel = set(always)
    while len(sel) < min(n, B * H * nch):
        sel.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(nch))))
    return sorted(sel)
