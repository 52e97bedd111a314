"""GPU parity of the alternative append semantics (kvarn_append_rebalance).
Tokens enter the cache as with kvarn_append (SC-11). When a token fills its
chunk, the chunk equals the oracle's block quantization of the 128 appended
tokens. The next chunk then opens with the re-balanced column scales, and the
oracle's append replayed from those agrees. Sequences fill their chunks at
different steps (steps with position -1 are skipped); a sequence that never
fills a chunk matches plain kvarn_append exactly. The error of a closed chunk
is logged against SC-11's."""
import numpy as np
import pytest
import torch

import kvgen
from gpu_util import SCALE_RTOL, assert_quant_parity, log

pytestmark = pytest.mark.gpu

STEPS = 150
SKIPS = {0: (), 1: tuple(range(20, 30)), 2: tuple(range(0, 40))}  # steps skipped per sequence


def _unpacked(oracle, cache, kind):
    return (oracle.unpack(cache.codes.cpu().numpy(), kind=kind),
            cache.row_scale.double().cpu().numpy(), cache.col_scale.double().cpu().numpy())


def _run(kvarn, kind, dtype, B=3, H=2, cap=256, oracle=None, flags=0):
    """With KVARN_FLAG_NO_ROTATE the tokens are handed over rotated (rounded to
    `dtype` after an fp64 rotation), and `hist` keeps the oracle input that
    reproduces exactly what the GPU read: the scaled rotation is its own
    inverse."""
    cache = kvarn.Cache.empty(B, H, cap, kind, device="cuda")
    plain = kvarn.Cache.empty(B, H, cap, kind, device="cuda")
    window = kvarn.append_window(B, H, dtype=dtype)
    count = [0] * B
    hist = {}          # (b, position) -> token [H, D] (fp64 copy of what the GPU read)
    for step in range(STEPS):
        x = kvgen.new_tokens(61, 0, kind, B, H, 0.5, step=step, dtype=dtype, device="cuda")
        if flags & kvarn.FLAG_NO_ROTATE:
            xr = oracle.rotate(x.double().cpu().numpy())
            x = torch.from_numpy(xr).to(dtype).cuda()
            xs = oracle.rotate(x.double().cpu().numpy())
        else:
            xs = x.double().cpu().numpy()
        pos = np.full(B, -1, np.int32)
        for b in range(B):
            if step not in SKIPS[b]:
                pos[b] = count[b]
                hist[(b, count[b])] = xs[b]
                count[b] += 1
        p = torch.from_numpy(pos).cuda()
        kvarn.append_rebalance(x, p, cache, window, flags=flags)
        kvarn.append(x, p, plain, flags=flags)
    torch.cuda.synchronize()
    return cache, plain, hist, count


@pytest.mark.parametrize("kind", [kvgen.K, kvgen.V])
@pytest.mark.parametrize("dtype,no_rotate", [(torch.float32, False), (torch.bfloat16, False),
                                             (torch.bfloat16, True)])
def test_rebalance_at_close(kvarn, oracle, kind, dtype, no_rotate):
    flags = kvarn.FLAG_NO_ROTATE if no_rotate else 0
    cache, plain, hist, count = _run(kvarn, kind, dtype, oracle=oracle, flags=flags)
    assert count == [150, 140, 110]
    codes, rp, c = _unpacked(oracle, cache, kind)
    pc, prp, pcs = _unpacked(oracle, plain, kind)
    for b in (0, 1):   # closed chunk 0
        xs = np.stack([hist[(b, t)] for t in range(128)], axis=1)  # [H, 128, D]
        ora = oracle.quantize_tensor(xs[None])
        st = assert_quant_parity(oracle, ora, codes[b:b + 1, :, :128], rp[b:b + 1, :, :128],
                                 c[b:b + 1, :, :1], f"closed chunk b={b}")
        # the open chunk 1: SC-11 from the re-balanced column scales
        n1 = count[b] - 128
        codes1 = np.zeros((1, codes.shape[1], 256, 128), np.uint8)
        rp1 = np.zeros((1, codes.shape[1], 256))
        c1 = np.ones((1, codes.shape[1], 2, 128))
        c1[0, :, 0] = c[b, :, 0]
        for t in range(128, 128 + n1):
            oracle.append(hist[(b, t)][None], [t], codes1, rp1, c1)
        np.testing.assert_allclose(c[b, :, 1], c1[0, :, 1], rtol=SCALE_RTOL, atol=0)
        np.testing.assert_allclose(rp[b, :, 128:128 + n1], rp1[0, :, 128:128 + n1],
                                   rtol=SCALE_RTOL, atol=0)
        mism = codes[b, :, 128:128 + n1] != codes1[0, :, 128:128 + n1]
        for h in range(codes.shape[1]):
            for i in range(n1):
                if mism[h, i].any():
                    y = oracle.rotate(hist[(b, 128 + i)][h])
                    u = y / (rp1[0, h, 128 + i] * c1[0, h, 1])
                    assert oracle.boundary_mask(u)[mism[h, i]].all()
        # error of the closed chunk: re-balanced vs frozen column scales
        x_t = torch.from_numpy(oracle.rotate(xs[None]) if no_rotate else xs[None]).to(dtype).cuda()
        sub = lambda cc: kvarn.Cache(cc.codes[b:b + 1], cc.row_scale[b:b + 1],  # noqa: E731
                                     cc.col_scale[b:b + 1], kind)
        r1, q1 = kvarn.token_error(x_t, sub(cache), flags=flags)
        r0, q0 = kvarn.token_error(x_t, sub(plain), flags=flags)
        e1 = float(((r1 - 1) ** 2 + 2 * r1 * (1 - q1)).mean())
        e0 = float(((r0 - 1) ** 2 + 2 * r0 * (1 - q0)).mean())
        log(f"[test] rebalance kind={kind} {dtype} no_rotate={no_rotate} b={b}: {st}; "
            f"relative squared error "
            f"re-balanced {e1:.5f}, frozen c (SC-11) {e0:.5f}")
    # sequence 2 never filled a chunk: identical to the plain append
    assert np.array_equal(codes[2], pc[2])
    assert np.array_equal(rp[2], prp[2])
    assert np.array_equal(c[2], pcs[2])
