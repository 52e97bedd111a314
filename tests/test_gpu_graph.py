"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph): a
serving loop's step -- quantize a chunk, append one token per sequence to K
and V, one decode step, advance the positions -- replayed several times with
eager work and synchronizations between the replays. Every replay must equal
the same step run eagerly, bit for bit (same kernels on the same inputs; with
`fused` the graph appends K and V in one launch, which codes them exactly as
the two separate appends of the eager step do)."""
import pytest
import torch

import kvgen
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,fused", [(128, False), (64, False), (256, False), (128, True)])
def test_graph_replays_match_eager(kvarn, D, fused):
    B, H, Hq, T, cap = 3, 2, 8, 384, 640
    dev = torch.device("cuda")
    xk = kvgen.kv_tensor(31, 0, kvgen.K, B, H, T, 0.5, device=dev, head_dim=D)
    xv = kvgen.kv_tensor(31, 0, kvgen.V, B, H, T, 0.5, device=dev, head_dim=D)
    xq = kvgen.kv_tensor(32, 0, kvgen.K, B, H, 128, 0.5, device=dev, head_dim=D)  # quantized in the step
    steps = 3
    nks = [kvgen.new_tokens(33 + i, 0, kvgen.K, B, H, 0.5, device=dev, head_dim=D)
           for i in range(steps)]
    nvs = [kvgen.new_tokens(33 + i, 0, kvgen.V, B, H, 0.5, device=dev, head_dim=D)
           for i in range(steps)]
    qs = [kvgen.queries(40 + i, 0, B, Hq, device=dev, head_dim=D) for i in range(steps)]

    def fresh_caches():
        kc = kvarn.Cache.empty(B, H, cap, kvarn.K, device=dev, head_dim=D)
        vc = kvarn.Cache.empty(B, H, cap, kvarn.V, device=dev, head_dim=D)
        kvarn.quantize(xk, kc)
        kvarn.quantize(xv, vc)
        return kc, vc

    # eager reference: the three steps one after the other
    kc_e, vc_e = fresh_caches()
    qc_e = kvarn.Cache.empty(B, H, 128, kvarn.K, device=dev, head_dim=D)
    ws_e = kvarn.decode_workspace(B, Hq, cap, device=dev, head_dim=D)
    outs_e, caches_e = [], []
    for i in range(steps):
        pos = torch.full((B,), T + i, dtype=torch.int32, device=dev)
        lens = pos + 1
        kvarn.quantize(xq, qc_e)
        kvarn.append(nks[i], pos, kc_e)       # the eager reference appends K and V apart
        kvarn.append(nvs[i], pos, vc_e)
        outs_e.append(kvarn.decode_attn(qs[i], kc_e, vc_e, lens, workspace=ws_e).clone())
        caches_e.append([t.clone() for c in (kc_e, vc_e) for t in (c.codes, c.row_scale, c.col_scale)])
    torch.cuda.synchronize()

    # the same step, captured once
    kc, vc = fresh_caches()
    qc = kvarn.Cache.empty(B, H, 128, kvarn.K, device=dev, head_dim=D)
    ws = kvarn.decode_workspace(B, Hq, cap, device=dev, head_dim=D)
    nk, nv, q = nks[0].clone(), nvs[0].clone(), qs[0].clone()
    pos = torch.full((B,), T, dtype=torch.int32, device=dev)
    lens = pos + 1
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvarn.quantize(xq, qc)
        if fused:
            kvarn.append_kv(nk, nv, pos, kc, vc)
        else:
            kvarn.append(nk, pos, kc)
            kvarn.append(nv, pos, vc)
        kvarn.decode_attn(q, kc, vc, lens, out=out, workspace=ws)
        pos.add_(1)
        lens.add_(1)
    torch.cuda.synchronize()
    # capture ran nothing: the caches are still the freshly quantized ones
    for i in range(steps):
        nk.copy_(nks[i])
        nv.copy_(nvs[i])
        q.copy_(qs[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(pos[0]) == T + i + 1
        assert torch.equal(out, outs_e[i]), f"replay {i}: decode output differs from eager"
        got = [t for c in (kc, vc) for t in (c.codes, c.row_scale, c.col_scale)]
        for a, b_ in zip(got, caches_e[i]):
            assert torch.equal(a, b_), f"replay {i}: cache differs from eager"
        assert torch.equal(qc.codes, qc_e.codes) and torch.equal(qc.row_scale, qc_e.row_scale) \
            and torch.equal(qc.col_scale, qc_e.col_scale), f"replay {i}: quantized chunk differs"
        # eager work on the same stream between replays
        torch.cuda.synchronize()
        _ = (out * 2).sum().item()
    log("[test] graph replays match eager")
