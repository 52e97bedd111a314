#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  for every layer: quantize K and V (all 128-token chunks), append one new
  token to each, and run one decode-attention step over the 2-bit cache.
(The Llama-3-8B-shaped workload quantizes its cache once, before timing, and
its step is append + decode per layer: steady-state decoding. Its step is
captured once in a HIP graph and the replays are timed: the GPU work per
layer (two appends, one decode) is shorter than the host's per-call launch
overhead, so eager launches would leave the GPU waiting on the host.)

Default workload: Qwen3-4B-shaped full cache (36 layers, batch 8, 8 kv-heads
x 128, 32768 tokens, 32 query heads), the largest of the workloads and the
one that does not fit in the 256 MB last-level cache.

Prints ONE JSON line. Per-kernel durations come from HIP events recorded on
the launch stream around every launch in the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantize GB/s (bf16 in) + 2-bit decode-attn tokens/s; % of HBM peak"
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, published
D, CHUNK = 128, 128
# algorithmic bytes per element of one quantize launch: 2 B bf16 in, 0.25 B
# codes, 4 B row scale per 128 channels, 4 B column scale per 128 tokens
QUANT_BYTES_PER_ELT_BF16 = 2.0 + 0.25 + 4.0 / 128 + 4.0 / 128
# MI355X fp32 vector peak, published: 256 CUs x 4 SIMDs x 32 lanes per clock
# x 2 flop per FMA x 2.4 GHz = 157.3 TFLOP/s. Plain (non-packed) v_fmac_f32
# reaches it too: a throughput probe of independent FMAs measured 120 TFLOP/s
# (DPP-sourced FMAs: 68-70).
VALU_F32_PEAK_TFLOPS = 256 * 4 * 32 * 2 * 2.4e9 / 1e12


def quant_flop_per_elt(iters: int) -> int:
    """Algorithmic fp32 operations per element of the quantizer: rotation 7
    add/sub, square 1, per balancing sweep a row and a column FMA (4 flop),
    scaling by 1/c 1, running |max| 1, code FMA 2, rounding 1."""
    return 7 + 1 + 4 * iters + 1 + 1 + 2 + 1


# algorithmic bytes per cached token per kv-head read by decode: 64 B codes
# (K and V), 8 B row scales, 8 B column scales amortized over the chunk
DECODE_BYTES_PER_TOKEN = 80.0


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", type=int, default=2,
                   help="index into kvgen.WORKLOADS (1..4; 2 = default)")
    p.add_argument("--iters", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-slices", type=int, default=0,
                   help="oracle slices for the CPU baseline (0 = 2 per thread)")
    p.add_argument("--no-ablations", action="store_true",
                   help="skip the ablation timings (balancing off, one scale, rotation off) "
                        "and the error diagnostics")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="one device-to-device copy of this many MiB before the warmup: "
                        "the reference kernel for calibrating HBM byte counters")
    return p.parse_args()


# Measured HBM traffic of a kernel: rocprofv3 FETCH_SIZE and WRITE_SIZE per
# dispatch, each scaled by the ratio that the same counter shows for a plain
# copy of known size (profiles/traffic.json, written from those runs). It is
# reported only while the kernel's sources are the ones that were profiled
# (their code: comments and layout are left out of the digest).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "quantize_block_kernel<bf16>": ["kv_cache_bit_kvarn_amd/csrc/kvarn_quantize.hip",
                                    "kv_cache_bit_kvarn_amd/csrc/kvarn_internal.h"],
    "decode_split_kernel + decode_combine_kernel": [
        "kv_cache_bit_kvarn_amd/csrc/kvarn_decode.hip",
        "kv_cache_bit_kvarn_amd/csrc/kvarn_internal.h"],
}


def sources_digest(kernel: str) -> str:
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter runs, or None when the
    kernel changed since (or was never profiled on this workload)."""
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f)[kernel][workload]
    except (OSError, KeyError, ValueError):
        return None
    if entry.get("sources_sha256") != sources_digest(kernel):
        return None
    return entry["hbm_bytes_per_launch"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path "
              "shards by sequence or kv-head with no exchange, so per-GPU throughput is "
              "the single-GPU figure. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_bit_kvarn_amd as kv
    import kvgen

    kv.load()
    wl = kvgen.WORKLOADS[args.workload]
    if args.workload == 0:
        sys.exit("workload 0 is the oracle-sized parity case, not a benchmark")
    steady = args.workload == 3           # cache built once; step = append + decode
    dev = torch.device("cuda:0")
    L, B, Hkv, Hq, T = wl.layers, wl.batch, wl.kv_heads, wl.q_heads, wl.tokens
    cap = T + CHUNK
    if steady and args.steps + args.warmup >= CHUNK:
        sys.exit("steady-state workload: steps + warmup must be < 128")

    log(f"[bench] workload {wl.name}: generating inputs on {dev} ...")
    t0 = time.time()
    xs, news, qs, caches = [], [], [], []
    for layer in range(L):
        xk = kvgen.kv_tensor(wl.seed, layer, kvgen.K, B, Hkv, T, wl.sigma, device=dev)
        xv = kvgen.kv_tensor(wl.seed, layer, kvgen.V, B, Hkv, T, wl.sigma, device=dev)
        xs.append((xk, xv))
        news.append((kvgen.new_tokens(wl.seed, layer, kvgen.K, B, Hkv, wl.sigma, device=dev),
                     kvgen.new_tokens(wl.seed, layer, kvgen.V, B, Hkv, wl.sigma, device=dev)))
        qs.append(kvgen.queries(wl.seed, layer, B, Hq, device=dev))
        caches.append((kv.Cache.empty(B, Hkv, cap, kv.K, device=dev),
                       kv.Cache.empty(B, Hkv, cap, kv.V, device=dev)))
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = kv.decode_workspace(B, Hq, cap, device=dev)
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s "
        f"({sum(x.numel() * 2 for p in xs for x in p) / 1e9:.2f} GB bf16 K/V)")

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    if steady:
        for layer in range(L):
            kv.quantize(xs[layer][0], caches[layer][0], iters=args.iters)
            kv.quantize(xs[layer][1], caches[layer][1], iters=args.iters)
        torch.cuda.synchronize()

    def step(i: int, rec: dict | None):
        p = (T + i) if steady else T
        pos = torch.full((B,), p, dtype=torch.int32, device=dev)
        lens = torch.full((B,), p + 1, dtype=torch.int32, device=dev)
        for layer in range(L):
            kc, vc = caches[layer]
            if not steady:
                for x, c in ((xs[layer][0], kc), (xs[layer][1], vc)):
                    if rec is not None:
                        a, b_ = ev(), ev()
                        a.record(stream)
                        kv.quantize(x, c, iters=args.iters, stream=stream)
                        b_.record(stream)
                        rec["quantize"].append((a, b_))
                    else:
                        kv.quantize(x, c, iters=args.iters, stream=stream)
            for n, c in ((news[layer][0], kc), (news[layer][1], vc)):
                if rec is not None:
                    a, b_ = ev(), ev()
                    a.record(stream)
                    kv.append(n, pos, c, stream=stream)
                    b_.record(stream)
                    rec["append"].append((a, b_))
                else:
                    kv.append(n, pos, c, stream=stream)
            if rec is not None:
                a, b_ = ev(), ev()
                a.record(stream)
            kv.decode_attn(qs[layer], kc, vc, lens, out=out, workspace=ws, stream=stream)
            if rec is not None:
                b_.record(stream)
                rec["decode"].append((a, b_))

    log(f"[bench] warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()

    rec = {"quantize": [], "append": [], "decode": []}
    if steady:
        ms_step, a_us, d_us = steady_graph_timing(kv, torch, args, caches, news, qs, out, ws, L, B, T)
        q_us = None
    else:
        log(f"[bench] timing {args.steps} steps")
        start, end = ev(), ev()
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            step(args.warmup + i, rec)
        end.record(stream)
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)
        ms_step = total_ms / args.steps

        def avg_us(name):
            v = [a.elapsed_time(b_) * 1e3 for a, b_ in rec[name]]
            return (sum(v) / len(v)) if v else None

        q_us, a_us, d_us = avg_us("quantize"), avg_us("append"), avg_us("decode")
    elts_per_quant = B * Hkv * T * D
    q_launches = 0 if steady else 2 * L
    bf16_bytes_step = q_launches * elts_per_quant * 2
    # tokens attended per decode: the graph-timed decodes of the steady-state
    # workload run after the timed steps, over T + warmup + steps + 1 tokens
    dec_tokens = (T + args.warmup + args.steps + 1) if steady else (T + 1)
    dec_bytes = DECODE_BYTES_PER_TOKEN * dec_tokens * B * Hkv + B * Hq * D * (2 + 4)
    decode_ms_step = L * d_us / 1e3

    res = {
        "metric": METRIC,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "batch": B, "kv_heads": Hkv,
                   "q_heads": Hq, "head_dim": D, "tokens": T, "chunk": CHUNK,
                   "balancing_iters": args.iters, "input_dtype": "bf16",
                   "token_scale_sigma": wl.sigma,
                   "step": "append+decode per layer" if steady else
                           "quantize K,V + append + decode per layer"},
    }
    dec = {"tokens_per_s": round(B / (decode_ms_step / 1e3), 1),
           "us_per_launch": round(d_us, 2), "launches_per_step": L,
           "GBps_algorithmic": round(dec_bytes / (d_us * 1e-6) / 1e9, 1),
           "hbm_frac": round(dec_bytes / (d_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "kernels": "decode_split_kernel + decode_combine_kernel"}
    dec_roof = {"bound": "hbm", "achieved": dec["GBps_algorithmic"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": dec["hbm_frac"],
                "traffic": measured_traffic(dec["kernels"], wl.name),
                "kernel": dec["kernels"], "bytes_per_launch": dec_bytes}
    if steady:
        res["value"] = dec["tokens_per_s"]
        res["unit"] = "tokens/s (decode attention, all layers)"
        res["step_tokens_per_s"] = round(B / (ms_step / 1e3), 1)
        res["roofline"] = dec_roof
    else:
        qbytes = QUANT_BYTES_PER_ELT_BF16 * elts_per_quant
        q_gbps = qbytes / (q_us * 1e-6) / 1e9
        res["value"] = round(bf16_bytes_step / (ms_step / 1e3) / 1e9, 2)
        res["unit"] = "GB/s (bf16 K/V in, whole quantize+append+decode step)"
        res["quantize"] = {"GBps_bf16_in": round(elts_per_quant * 2 / (q_us * 1e-6) / 1e9, 1),
                           "us_per_launch": round(q_us, 2), "launches_per_step": q_launches,
                           "GBps_algorithmic": round(q_gbps, 1),
                           "hbm_frac": round(q_gbps / HBM_PEAK_GBPS, 4)}
        # roofline of the quantizer: the larger of its ideal HBM time (bytes at
        # the HBM peak) and its ideal ALU time (algorithmic fp32 operations at
        # the VALU peak) names the bound; the other resource stays beside it
        q_flop = quant_flop_per_elt(args.iters) * elts_per_quant
        q_tflops = q_flop / (q_us * 1e-6) / 1e12
        t_hbm = qbytes / (HBM_PEAK_GBPS * 1e9)
        t_alu = q_flop / (VALU_F32_PEAK_TFLOPS * 1e12)
        alu = {"achieved": round(q_tflops, 2), "peak": round(VALU_F32_PEAK_TFLOPS, 2),
               "unit": "TFLOP/s", "frac": round(q_tflops / VALU_F32_PEAK_TFLOPS, 4),
               "flop_per_element": quant_flop_per_elt(args.iters)}
        hbm = {"achieved": round(q_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
               "frac": round(q_gbps / HBM_PEAK_GBPS, 4)}
        bound, main, other = ("hbm", hbm, alu) if t_hbm >= t_alu else ("alu", alu, dict(hbm))
        res["roofline"] = {"bound": bound, **main,
                           "traffic": measured_traffic("quantize_block_kernel<bf16>", wl.name),
                           "kernel": "quantize_block_kernel<bf16>",
                           "elements_per_launch": elts_per_quant,
                           "bytes_per_launch": qbytes,
                           "ideal_us": {"hbm": round(t_hbm * 1e6, 2), "alu": round(t_alu * 1e6, 2)},
                           ("alu" if bound == "hbm" else "hbm"): other}
        res["roofline_decode"] = dec_roof
    res["decode"] = dec
    res["append"] = {"us_per_launch": round(a_us, 2), "launches_per_step": 2 * L}
    if not args.no_ablations:
        res["ablations"] = ablations(kv, torch, stream, xs[0], qs[0], caches[0], ws, out,
                                     T + (args.warmup + args.steps if steady else 1), args.iters)
        res["error_diagnostics"] = error_diagnostics(kv, torch, stream, xs[0], caches[0],
                                                     args.iters)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, wl, xs, news, qs, steady, res["unit"],
                                           bf16_bytes_step, cap)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def error_diagnostics(kv, torch, stream, x_pair, cache_pair, iters):
    """Magnitude vs direction of the quantization error on layer 0 (outside
    the timed step): each token's squared error relative to ||x||^2 splits
    exactly into (rho - 1)^2 (magnitude, rho = ||x_hat|| / ||x||) and
    2 rho (1 - cos) (direction). Means over all tokens of K and V, quantized
    with the balancing and without it, through kvarn_token_error."""
    res = {}
    for name, x, cache in (("K", x_pair[0], cache_pair[0]), ("V", x_pair[1], cache_pair[1])):
        scratch = kv.Cache.empty(cache.batch, cache.kv_heads, cache.capacity, cache.kind,
                                 device=x.device)
        for it in (iters, 0):
            kv.quantize(x, scratch, iters=it, stream=stream)
            ratio, cosine = kv.token_error(x, scratch, stream=stream)
            torch.cuda.synchronize()
            r, c = ratio.double(), cosine.double()
            res[f"{name}_iters_{it}"] = {
                "magnitude": round(float(((r - 1) ** 2).mean()), 6),
                "direction": round(float((2 * r * (1 - c)).mean()), 6),
                "mean_ratio": round(float(r.mean()), 5),
                "mean_cos": round(float(c.mean()), 5)}
        del scratch
    res["note"] = ("per-token squared error / ||x||^2 = magnitude + direction; means over "
                   "layer 0's tokens")
    return res


def ablations(kv, torch, stream, x_pair, q, cache_pair, ws, out, length, iters, reps=20,
              rounds=3):
    """Layer-0 launches timed with HIP events outside the timed step:
    the quantizer with and without balancing (iters vs 0: the cost of the
    dual-scaling normalization), decode with both scales and with the column
    scales taken as 1 (the cost of the second scale), and decode with the
    rotation absorbed into the weights (no query rotation, no output
    un-rotation). The variants are timed in turn, `rounds` times over, and
    each reports the median of its rounds: the shader clock moves by several
    percent within a second of a change of load, which one short run per
    variant, always in the same order, would take for a difference between
    the variants. Scratch caches keep the benchmark's caches intact."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    xk = x_pair[0]
    kc, vc = cache_pair
    scratch = kv.Cache.empty(kc.batch, kc.kv_heads, kc.capacity, kv.K, device=xk.device)
    lens = torch.full((kc.batch,), length, dtype=torch.int32, device=xk.device)

    def dec(flags):
        return lambda: kv.decode_attn(q, kc, vc, lens, out=out, workspace=ws, stream=stream,
                                      flags=flags)
    variants = {
        "q_full": lambda: kv.quantize(xk, scratch, iters=iters, stream=stream),
        "q_none": lambda: kv.quantize(xk, scratch, iters=0, stream=stream),
        "q_norot": lambda: kv.quantize(xk, scratch, iters=iters, stream=stream,
                                       flags=kv.FLAG_NO_ROTATE),
        "d_two": dec(0),
        "d_one": dec(kv.FLAG_ONE_SCALE),
        "d_norot": dec(kv.FLAG_NO_ROTATE),
    }
    times = {k: [] for k in variants}
    for _ in range(rounds):
        for k, fn in variants.items():
            times[k].append(timed(fn))
    del scratch
    t = {k: sorted(v)[len(v) // 2] for k, v in times.items()}
    return {
        "quantize_us": {f"iters_{iters}": round(t["q_full"], 2), "iters_0": round(t["q_none"], 2),
                        "no_rotate": round(t["q_norot"], 2),
                        "balancing_share": round((t["q_full"] - t["q_none"]) / t["q_full"], 4)},
        "decode_us": {"two_scales": round(t["d_two"], 2), "one_scale": round(t["d_one"], 2),
                      "no_rotate": round(t["d_norot"], 2),
                      "second_scale_overhead": round((t["d_two"] - t["d_one"]) / t["d_one"], 4)},
        "note": f"layer 0, K tensor for quantize; HIP events over {reps} launches after one "
                f"warm launch; variants timed in turn, median of {rounds} rounds",
    }


def steady_graph_timing(kv, torch, args, caches, news, qs, out, ws, L, B, T):
    """Steady-state decoding timed on HIP-graph replays (torch.cuda.CUDAGraph).

    G_step holds one step: for every layer, append K and V at pos, decode over
    lens; then pos and lens advance by one, so each replay is the next step.
    G_dec holds the L decodes alone and G_app the 2 L appends alone (at a fixed
    position, so replaying them rewrites the same slots); their replays give
    the per-launch times. The positions continue from the eager warmup steps.
    Returns (ms per step, us per append, us per decode)."""
    dev = out.device
    pos = torch.full((B,), T + args.warmup, dtype=torch.int32, device=dev)
    lens = pos + 1
    torch.cuda.synchronize()

    def layer_appends(layer):
        kc, vc = caches[layer]
        kv.append(news[layer][0], pos, kc)
        kv.append(news[layer][1], pos, vc)

    def layer_decode(layer):
        kc, vc = caches[layer]
        kv.decode_attn(qs[layer], kc, vc, lens, out=out, workspace=ws)

    g_step, g_dec, g_app = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        for layer in range(L):
            layer_appends(layer)
            layer_decode(layer)
        pos.add_(1)
        lens.add_(1)
    with torch.cuda.graph(g_dec):
        for layer in range(L):
            layer_decode(layer)
    with torch.cuda.graph(g_app):
        for layer in range(L):
            layer_appends(layer)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def timed(g, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n  # ms per replay

    log(f"[bench] timing {args.steps} steps (HIP graph replays)")
    ms_step = timed(g_step, args.steps)
    reps = max(args.steps, 10)
    d_us = timed(g_dec, reps) * 1e3 / L
    a_us = timed(g_app, reps) * 1e3 / (2 * L)
    return ms_step, a_us, d_us


def cpu_baseline(args, wl, xs, news, qs, steady, unit, bf16_bytes_step, cap):
    """The oracle (fp64 C, unmodified) timed on this host's cores on a bounded
    sample of the same step: whole (layer 0, sequence b, kv-head g) slices --
    quantize all chunks of K and V, append the new token, decode the group's
    query heads -- run one slice per thread, then scaled to the full step."""
    import numpy as np

    import oracle

    oracle.lib()
    threads = max(1, min(16, os.cpu_count() or 1))
    n = args.cpu_slices or 2 * threads
    B, Hkv, Hq, T = wl.batch, wl.kv_heads, wl.q_heads, wl.tokens
    G = Hq // Hkv
    rng = np.random.default_rng(0)
    pairs = [(int(rng.integers(B)), int(rng.integers(Hkv))) for _ in range(n)]
    inputs = []
    for b, g in pairs:
        xk = xs[0][0][b:b + 1, g:g + 1].double().cpu().numpy()
        xv = xs[0][1][b:b + 1, g:g + 1].double().cpu().numpy()
        nk = news[0][0][b:b + 1, g:g + 1].double().cpu().numpy()
        nv = news[0][1][b:b + 1, g:g + 1].double().cpu().numpy()
        q = qs[0][b:b + 1, g * G:(g + 1) * G].double().cpu().numpy()
        inputs.append((xk, xv, nk, nv, q))

    def one(item):
        xk, xv, nk, nv, q = item
        outs = []
        for x, nt in ((xk, nk), (xv, nv)):
            o = oracle.quantize_tensor(x, iters=args.iters, want_u=False)
            codes = np.zeros((1, 1, cap, D), np.uint8)
            rp = np.zeros((1, 1, cap))
            c = np.zeros((1, 1, cap // CHUNK, D))
            codes[:, :, :T], rp[:, :, :T], c[:, :, :T // CHUNK] = o["codes"], o["rp"], o["c"]
            oracle.append(nt, [T], codes, rp, c)
            outs.append((codes, rp, c))
        oracle.decode_attn(q, *outs[0], *outs[1], [T + 1])

    work = list(inputs)
    lock = threading.Lock()

    def worker():
        while True:
            with lock:
                if not work:
                    return
                item = work.pop()
            one(item)

    log(f"[bench] cpu baseline: {n} slices on {threads} threads ...")
    t0 = time.perf_counter()
    ts = [threading.Thread(target=worker) for _ in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    wall = time.perf_counter() - t0
    slices_per_step = wl.layers * B * Hkv
    step_s = wall * slices_per_step / n
    if steady:
        value = B / step_s
    else:
        value = bf16_bytes_step / step_s / 1e9
    return {"value": round(value, 6), "unit": unit, "cores": threads, "kind": "oracle",
            "wall_s": round(wall, 2),
            "sample": f"{n} whole (layer 0, seq, kv-head) slices of the step "
                      f"(quantize {2 * T // CHUNK} chunks of K+V incl. the oracle's "
                      f"O(D^2) rotation, append 1 token each, decode {G} query heads over "
                      f"{T + 1} tokens), {threads} threads, scaled by "
                      f"{slices_per_step}/{n} to the full step"}


if __name__ == "__main__":
    main()
