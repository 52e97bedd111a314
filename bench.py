#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  quantize K and V of every layer (all 128-token chunks), then, layer by
  layer, append one new token to K and V (one launch for both) and run one
  decode-attention step over the 2-bit cache.
Quantizing every layer before the first decode keeps each decode reading a
cache that was written more than 256 MB earlier: the 256 MB memory-side cache
(MALL) holds none of it, so every reported decode time is an HBM time.
(The Llama-3-8B-shaped workload quantizes its cache once, before timing, and
its step is append + decode per layer: steady-state decoding. Its step is
captured once in a HIP graph and the replays are timed: the GPU work per
layer (one K+V append, one decode) is shorter than the host's per-call
launch overhead, so eager launches would leave the GPU waiting on the host.)

Default workload: Qwen3-4B-shaped full cache (36 layers, batch 8, 8 kv-heads
x 128, 32768 tokens, 32 query heads). The same JSON line also carries the
Llama-3-8B-shaped steady-state decode and the long-horizon stress shape as
sub-results (`workloads`), measured after the timed step.

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
MALL_BYTES = 256 << 20           # MI355X memory-side last-level cache
D, CHUNK = 128, 128
# algorithmic bytes per element of one quantize launch: 2 B bf16 in, 0.25 B
# codes, 4 B row scale per 128 channels, 4 B column scale per 128 tokens
QUANT_BYTES_PER_ELT_BF16 = 2.0 + 0.25 + 4.0 / 128 + 4.0 / 128
# MI355X fp32 vector peak, published: 256 CUs x 4 SIMDs x 32 lanes per clock
# x 2 flop per FMA x 2.4 GHz = 157.3 TFLOP/s, which counts packed (two-wide)
# fp32 instructions. The kernels here are built without packed fp32 (it is
# switched off in the build), and a throughput probe measures a wave64
# non-packed fp32 instruction (fma, mul, add, DPP-sourced add, cvt_pk_u8)
# at 4.2 cycles of its SIMD, i.e. 16 lanes per clock: 78.6 TFLOP/s for FMAs.
VALU_F32_PEAK_TFLOPS = 256 * 4 * 32 * 2 * 2.4e9 / 1e12
VALU_F32_NONPACKED_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
# the machine's CPU share for one GPU: worker pools stay within it
HOST_THREAD_CAP = 16

QUANT_ARITH = ("rotation: bf16 x (+-1) products on the matrix cores with fp32 accumulation "
               "(exact for bf16 input); balancing, range step and code decision: fp32 VALU")
DECODE_ARITH = ("scaled MFMA f8f6f4: 2-bit cache codes as fp4 e2m1 operands; query*c_K as "
                "4 fp8 e4m3 terms (~16 significant bits), p*r'_V as 3 fp8 e4m3 terms (~12 bits), "
                "per-head power-of-two range scales; fp32 accumulation; online softmax, "
                "split merge and inverse rotation in fp32")

# the pages' own figure (rndamp.com article on KVarN, section "Numbers"):
# 1.9 ms of variance normalization against 1050 ms of token generation for
# Qwen3-4B on an unnamed GPU; batch, length and call count are not stated
PAGES_NORMALIZATION_MS = 1.9
PAGES_GENERATION_MS = 1050.0


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
    p.add_argument("--no-subworkloads", action="store_true",
                   help="skip the Llama-3-8B steady-state and stress sub-results")
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
    "decode_kernel": [
        "kv_cache_bit_kvarn_amd/csrc/kvarn_decode.hip",
        "kv_cache_bit_kvarn_amd/csrc/kvarn_internal.h"],
}
DECODE_KERNELS = "decode_kernel"


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


def decode_bytes(tokens: int, B: int, Hkv: int, Hq: int) -> float:
    """Algorithmic bytes of one decode call: the cache stream plus q and out."""
    return DECODE_BYTES_PER_TOKEN * tokens * B * Hkv + B * Hq * D * (2 + 4)


def hbm_entry(nbytes: float, us: float) -> dict:
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"GBps_algorithmic": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}


def timed_events(torch, stream, fns):
    """HIP events on `stream` around each call of fns; returns microseconds."""
    evs = []
    for fn in fns:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


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
        if steady:
            xs.append(None)
        else:
            xs.append((kvgen.kv_tensor(wl.seed, layer, kvgen.K, B, Hkv, T, wl.sigma, device=dev),
                       kvgen.kv_tensor(wl.seed, layer, kvgen.V, B, Hkv, T, wl.sigma, device=dev)))
        news.append((kvgen.new_tokens(wl.seed, layer, kvgen.K, B, Hkv, wl.sigma, device=dev),
                     kvgen.new_tokens(wl.seed, layer, kvgen.V, B, Hkv, wl.sigma, device=dev)))
        qs.append(kvgen.queries(wl.seed, layer, B, Hq, device=dev))
        caches.append((kv.Cache.empty(B, Hkv, cap, kv.K, device=dev),
                       kv.Cache.empty(B, Hkv, cap, kv.V, device=dev)))
    if steady:
        build_steady_caches(kv, kvgen, torch, wl, caches, args.iters, dev)
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
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(i: int):
        """One untimed (warmup) step, launched eagerly."""
        p = (T + i) if steady else T
        pos = torch.full((B,), p, dtype=torch.int32, device=dev)
        lens = torch.full((B,), p + 1, dtype=torch.int32, device=dev)
        if not steady:
            for layer in range(L):
                for x, c in ((xs[layer][0], caches[layer][0]), (xs[layer][1], caches[layer][1])):
                    kv.quantize(x, c, iters=args.iters, stream=stream)
        for layer in range(L):
            kc, vc = caches[layer]
            kv.append_kv(news[layer][0], news[layer][1], pos, kc, vc, stream=stream)
            kv.decode_attn(qs[layer], kc, vc, lens, out=out, workspace=ws, stream=stream)

    log(f"[bench] warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    rec = {"quantize": []}
    if steady:
        ms_step, a_us, d_us = steady_graph_timing(kv, torch, args.warmup, args.steps, caches,
                                                  news, qs, out, ws, L, B, T)
        q_us = None
    else:
        # The quantize launches run eagerly (each keeps the GPU busy far longer
        # than its launch takes). The append + decode phase, whose launches are
        # shorter than the host's cost per call, runs as one captured HIP graph,
        # so that the step is not timed waiting for the host; graphs of the
        # decodes alone and the appends alone give their per-launch times.
        pos_g = torch.full((B,), T, dtype=torch.int32, device=dev)
        lens_g = pos_g + 1

        def appends():
            for layer in range(L):
                kc, vc = caches[layer]
                kv.append_kv(news[layer][0], news[layer][1], pos_g, kc, vc)

        def decodes(layer=None):
            for la in (range(L) if layer is None else [layer]):
                kc, vc = caches[la]
                kv.decode_attn(qs[la], kc, vc, lens_g, out=out, workspace=ws)

        def phase2():
            for layer in range(L):
                kc, vc = caches[layer]
                kv.append_kv(news[layer][0], news[layer][1], pos_g, kc, vc)
                decodes(layer)

        torch.cuda.synchronize()
        graphs = {}
        for name, fn in (("step", phase2), ("decode", decodes), ("append", appends)):
            graphs[name] = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graphs[name]):
                fn()
        graphs["step"].replay()
        torch.cuda.synchronize()

        log(f"[bench] timing {args.steps} steps (append + decode as HIP graph replays)")
        start, end = ev(), ev()
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(args.steps):
            for layer in range(L):
                for x, c in ((xs[layer][0], caches[layer][0]), (xs[layer][1], caches[layer][1])):
                    a, b_ = ev(), ev()
                    a.record(stream)
                    kv.quantize(x, c, iters=args.iters, stream=stream)
                    b_.record(stream)
                    rec["quantize"].append((a, b_))
            graphs["step"].replay()
        end.record(stream)
        torch.cuda.synchronize()
        ms_step = start.elapsed_time(end) / args.steps

        def replay_us(g, n):
            a, b_ = ev(), ev()
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(n):
                g.replay()
            b_.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b_) * 1e3 / n

        v = [a.elapsed_time(b_) * 1e3 for a, b_ in rec["quantize"]]
        q_us = sum(v) / len(v)
        d_us = replay_us(graphs["decode"], max(args.steps, 5)) / L
        a_us = replay_us(graphs["append"], max(args.steps, 5)) / L
        del graphs
    elts_per_quant = B * Hkv * T * D
    q_launches = 0 if steady else 2 * L
    bf16_bytes_step = q_launches * elts_per_quant * 2
    # tokens attended per decode: the graph-timed decodes of the steady-state
    # workload run after the timed steps, over T + warmup + steps + 1 tokens
    dec_tokens = (T + args.warmup + args.steps + 1) if steady else (T + 1)
    dec_bytes = decode_bytes(dec_tokens, B, Hkv, Hq)
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
                           "quantize K,V of every layer, then append + decode per layer "
                           "(the append + decode phase as one HIP graph replay)"},
    }
    dec = {"tokens_per_s": round(B / (decode_ms_step / 1e3), 1),
           "us_per_launch": round(d_us, 2), "launches_per_step": L,
           **hbm_entry(dec_bytes, d_us), "kernels": DECODE_KERNELS,
           "decode_arith": DECODE_ARITH,
           "cache_regime": "HBM: each decode reads a layer whose cache was written more "
                           "than 256 MB of traffic earlier"}
    dec_roof = {"bound": "hbm", "achieved": dec["GBps_algorithmic"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": dec["hbm_frac"],
                "traffic": measured_traffic(DECODE_KERNELS, wl.name),
                "kernel": DECODE_KERNELS, "bytes_per_launch": dec_bytes}
    if steady:
        res["value"] = dec["tokens_per_s"]
        res["unit"] = "tokens/s (decode attention, all layers)"
        res["step_tokens_per_s"] = round(B / (ms_step / 1e3), 1)
        res["roofline"] = dec_roof
    else:
        qbytes = QUANT_BYTES_PER_ELT_BF16 * elts_per_quant
        res["value"] = round(bf16_bytes_step / (ms_step / 1e3) / 1e9, 2)
        res["unit"] = "GB/s (bf16 K/V in, whole quantize+append+decode step)"
        res["quantize"] = {"GBps_bf16_in": round(elts_per_quant * 2 / (q_us * 1e-6) / 1e9, 1),
                           "us_per_launch": round(q_us, 2), "launches_per_step": q_launches,
                           **hbm_entry(qbytes, q_us), "quantize_arith": QUANT_ARITH}
        res["roofline"] = quant_roofline(qbytes, elts_per_quant, q_us, args.iters, wl.name)
        res["roofline_decode"] = dec_roof
        res["pages_context"] = {
            "pages_normalization_ms": PAGES_NORMALIZATION_MS,
            "pages_generation_ms": PAGES_GENERATION_MS,
            "pages_share": round(PAGES_NORMALIZATION_MS / PAGES_GENERATION_MS, 5),
            "source": "rndamp.com article on KVarN, section Numbers (Qwen3-4B, unnamed GPU, "
                      "batch and length not stated)",
            "this_quantize_ms_per_step": round(q_launches * q_us / 1e3, 3),
            "this_step_ms": round(ms_step, 3),
            "this_quantize_share_of_step": round(q_launches * q_us / 1e3 / ms_step, 4),
            "note": "context only, not a like-for-like comparison: here the whole 36-layer "
                    "cache of batch 8 x 32768 tokens is quantized in every step"}
    res["decode"] = dec
    res["append"] = {"us_per_launch": round(a_us, 2), "launches_per_step": L,
                     "kernel": "append_kv_kernel: a layer's new K and V token in one launch"}

    cpu_inputs = None
    if not args.no_cpu_baseline and not steady:
        cpu_inputs = cpu_sample(args, wl, xs, news, qs)
    if not steady:
        res["host_us_per_call"] = host_cost(
            kv, torch, stream, xs[0][0], caches[0], news[0], qs[0], out, ws,
            torch.full((B,), T + 1, dtype=torch.int32, device=dev),
            torch.full((B,), T, dtype=torch.int32, device=dev))
    if not args.no_ablations and not steady:
        res["ablations"] = ablations(kv, torch, stream, xs, qs, caches, ws, out, T + 1,
                                     args.iters)
        res["error_diagnostics"] = error_diagnostics(kv, torch, stream, xs[0], caches[0],
                                                     args.iters, res["ablations"])
    if not args.no_subworkloads and args.workload == 2:
        del xs, caches, news, qs, out, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        res["workloads"] = {}
        sub = kvgen.WORKLOADS[3]
        res["workloads"][sub.name] = steady_workload(kv, kvgen, torch, sub, args, dev)
        torch.cuda.empty_cache()
        sub = kvgen.WORKLOADS[4]
        res["workloads"][sub.name] = stress_workload(kv, kvgen, torch, sub, args, dev, stream)
        torch.cuda.empty_cache()
        res["next_rows"] = next_rows_workload(kv, kvgen, torch, args, dev, stream)
        torch.cuda.empty_cache()
    if cpu_inputs is not None:
        res["cpu_baseline"] = cpu_baseline(args, wl, cpu_inputs, res["unit"], bf16_bytes_step,
                                           cap)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def quant_roofline(qbytes, elts, q_us, iters, wl_name):
    """Roofline of the quantizer: the larger of its ideal HBM time (bytes at
    the HBM peak) and its ideal ALU time (algorithmic fp32 operations at the
    VALU peak) names the bound; the other resource stays beside it."""
    q_gbps = qbytes / (q_us * 1e-6) / 1e9
    q_flop = quant_flop_per_elt(iters) * elts
    q_tflops = q_flop / (q_us * 1e-6) / 1e12
    t_hbm = qbytes / (HBM_PEAK_GBPS * 1e9)
    t_alu = q_flop / (VALU_F32_PEAK_TFLOPS * 1e12)
    alu = {"achieved": round(q_tflops, 2), "peak": round(VALU_F32_PEAK_TFLOPS, 2),
           "unit": "TFLOP/s", "frac": round(q_tflops / VALU_F32_PEAK_TFLOPS, 4),
           "flop_per_element": quant_flop_per_elt(iters),
           "peak_nonpacked": round(VALU_F32_NONPACKED_TFLOPS, 2),
           "frac_nonpacked": round(q_tflops / VALU_F32_NONPACKED_TFLOPS, 4),
           "ideal_us_nonpacked": round(q_flop / (VALU_F32_NONPACKED_TFLOPS * 1e12) * 1e6, 2)}
    hbm = {"achieved": round(q_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": round(q_gbps / HBM_PEAK_GBPS, 4)}
    bound, main, other = ("hbm", hbm, alu) if t_hbm >= t_alu else ("alu", alu, dict(hbm))
    return {"bound": bound, **main,
            "traffic": measured_traffic("quantize_block_kernel<bf16>", wl_name),
            "kernel": "quantize_block_kernel<bf16>",
            "elements_per_launch": elts, "bytes_per_launch": qbytes,
            "ideal_us": {"hbm": round(t_hbm * 1e6, 2), "alu": round(t_alu * 1e6, 2)},
            ("alu" if bound == "hbm" else "hbm"): other}


def error_diagnostics(kv, torch, stream, x_pair, cache_pair, iters, abl):
    """Magnitude vs direction of the quantization error on layer 0 (outside
    the timed step), for the 2 x 2 of rotation {on, off} x balancing
    {iters, 0} sweeps. Each token's squared error relative to ||x||^2 splits
    exactly into (rho - 1)^2 (magnitude, rho = ||x_hat|| / ||x||) and
    2 rho (1 - cos) (direction). Rotation off quantizes x itself in its own
    basis (KVARN_FLAG_NO_ROTATE on the raw input) and measures the error in
    that basis. Means over all tokens of K and V, through kvarn_token_error;
    each cell carries the quantize time of that variant (ablations)."""
    res = {}
    qt = abl["quantize_us"] if abl else {}
    cell_time = {(True, iters): qt.get(f"iters_{iters}"), (True, 0): qt.get("iters_0"),
                 (False, iters): qt.get("no_rotate"), (False, 0): qt.get("no_rotate_iters_0")}
    for name, x, cache in (("K", x_pair[0], cache_pair[0]), ("V", x_pair[1], cache_pair[1])):
        scratch = kv.Cache.empty(cache.batch, cache.kv_heads, cache.capacity, cache.kind,
                                 device=x.device)
        for rot in (True, False):
            flags = 0 if rot else kv.FLAG_NO_ROTATE
            for it in (iters, 0):
                kv.quantize(x, scratch, iters=it, stream=stream, flags=flags)
                ratio, cosine = kv.token_error(x, scratch, stream=stream, flags=flags)
                torch.cuda.synchronize()
                r, c = ratio.double(), cosine.double()
                res[f"{name}_rotate_{'on' if rot else 'off'}_iters_{it}"] = {
                    "magnitude": round(float(((r - 1) ** 2).mean()), 6),
                    "direction": round(float((2 * r * (1 - c)).mean()), 6),
                    "mean_ratio": round(float(r.mean()), 5),
                    "mean_cos": round(float(c.mean()), 5),
                    "quantize_us": cell_time.get((rot, it))}
        del scratch
    res["note"] = ("per-token squared error / ||x||^2 = magnitude + direction; means over "
                   "layer 0's tokens; rotation off = quantized in the original basis")
    return res


def ablations(kv, torch, stream, xs, qs, caches, ws, out, length, iters, rounds=3):
    """Launch times of the variants outside the timed step, with HIP events:
    the quantizer with and without balancing (iters vs 0: the cost of the
    dual-scaling normalization) and with the rotation absorbed (with and
    without balancing), decode with both scales and with the column scales
    taken as 1 (the cost of the second scale), and decode with the rotation
    absorbed (no query rotation, no output un-rotation).
    Each repetition reads another layer's input (quantize: 537 MB of K per
    layer) or cache (decode: 168 MB per layer), in turn over all layers, so
    no repetition finds its data in the 256 MB memory-side cache: these are
    HBM times, as in the timed step. The variants are timed in turn, `rounds`
    times over, and each reports the median of its rounds: the shader clock
    moves by several percent within a second of a change of load. Scratch
    caches keep the benchmark's caches intact."""
    L = len(xs)
    kc0 = caches[0][0]
    scratch = kv.Cache.empty(kc0.batch, kc0.kv_heads, kc0.capacity, kv.K, device=kc0.codes.device)
    lens = torch.full((kc0.batch,), length, dtype=torch.int32, device=kc0.codes.device)

    def quant(it, flags):
        return lambda i: kv.quantize(xs[i % L][0], scratch, iters=it, stream=stream, flags=flags)

    def dec(flags):
        return lambda i: kv.decode_attn(qs[i % L], caches[i % L][0], caches[i % L][1], lens,
                                        out=out, workspace=ws, stream=stream, flags=flags)
    variants = {
        "q_full": quant(iters, 0),
        "q_none": quant(0, 0),
        "q_norot": quant(iters, kv.FLAG_NO_ROTATE),
        "q_norot_none": quant(0, kv.FLAG_NO_ROTATE),
        "d_two": dec(0),
        "d_one": dec(kv.FLAG_ONE_SCALE),
        "d_norot": dec(kv.FLAG_NO_ROTATE),
    }

    def timed(fn):
        fn(L - 1)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(L):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / L

    times = {k: [] for k in variants}
    for _ in range(rounds):
        for k, fn in variants.items():
            times[k].append(timed(fn))
    del scratch
    t = {k: sorted(v)[len(v) // 2] for k, v in times.items()}
    return {
        "quantize_us": {f"iters_{iters}": round(t["q_full"], 2), "iters_0": round(t["q_none"], 2),
                        "no_rotate": round(t["q_norot"], 2),
                        "no_rotate_iters_0": round(t["q_norot_none"], 2),
                        "balancing_share": round((t["q_full"] - t["q_none"]) / t["q_full"], 4)},
        "decode_us": {"two_scales": round(t["d_two"], 2), "one_scale": round(t["d_one"], 2),
                      "no_rotate": round(t["d_norot"], 2),
                      "second_scale_overhead": round((t["d_two"] - t["d_one"]) / t["d_one"], 4),
                      # the column scales are 8 of the 80 bytes per cached token and
                      # kv-head, which the one-scale variant does not read: the
                      # overhead per byte read is what the fused scale costs beyond them
                      "second_scale_extra_bytes": round(80 / 72 - 1, 4),
                      "second_scale_overhead_per_byte": round(
                          (t["d_two"] / 80) / (t["d_one"] / 72) - 1, 4)},
        "regime": f"HBM: each of the {L} launches per timing reads another layer's input or "
                  f"cache (none fits in the {MALL_BYTES >> 20} MB memory-side cache)",
        "note": f"K tensor for quantize; HIP events over {L} launches after one warm launch; "
                f"variants timed in turn, median of {rounds} rounds",
    }


def build_steady_caches(kv, kvgen, torch, wl, caches, iters, dev):
    """Quantize the steady-state workload's cache once (outside timing), one
    layer's bf16 K or V at a time, so its 34 GB of input never coexist."""
    for layer, (kc, vc) in enumerate(caches):
        for kind, c in ((kvgen.K, kc), (kvgen.V, vc)):
            x = kvgen.kv_tensor(wl.seed, layer, kind, wl.batch, wl.kv_heads, wl.tokens,
                                wl.sigma, device=dev)
            kv.quantize(x, c, iters=iters)
            del x
    torch.cuda.synchronize()


def steady_graph_timing(kv, torch, warmup, steps, caches, news, qs, out, ws, L, B, T):
    """Steady-state decoding timed on HIP-graph replays (torch.cuda.CUDAGraph).

    G_step holds one step: for every layer, append K and V at pos (one
    launch), decode over lens; then pos and lens advance by one, so each replay
    is the next step. G_dec holds the L decodes alone and G_app the L appends
    alone (at a fixed position, so replaying them rewrites the same slots);
    their replays give the per-launch times. The positions continue from
    `warmup` eager steps. Returns (ms per step, us per K+V append launch, us
    per decode)."""
    dev = out.device
    pos = torch.full((B,), T + warmup, dtype=torch.int32, device=dev)
    lens = pos + 1
    torch.cuda.synchronize()

    def layer_appends(layer):
        kc, vc = caches[layer]
        kv.append_kv(news[layer][0], news[layer][1], pos, kc, vc)

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

    log(f"[bench] timing {steps} steps (HIP graph replays)")
    ms_step = timed(g_step, steps)
    reps = max(steps, 10)
    d_us = timed(g_dec, reps) * 1e3 / L
    a_us = timed(g_app, reps) * 1e3 / L
    return ms_step, a_us, d_us


def steady_workload(kv, kvgen, torch, wl, args, dev):
    """Sub-result: the Llama-3-8B-shaped steady-state decode (32 layers, batch
    32, 8192-token cache, one appended token per sequence and layer per
    step), graph-timed as in --workload 3."""
    L, B, Hkv, Hq, T = wl.layers, wl.batch, wl.kv_heads, wl.q_heads, wl.tokens
    cap = T + CHUNK
    log(f"[bench] sub-workload {wl.name}: building the cache ...")
    caches = [(kv.Cache.empty(B, Hkv, cap, kv.K, device=dev),
               kv.Cache.empty(B, Hkv, cap, kv.V, device=dev)) for _ in range(L)]
    build_steady_caches(kv, kvgen, torch, wl, caches, args.iters, dev)
    news = [(kvgen.new_tokens(wl.seed, layer, kvgen.K, B, Hkv, wl.sigma, device=dev),
             kvgen.new_tokens(wl.seed, layer, kvgen.V, B, Hkv, wl.sigma, device=dev))
            for layer in range(L)]
    qs = [kvgen.queries(wl.seed, layer, B, Hq, device=dev) for layer in range(L)]
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = kv.decode_workspace(B, Hq, cap, device=dev)
    warm, steps = 2, 10
    for i in range(warm):
        pos = torch.full((B,), T + i, dtype=torch.int32, device=dev)
        for layer in range(L):
            kv.append_kv(news[layer][0], news[layer][1], pos, caches[layer][0],
                         caches[layer][1])
            kv.decode_attn(qs[layer], caches[layer][0], caches[layer][1], pos + 1, out=out,
                           workspace=ws)
    torch.cuda.synchronize()
    ms_step, a_us, d_us = steady_graph_timing(kv, torch, warm, steps, caches, news, qs, out, ws,
                                              L, B, T)
    nb = decode_bytes(T + warm + steps + 1, B, Hkv, Hq)
    res = {"config": {"layers": L, "batch": B, "kv_heads": Hkv, "q_heads": Hq, "tokens": T,
                      "step": "append K and V (one launch) + decode per layer (HIP graph "
                              "replays)"},
           "step_ms": round(ms_step, 4), "step_tokens_per_s": round(B / (ms_step / 1e3), 1),
           "decode_tokens_per_s": round(B / (L * d_us * 1e-6), 1),
           "decode_us_per_launch": round(d_us, 2), "append_kv_us_per_launch": round(a_us, 2),
           "decode": hbm_entry(nb, d_us)}
    del caches, news, qs, out, ws
    return res


def stress_workload(kv, kvgen, torch, wl, args, dev, stream):
    """Sub-result: the long-horizon stress shape (1 layer, batch 64, 131072
    tokens quantized in 128-token chunks, token scales lognormal(0, 1)):
    quantize K and V, append one token, decode over the whole cache."""
    B, Hkv, Hq, T = wl.batch, wl.kv_heads, wl.q_heads, wl.tokens
    cap = T + CHUNK
    log(f"[bench] sub-workload {wl.name}: generating inputs ...")
    xk = kvgen.kv_tensor(wl.seed, 0, kvgen.K, B, Hkv, T, wl.sigma, device=dev)
    xv = kvgen.kv_tensor(wl.seed, 0, kvgen.V, B, Hkv, T, wl.sigma, device=dev)
    kc = kv.Cache.empty(B, Hkv, cap, kv.K, device=dev)
    vc = kv.Cache.empty(B, Hkv, cap, kv.V, device=dev)
    nk = kvgen.new_tokens(wl.seed, 0, kvgen.K, B, Hkv, wl.sigma, device=dev)
    nv = kvgen.new_tokens(wl.seed, 0, kvgen.V, B, Hkv, wl.sigma, device=dev)
    q = kvgen.queries(wl.seed, 0, B, Hq, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = kv.decode_workspace(B, Hq, cap, device=dev)
    pos = torch.full((B,), T, dtype=torch.int32, device=dev)
    lens = pos + 1
    quant = [lambda: kv.quantize(xk, kc, iters=args.iters, stream=stream),
             lambda: kv.quantize(xv, vc, iters=args.iters, stream=stream)]
    for f in quant:
        f()
    kv.append_kv(nk, nv, pos, kc, vc, stream=stream)
    kv.decode_attn(q, kc, vc, lens, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    q_us = timed_events(torch, stream, quant * 3)
    d_us = timed_events(torch, stream, [lambda: kv.decode_attn(q, kc, vc, lens, out=out,
                                                               workspace=ws, stream=stream)] * 10)
    elts = B * Hkv * T * D
    qm, dm = sum(q_us) / len(q_us), sum(d_us) / len(d_us)
    res = {"config": {"layers": 1, "batch": B, "kv_heads": Hkv, "q_heads": Hq, "tokens": T,
                      "token_scale_sigma": wl.sigma},
           "quantize_us_per_launch": round(qm, 2),
           "quantize": hbm_entry(QUANT_BYTES_PER_ELT_BF16 * elts, qm),
           "decode_us_per_launch": round(dm, 2),
           "decode_tokens_per_s": round(B / (dm * 1e-6), 1),
           "decode": hbm_entry(decode_bytes(T + 1, B, Hkv, Hq), dm),
           "note": "HIP events; quantize mean of 6 launches (K, V alternating), decode mean of "
                   "10 calls over a 5.4 GB cache"}
    del xk, xv, kc, vc, nk, nv, q, out, ws
    return res


def host_cost(kv, torch, stream, x, cache_pair, new_toks, q, out, ws, lens, pos,
              n: int = 200):
    """Host microseconds per call, enqueue only: wall time of n back-to-back
    calls with no synchronization inside (the GPU work queues up behind
    them), for the Python binding's quantize, append (one cache, and K and V
    in one call) and decode, and for decode through the C ABI directly with
    its arguments marshalled once (the library's own host share)."""
    import ctypes
    kc, vc = cache_pair
    new_tok, new_tok_v = new_toks
    lib = kv.load()
    kd, vd = kc.desc(), vc.desc()
    sh = stream.cuda_stream
    raw = (q.data_ptr(), kv._dtype_code(q), q.shape[1], ctypes.byref(kd), ctypes.byref(vd),
           lens.data_ptr(), q.shape[2] ** -0.5, 0, out.data_ptr(), 0, ws.data_ptr(),
           ws.numel() * ws.element_size(), sh)
    calls = {
        "quantize_binding": lambda: kv.quantize(x, kc, stream=stream),
        "append_binding": lambda: kv.append(new_tok, pos, kc, stream=stream),
        "append_kv_binding": lambda: kv.append_kv(new_tok, new_tok_v, pos, kc, vc, stream=stream),
        "decode_binding": lambda: kv.decode_attn(q, kc, vc, lens, out=out, workspace=ws,
                                                 stream=stream),
        "decode_c_abi": lambda: lib.kvarn_decode_attn_ex(*raw),
    }
    res = {}
    for name, fn in calls.items():
        reps = 8 if name.startswith("quantize") else n
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        res[name] = round((t1 - t0) / reps * 1e6, 2)
    res["note"] = ("host wall time per enqueued call, no synchronization inside the loop; "
                   "decode_c_abi calls kvarn_decode_attn_ex through ctypes with prebuilt "
                   "arguments")
    return res


def graph_us(torch, fn, reps: int = 5) -> float:
    """Microseconds of one replay of a HIP graph holding fn's launches: the
    median of `reps` timed replays after one untimed replay."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        g.replay()
        b.record(st)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    del g
    return sorted(ts)[reps // 2]


def next_rows_workload(kv, kvgen, torch, args, dev, stream):
    """Sub-result: the rows built beyond the hot path, measured to the same
    bar as the path itself.
    - append_rebalance (the append that re-quantizes a chunk when it fills) at
      the Llama-3-8B layer shape (32 sequences, 8 kv-heads): 128 steps of K and
      V appends filling one chunk, captured in a HIP graph, against the same
      steps with the plain append; the difference over the two chunk closes is
      the cost of re-quantizing a full chunk of 256 (sequence, kv-head) blocks.
    - head sizes 64 and 256 at the Qwen3-4B layer shape (8 sequences,
      8 kv-heads, 32 query heads, 32768 tokens; quantize and decode run the
      kernels every head size shares): quantize of bf16
      K over 4 layers' inputs and decode over 4 layers' caches, each cycled so
      that nothing is served from the memory-side cache; HIP events, 12 launches
      after a warm one, median of 3 rounds."""
    res = {}
    B, H = 32, 8
    kc = kv.Cache.empty(B, H, 2 * CHUNK, kv.K, device=dev)
    vc = kv.Cache.empty(B, H, 2 * CHUNK, kv.V, device=dev)
    wk, wv = kv.append_window(B, H, device=dev), kv.append_window(B, H, device=dev)
    toks = [(kvgen.new_tokens(11, 0, kvgen.K, B, H, 0.5, step=t, device=dev),
             kvgen.new_tokens(11, 0, kvgen.V, B, H, 0.5, step=t, device=dev)) for t in range(CHUNK)]
    poss = [torch.full((B,), t, dtype=torch.int32, device=dev) for t in range(CHUNK)]

    def fill(rebalance: bool):
        for t in range(CHUNK):
            if rebalance:
                kv.append_rebalance(toks[t][0], poss[t], kc, wk, iters=args.iters)
                kv.append_rebalance(toks[t][1], poss[t], vc, wv, iters=args.iters)
            else:
                kv.append(toks[t][0], poss[t], kc)
                kv.append(toks[t][1], poss[t], vc)

    t_re = graph_us(torch, lambda: fill(True))
    t_plain = graph_us(torch, lambda: fill(False))
    res["append_rebalance"] = {
        "config": {"batch": B, "kv_heads": H, "tokens_appended": CHUNK},
        "us_per_call": round(t_re / (2 * CHUNK), 2),
        "plain_append_us_per_call": round(t_plain / (2 * CHUNK), 2),
        "extra_us_per_128_steps": round(t_re - t_plain, 2),
        "note": "HIP-graph replays of 128 steps (K and V); each append_rebalance call is an "
                "append plus a launch of the chunk re-quantizer, whose workgroups leave at "
                "once except at the step that closes the chunk (the extra time covers those "
                "launches and the two closes)"}
    del kc, vc, wk, wv, toks, poss
    torch.cuda.empty_cache()

    B, H, Hq, T, L = 8, 8, 32, 32768, 4
    for dh in (64, 256):
        log(f"[bench] head size {dh}: generating inputs ...")
        xs = [kvgen.kv_tensor(5, l, kvgen.K, B, H, T, 0.5, device=dev, head_dim=dh)
              for l in range(L)]
        qcs = [kv.Cache.empty(B, H, T, kv.K, device=dev, head_dim=dh) for _ in range(L)]
        caches = []
        for l in range(L):
            pair = []
            for kind in (kv.K, kv.V):
                x = kvgen.kv_tensor(5, l, kind, B, H, T, 0.5, device=dev, head_dim=dh)
                c = kv.Cache.empty(B, H, T + CHUNK, kind, device=dev, head_dim=dh)
                kv.quantize(x, c, iters=args.iters, stream=stream)
                del x
                pair.append(c)
            caches.append(pair)
        q = [kvgen.queries(5, l, B, Hq, device=dev, head_dim=dh) for l in range(L)]
        out = torch.empty((B, Hq, dh), dtype=torch.float32, device=dev)
        ws = kv.decode_workspace(B, Hq, T + CHUNK, device=dev, head_dim=dh)
        lens = torch.full((B,), T + 1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        # as in the step: the quantizer with HIP events around each launch
        # (median of three rounds of 12), decode as graph replays of 12 calls,
        # since events around an eager decode call would also count the
        # binding's host time (a call's host cost is close to a head-size-64
        # decode's duration); layers cycled in both
        qf = [lambda i=i: kv.quantize(xs[i % L], qcs[i % L], iters=args.iters, stream=stream)
              for i in range(12)]
        qm = []
        for _ in range(3):
            qf[0]()
            qu = timed_events(torch, stream, qf)
            qm.append(sum(qu) / len(qu))
        qm = sorted(qm)[1]
        dm = graph_us(torch, lambda: [kv.decode_attn(q[i % L], caches[i % L][0],
                                                     caches[i % L][1], lens, out=out, workspace=ws)
                                      for i in range(12)]) / 12
        # one-token appends of K and V in one launch, as in the step: graph
        # replays of 36 launches (the layers' appends nine times over; each
        # rewrites the same slots), since each launch is shorter than the
        # host's cost per call and a replay's own start-up is spread over as
        # many launches as in the step
        tok = [kvgen.new_tokens(5, l, kind, B, H, 0.5, device=dev, head_dim=dh)
               for l in range(L) for kind in (kv.K, kv.V)]
        pos = torch.full((B,), T, dtype=torch.int32, device=dev)
        am = graph_us(torch, lambda: [kv.append_kv(tok[2 * l], tok[2 * l + 1], pos,
                                                   caches[l][0], caches[l][1])
                                      for _ in range(9) for l in range(L)]) / (9 * L)
        elts = B * H * T * dh
        qbytes = (2.0 + 0.25 + 4.0 / dh + 4.0 / CHUNK) * elts
        dbytes = (dh / 2 + 8 + dh / 16) * (T + 1) * B * H + B * Hq * dh * 6
        res[f"head_dim_{dh}"] = {
            "config": {"batch": B, "kv_heads": H, "q_heads": Hq, "tokens": T, "head_dim": dh},
            "quantize_us_per_launch": round(qm, 2), "quantize": hbm_entry(qbytes, qm),
            "decode_us_per_launch": round(dm, 2), "decode": hbm_entry(dbytes, dm),
            "append_kv_us_per_launch": round(am, 2),
            "note": "quantize and decode: the matrix-core kernels shared by every head size; "
                    "append: one launch for a layer's K and V token (latency-bound, no "
                    "bandwidth claim)"}
        del xs, qcs, caches, q, out, ws, tok
        torch.cuda.empty_cache()
    return res


def cpu_sample(args, wl, xs, news, qs):
    """Host copies of the (layer 0, sequence, kv-head) slices the CPU baseline
    runs: whole slices of the step, drawn with a fixed seed."""
    import numpy as np
    threads = cpu_threads()
    n = args.cpu_slices or 2 * threads
    B, Hkv, Hq = wl.batch, wl.kv_heads, wl.q_heads
    G = Hq // Hkv
    rng = np.random.default_rng(0)
    pairs = [(int(rng.integers(B)), int(rng.integers(Hkv))) for _ in range(n + 1)]
    inputs = []
    for b, g in pairs:
        inputs.append(tuple(t.double().cpu().numpy() for t in (
            xs[0][0][b:b + 1, g:g + 1], xs[0][1][b:b + 1, g:g + 1],
            news[0][0][b:b + 1, g:g + 1], news[0][1][b:b + 1, g:g + 1],
            qs[0][b:b + 1, g * G:(g + 1) * G])))
    return inputs


def cpu_threads() -> int:
    """Host threads for the oracle: every CPU this process may run on, up to
    the box's share for one GPU."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(HOST_THREAD_CAP, avail))


def cpu_baseline(args, wl, inputs, unit, bf16_bytes_step, cap):
    """The oracle (fp64 C, unmodified) timed on this host's cores on a bounded
    sample of the same step: whole (layer 0, sequence b, kv-head g) slices --
    quantize all chunks of K and V, append the new token, decode the group's
    query heads -- one slice per thread at a time, then scaled to the full
    step. One more slice runs alone on one thread for the one-core figure."""
    import numpy as np

    import oracle

    oracle.lib()
    threads = cpu_threads()
    T = wl.tokens
    G = wl.q_heads // wl.kv_heads

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

    work = list(inputs[:-1])
    n = len(work)
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
    log("[bench] cpu baseline: one slice on one thread ...")
    t1 = time.perf_counter()
    one(inputs[-1])
    wall1 = time.perf_counter() - t1
    slices_per_step = wl.layers * wl.batch * wl.kv_heads

    def value(step_s):
        return round(bf16_bytes_step / step_s / 1e9, 6)

    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": value(wall * slices_per_step / n), "unit": unit, "cores": threads,
            "kind": "oracle", "wall_s": round(wall, 2),
            "host_cpus": os.cpu_count(), "affinity_cpus": affinity,
            "one_core": {"value": value(wall1 * slices_per_step), "wall_s": round(wall1, 2),
                         "sample": "1 slice on 1 thread, scaled by "
                                   f"{slices_per_step} to the full step"},
            "sample": f"{n} whole (layer 0, seq, kv-head) slices of the step "
                      f"(quantize {2 * T // CHUNK} chunks of K+V incl. the oracle's "
                      f"O(D^2) rotation, append 1 token each, decode {G} query heads over "
                      f"{T + 1} tokens), {threads} threads (the host's CPUs available to this "
                      f"process, at most {HOST_THREAD_CAP}: the box's share for one GPU), "
                      f"scaled by {slices_per_step}/{n} to the full step"}


if __name__ == "__main__":
    main()
