#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 linear-layer hot path on one MI355X.

One step = one pass of the whole path over the 8192-token MLP pair: dynamic
NVFP4 quantization of X [8192, 5120] -> fused gate|up GEMM (two segments,
each with its own global scale) with SiLU*mul and the amax partials of h in
its epilogue -> quantization of h [8192, 17408] -> down GEMM.  Every step runs in the
library's HIP kernels on torch's current stream; inputs are synthetic,
seeded and resident in HBM before the timed region.

Prints ONE JSON line: TFLOP/s including activation quantization (algorithmic
2*M*N*K of both GEMMs over the time of every stage), the roofline of the
dominant kernel (the gate|up GEMM with the SiLU*mul epilogue, timed live
with HIP events on the launch stream), the decode-shape (M=8)
weight-streaming GB/s, the other linear-layer workloads (the tiny 32x128x256
layer's latency, the 4096x5120x5120 act-quant GEMM, the 32K-token GDN
in-projection) and, for context only, dense bf16 torch.matmul at the MLP
pair's shapes under "secondary", and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 W4A4 GEMM TFLOP/s incl. act-quant (M=8192) + % peak; GB/s at M=8"
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_m8192_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_m8192_mfma.json")
NOMINAL_CLOCK_GHZ = 2.4
# sources the gate|up GEMM kernel is compiled from: the committed HBM
# counters are reported only while all of them are unchanged
GEMM_SRC = [os.path.join(ROOT, "bit_linear_layer_amd", "csrc", f)
            for f in ("gemm.hip", "device_util.h", "quant_block.h", "internal.h")]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-secondary", action="store_true", help="skip the decode / GDN measurements")
    ap.add_argument("--parts", default="all",
                    help="comma list of secondary measurements to run (small, decode, gdn_in_proj, gdn, kv, "
                         "variants, context) or 'all'; for profiling runs")
    ap.add_argument("--cpu-rows", type=int, default=4608, help="rows of the oracle's timed sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration) and exit")
    return ap.parse_args()


def sha256(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per launch of the gate|up GEMM from the committed rocprofv3
    counter summary, or None if absent or taken on another kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256") != sha256(GEMM_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


def read_mfma_counters():
    """Observed shader clock and MFMA-busy fraction of the gate|up GEMM from
    the committed rocprofv3 counter summary, or None if absent or taken on
    another kernel source."""
    try:
        with open(MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256") != sha256(GEMM_SRC):
        return None
    return t


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported (the layers shard "
              "along N without communication: each GPU would run this step on its slice of every "
              "weight segment)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_linear_layer_amd as nv
    import workloads as W

    nv.load()  # fails loudly without the HIP library
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ------------------------------------------------------------ inputs
    log("generating the 8192-token MLP pair workload (seed 0)")
    wl = W.mlp_pair()
    m, k = wl.x.shape
    inter = wl.weights[0][1].shape[0]
    x = wl.x.to(dev)

    def quant_segments(segs):
        rows = sum(w.shape[0] for w in segs)
        kk = segs[0].shape[1]
        q = nv.empty_nvfp4(rows, kk, dev)
        g = torch.empty(len(segs), dtype=torch.float32, device=dev)
        ws = nv.workspace_for(max(w.shape[0] for w in segs), kk, dev)
        offs = [0]
        for s, w in enumerate(segs):
            part = q.row_slice(offs[-1], offs[-1] + w.shape[0])
            nv.nvfp4_quantize(w.to(dev), nv.NVFP4Tensor(part.codes, part.scales, g[s:s + 1], part.rows, kk),
                              nv.SCALE_DYNAMIC, ws)
            offs.append(offs[-1] + w.shape[0])
        return q, offs, g

    w_gu, gu_offs, gu_g = quant_segments([w for _, w in wl.weights])  # offline, untimed
    w_d, d_offs, d_g = quant_segments([wl.extra["w_down"]])
    a = nv.empty_nvfp4(m, k, dev)
    hq = nv.empty_nvfp4(m, inter, dev)
    h = torch.empty((m, inter), dtype=torch.bfloat16, device=dev)
    out = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    ws_x = nv.workspace_for(m, k, dev)
    ws_h = nv.workspace_for(m, inter, dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        nv.nvfp4_quantize(x, a, nv.SCALE_DYNAMIC, ws_x)
        if ev is not None:
            ev[0].record(stream)
        nv.nvfp4_gemm_swiglu(a, w_gu, gu_g, h=h, amax_workspace=ws_h)
        if ev is not None:
            ev[1].record(stream)
        nv.nvfp4_quantize(h, hq, nv.AMAX_PRECOMPUTED, ws_h)
        nv.nvfp4_gemm_fused_segments(hq, w_d, d_offs, d_g, out)

    flops_gu = 2.0 * m * (2 * inter) * k
    flops_d = 2.0 * m * k * inter
    flops = flops_gu + flops_d

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    elapsed_ms = t0.elapsed_time(t1)
    ms_per_step = elapsed_ms / args.steps
    value = flops * args.steps / (elapsed_ms * 1e-3) / 1e12
    gu_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    achieved = flops_gu / (gu_ms * 1e-3) / 1e12
    traffic = read_traffic()
    roofline = {"bound": "mfma", "kernel": "nvfp4 gemm + swiglu epilogue (gate|up, 8192x34816x5120)",
                "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
                "avg_launch_ms": round(gu_ms, 4)}
    log(f"step {ms_per_step:.3f} ms, {value:.1f} TFLOP/s; gate|up GEMM {gu_ms:.3f} ms = {achieved:.1f} TFLOP/s")

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 (e2m1+e4m3) -> f16 mfma, f32 accumulate",
        "data": "synthetic (seeded; random-init weights)",
        "config": {"workload": wl.name, "M": m, "K": k, "inter": inter,
                   "gate_up": [2 * inter, k], "down": [k, inter], "glue": "silu*mul + amax in gate|up epilogue",
                   "parallelism": "single-gpu"},
        "pct_of_mfma_peak": round(100.0 * value / MFMA_F16_PEAK_TFLOPS, 2),
        "roofline": roofline,
    }
    mc = read_mfma_counters()
    if mc is not None:
        clk = mc["observed_clock_ghz"]
        result["clock"] = {
            "observed_ghz": clk, "nominal_ghz": NOMINAL_CLOCK_GHZ,
            "source": "rocprofv3 GRBM_GUI_ACTIVE / 8 XCDs / duration of the gate|up GEMM "
                      "(profiles/gemm_gate_up_m8192_mfma.json)",
            "pct_of_mfma_peak_at_observed_clock": round(
                100.0 * value / (MFMA_F16_PEAK_TFLOPS * clk / NOMINAL_CLOCK_GHZ), 2),
            "gate_up_mfma_busy_frac": mc["mfma_busy_frac"]}

    # --------------------------------------------- decode shape (M = 8)
    if not args.no_secondary:
        parts = PARTS if args.parts == "all" else set(args.parts.split(","))
        if parts - PARTS:
            sys.exit(f"bench.py: unknown parts {sorted(parts - PARTS)}")
        sec = result["secondary"] = {}
        if "small" in parts:
            sec.update(small_configs(nv, W, torch, dev, stream, log))
        if "decode" in parts:
            sec.update(decode(nv, W, torch, dev, stream, log))
        if "gdn_in_proj" in parts:
            sec.update(gdn_in_proj(nv, W, torch, dev, stream, log))
        if "gdn" in parts:
            sec["gdn_recurrence"] = gdn_study(nv, W, torch, stream, log, dev)
        if "kv" in parts:
            sec.update(kv_fp8(nv, W, torch, dev, stream, log))
        if "variants" in parts:
            sec.update(mlp_variants(nv, torch, dev, stream, log, x, a, w_gu, gu_offs, gu_g,
                                    w_d, d_offs, d_g, hq, h, out, ws_x, ws_h, flops))
        if "context" in parts:
            sec.update(bf16_context(torch, dev, stream, log, x, h, k, inter))

    # --------------------------------------------------- CPU oracle leg
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(nv, W, torch, np, wl, a, w_gu, gu_offs, gu_g, w_d, d_offs, d_g,
                                              args.cpu_rows, log)
    print(json.dumps(result), flush=True)


def graph_replay_us(torch, stream, fn, per_graph=50, replays=10):
    """Average time of one fn() when per_graph calls of it are captured in
    one HIP graph and the graph is replayed (no host work between the
    launches), or None if the capture is refused."""
    try:
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                fn()
        graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (replays * per_graph) * 1e3
    except RuntimeError:
        return None


# Rotating input copies of the HBM-bound secondary measurements, so that a
# launch finds none of its data in the 256 MB last-level cache (MALL).
# Measured: with 4 rotating 32768 x 1024 KV buffers the KV write and read ran
# 15-25 % faster than with 12, 16 or 24 (which agree), i.e. part of their
# data still came from the MALL; the decode GEMM (100 MB per copy) was the
# same with 4 to 24.
ROTATE = 16


def time_steps(torch, stream, fn, steps=10, warmup=3):
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bf16_context(torch, dev, stream, log, x, h, k, inter):
    """Context, not a target: the same two GEMM shapes as dense bf16
    products through torch.matmul (the vendor GEMM library), bf16 inputs of
    the step's own X and h, N(0, 0.02) bf16 weights in [K, N] layout."""
    gen = torch.Generator(device=dev).manual_seed(0)
    w1 = (torch.randn((k, 2 * inter), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn((inter, k), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    o1 = torch.empty((x.shape[0], 2 * inter), dtype=torch.bfloat16, device=dev)
    o2 = torch.empty((h.shape[0], k), dtype=torch.bfloat16, device=dev)
    t1 = time_steps(torch, stream, lambda: torch.matmul(x, w1, out=o1))
    t2 = time_steps(torch, stream, lambda: torch.matmul(h, w2, out=o2))
    f1 = 2.0 * x.shape[0] * 2 * inter * k
    f2 = 2.0 * h.shape[0] * k * inter
    res = {"context_bf16_torch_matmul": {
        "note": "dense bf16 GEMMs of the same shapes (vendor library), for context only",
        "gate_up_ms": round(t1, 4), "gate_up_tflops": round(f1 / (t1 * 1e-3) / 1e12, 1),
        "down_ms": round(t2, 4), "down_tflops": round(f2 / (t2 * 1e-3) / 1e12, 1)}}
    log(f"context: bf16 torch.matmul gate|up {t1:.3f} ms = {f1 / (t1 * 1e-3) / 1e12:.0f} TFLOP/s, "
        f"down {t2:.3f} ms = {f2 / (t2 * 1e-3) / 1e12:.0f} TFLOP/s")
    del w1, w2, o1, o2
    return res


def mlp_variants(nv, torch, dev, stream, log, x, a, w_gu, gu_offs, gu_g, w_d, d_offs, d_g, hq, h, out,
                 ws_x, ws_h, flops):
    """The same MLP pair step two other ways: unfused glue (bf16 gate|up
    tensor, SiLU*mul kernel), and h quantized in the gate|up epilogue with a
    static (calibrated) global scale, here h's dynamic scale from one
    untimed pass, standing in for a checkpoint's calibrated value."""
    m, inter = h.shape
    gu = torch.empty((m, 2 * inter), dtype=torch.bfloat16, device=dev)

    def unfused():
        nv.nvfp4_quantize(x, a, nv.SCALE_DYNAMIC, ws_x)
        nv.nvfp4_gemm_fused_segments(a, w_gu, gu_offs, gu_g, gu)
        nv.nvfp4_silu_mul(gu, h, inter, ws_h)
        nv.nvfp4_quantize(h, hq, nv.AMAX_PRECOMPUTED, ws_h)
        nv.nvfp4_gemm_fused_segments(hq, w_d, d_offs, d_g, out)

    hs = nv.empty_nvfp4(m, inter, dev)
    unfused()
    hs.global_scale.copy_(hq.global_scale)  # calibration pass (untimed)

    def static_h():
        nv.nvfp4_quantize(x, a, nv.SCALE_DYNAMIC, ws_x)
        nv.nvfp4_gemm_swiglu(a, w_gu, gu_g, h_q=hs)
        nv.nvfp4_gemm_fused_segments(hs, w_d, d_offs, d_g, out)

    res = {}
    for name, fn in (("mlp_pair_unfused_glue", unfused), ("mlp_pair_static_h_scale", static_h)):
        ms = time_steps(torch, stream, fn)
        res[name] = {"ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        log(f"{name}: {ms:.3f} ms/step = {res[name]['tflops']} TFLOP/s")
    return res


def kv_fp8(nv, W, torch, dev, stream, log):
    """FP8 KV-cache write and read of one layer's K tensor [32768, 1024]
    (bf16), ROTATE rotating input/cache pairs (well past the 256 MB MALL), with the
    calibrated scale and with the unit (uncalibrated) scale."""
    wl = W.kv_cache()
    xs = [wl.x.to(dev)] + [wl.x.to(dev).mul_(1.0 + 0.001 * i) for i in range(1, ROTATE)]
    rows, cols = xs[0].shape
    caches = [torch.empty((rows, cols), dtype=torch.uint8, device=dev) for _ in range(ROTATE)]
    outs = [torch.empty((rows, cols), dtype=torch.bfloat16, device=dev) for _ in range(ROTATE)]
    s_cal = nv.kv_fp8_calibrate(xs[0])
    s_one = torch.ones(1, dtype=torch.float32, device=dev)
    ws = nv.workspace_for(rows, cols, dev)
    n = rows * cols
    res = {}

    def rate(name, fn, nbytes):
        ms = time_steps(torch, stream, fn, steps=40, warmup=4)  # fn itself rotates buffers
        res[name] = {"us": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    it = [0]

    def nxt():
        it[0] += 1
        return it[0] % ROTATE

    rate("kv_fp8_write_calibrated", lambda: (lambda i: nv.nvfp4_kv_fp8_quantize(xs[i], caches[i], s_cal))(nxt()), 3 * n)
    rate("kv_fp8_write_unit_scale", lambda: (lambda i: nv.nvfp4_kv_fp8_quantize(xs[i], caches[i], s_one))(nxt()), 3 * n)
    rate("kv_fp8_read_bf16", lambda: (lambda i: nv.nvfp4_kv_fp8_dequantize(caches[i], s_cal, outs[i]))(nxt()), 3 * n)
    rate("kv_fp8_calibrate", lambda: (lambda i: nv.nvfp4_kv_fp8_calibrate(xs[i], s_cal, ws))(nxt()), 2 * n)
    # context, not a kernel of this library: a plain device copy of the
    # same rotating bf16 tensors (2 B read + 2 B written per element)
    rate("context_torch_copy_bf16", lambda: (lambda i: outs[i].copy_(xs[i]))(nxt()), 4 * n)
    for k, v in res.items():
        log(f"{k}: {v['us']} us = {v['GBps']} GB/s")
    return {"kv_fp8_cache": {"workload": wl.name, "algorithmic_bytes_per_element": "write 3, read 3, calibrate 2",
                             **res}}


def small_configs(nv, W, torch, dev, stream, log):
    """The two smaller linear-layer workloads: the tiny 32x128x256 layer
    (fp32 output; latency of quantize X + GEMM, the weight pre-quantized)
    and the 4096x5120x5120 activation-quantize + GEMM (bf16 output,
    TFLOP/s including the activation quantization)."""
    res = {}
    for wl, key in ((W.tiny(), "tiny_m32"), (W.act_quant_gemm(), "act_quant_gemm_m4096")):
        x = wl.x.to(dev)
        w = nv.quantize(wl.weights[0][1].to(dev))
        a = nv.empty_nvfp4(x.shape[0], x.shape[1], dev)
        ws = nv.workspace_for(x.shape[0], x.shape[1], dev)
        out = torch.empty((x.shape[0], w.rows), dtype=torch.float32 if wl.out_dtype == "f32" else torch.bfloat16,
                          device=dev)

        def step():
            nv.nvfp4_quantize(x, a, nv.SCALE_DYNAMIC, ws)
            nv.nvfp4_gemm(a, w, out)

        ms = time_steps(torch, stream, step, steps=100, warmup=10)
        fl = 2.0 * x.shape[0] * w.rows * x.shape[1]
        res[key] = {"workload": wl.name, "us_quantize_plus_gemm": round(ms * 1e3, 2),
                    "TFLOPs_incl_act_quant": round(fl / (ms * 1e-3) / 1e12, 2)}
        log(f"{wl.name}: quantize + gemm {ms * 1e3:.1f} us = {fl / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
        if key == "tiny_m32":
            # the calls above are bound by the Python binding's host time;
            # the same two launches captured in a HIP graph and replayed give
            # the GPU side (both kernels and the gap between them)
            g_us = graph_replay_us(torch, stream, step)
            if g_us is not None:
                res[key]["us_quantize_plus_gemm_graph_replay"] = round(g_us, 2)
                log(f"{wl.name}: quantize + gemm replayed from a HIP graph {g_us:.1f} us")
    return res


PARTS = {"small", "decode", "gdn_in_proj", "gdn", "kv", "variants", "context"}


def decode(nv, W, torch, dev, stream, log):
    """Decode-shape weight streaming: M=8 x [34816, 5120] (gate|up, two
    segments), ROTATE rotating weight copies so reads come from HBM, not the
    256 MB MALL.  Two GEMM paths on pre-quantized activations: the row-major
    weight (nvfp4_gemm_fused_segments) and the weight in the decode layout
    (packed offline, like its quantization; nvfp4_gemm_decode); gemm_us is
    the faster, both are reported.  quantize_plus_gemm = the whole linear
    layer, nvfp4_linear_decode (activations quantized inside the launch),
    beside the two-launch quantize + row-major GEMM."""
    res = {}
    log(f"decode M=8 x 34816x5120: {ROTATE} rotating NVFP4 weight copies")
    dw = W.decode()
    xd = dw.x.to(dev)
    segs = [w for _, w in dw.weights]
    rows = sum(w.shape[0] for w in segs)
    kk = segs[0].shape[1]
    base = nv.empty_nvfp4(rows, kk, dev)
    g = torch.empty(len(segs), dtype=torch.float32, device=dev)
    ws = nv.workspace_for(segs[0].shape[0], kk, dev)
    offs = [0]
    for s, w in enumerate(segs):
        part = base.row_slice(offs[-1], offs[-1] + w.shape[0])
        nv.nvfp4_quantize(w.to(dev), nv.NVFP4Tensor(part.codes, part.scales, g[s:s + 1], part.rows, kk),
                          nv.SCALE_DYNAMIC, ws)
        offs.append(offs[-1] + w.shape[0])
    packed = [nv.pack_decode(base) for _ in range(ROTATE)]
    rowmajor = [base] + [nv.NVFP4Tensor(base.codes.clone(), base.scales.clone(), base.global_scale, rows, kk)
                         for _ in range(ROTATE - 1)]
    ad = nv.quantize(xd)
    outd = torch.empty((xd.shape[0], rows), dtype=torch.bfloat16, device=dev)
    wsd = nv.workspace_for(xd.shape[0], kk, dev)
    iters = 200

    def timed(fn):
        for i in range(8):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(iters):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters * 1e-3

    t_gemm = timed(lambda i: nv.nvfp4_gemm_decode(ad, packed[i % ROTATE], offs, g, outd))
    t_full = timed(lambda i: nv.nvfp4_linear_decode(xd, packed[i % ROTATE], offs, g, outd))
    t_row = timed(lambda i: nv.nvfp4_gemm_fused_segments(ad, rowmajor[i % ROTATE], offs, g, outd))
    t_row_q = timed(lambda i: (nv.nvfp4_quantize(xd, ad, nv.SCALE_DYNAMIC, wsd),
                               nv.nvfp4_gemm_fused_segments(ad, rowmajor[i % ROTATE], offs, g, outd)))
    # context, not a kernel of this library: torch reading the same rotating
    # 100 MB weight copies once (a max-reduction over their bytes)
    flat = [p.data.view(torch.int32) for p in packed]
    t_ctx = timed(lambda i: torch.amax(flat[i % ROTATE]))
    m = xd.shape[0]
    alg_bytes = rows * kk // 2 + rows * kk // 16 + m * kk // 2 + m * kk // 16 + m * rows * 2
    alg_full = rows * kk // 2 + rows * kk // 16 + m * kk * 2 + m * rows * 2
    best = min(t_gemm, t_row)
    res["decode_m8"] = {"workload": dw.name, "algorithmic_bytes": alg_bytes,
                        "gemm_us": round(best * 1e6, 2),
                        "gemm_GBps": round(alg_bytes / best / 1e9, 1),
                        "frac_of_hbm_peak": round(alg_bytes / best / 1e9 / HBM_PEAK_GBS, 4),
                        "gemm_path": "decode layout" if t_gemm <= t_row else "row-major",
                        "gemm_rowmajor_us": round(t_row * 1e6, 2),
                        "gemm_decode_layout_us": round(t_gemm * 1e6, 2),
                        "quantize_plus_gemm_us": round(t_full * 1e6, 2),
                        "quantize_plus_gemm_frac_of_hbm_peak": round(alg_full / t_full / 1e9 / HBM_PEAK_GBS, 4),
                        "quantize_plus_gemm_path": "nvfp4_linear_decode (activations quantized in the launch)",
                        "rowmajor_quantize_plus_gemm_us": round(t_row_q * 1e6, 2),
                        "context_torch_read_weight_us": round(t_ctx * 1e6, 2),
                        "context_torch_read_weight_GBps": round(flat[0].numel() * 4 / t_ctx / 1e9, 1)}
    log(f"decode: gemm {best * 1e6:.1f} us = {alg_bytes / best / 1e9:.0f} GB/s (row-major {t_row * 1e6:.1f}, decode "
        f"layout {t_gemm * 1e6:.1f} us); linear layer with in-launch quantization {t_full * 1e6:.1f} us; "
        f"row-major quantize + gemm {t_row_q * 1e6:.1f} us; torch reading the weight once {t_ctx * 1e6:.1f} us")
    del packed, rowmajor, base, outd, flat
    return res


def gdn_in_proj(nv, W, torch, dev, stream, log):
    """The 32768-token fused GDN in-projection with gates (six segments),
    and the scale-harmonization study on it."""
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log("fused GDN in-projection 32768 x 16480 x 5120 with gates")
    gw = W.gdn_in_proj()
    xg = gw.x.to(dev)
    segs = [w for _, w in gw.weights]
    rows = sum(w.shape[0] for w in segs)
    kk = segs[0].shape[1]
    wq = nv.empty_nvfp4(rows, kk, dev)
    sg = torch.empty(len(segs), dtype=torch.float32, device=dev)
    offs = [0]
    ws = nv.workspace_for(max(w.shape[0] for w in segs), kk, dev)
    for s, w in enumerate(segs):
        part = wq.row_slice(offs[-1], offs[-1] + w.shape[0])
        nv.nvfp4_quantize(w.to(dev), nv.NVFP4Tensor(part.codes, part.scales, sg[s:s + 1], part.rows, kk),
                          nv.SCALE_DYNAMIC, ws)
        offs.append(offs[-1] + w.shape[0])
    gate = dict(b_segment=4, a_segment=5, A_log=gw.extra["A_log"].to(dev), dt_bias=gw.extra["dt_bias"].to(dev))
    ag = nv.empty_nvfp4(xg.shape[0], kk, dev)
    wsg = nv.workspace_for(xg.shape[0], kk, dev)
    outg = torch.empty((xg.shape[0], rows), dtype=torch.bfloat16, device=dev)

    def gstep():
        nv.nvfp4_quantize(xg, ag, nv.SCALE_DYNAMIC, wsg)
        nv.nvfp4_gemm_fused_segments(ag, wq, offs, sg, outg, gate)
    for _ in range(2):
        gstep()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        gstep()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 5 * 1e-3
    fl = 2.0 * xg.shape[0] * rows * kk
    res["gdn_in_proj_m32768"] = {"workload": gw.name, "ms": round(t * 1e3, 3),
                                 "TFLOPs_incl_act_quant": round(fl / t / 1e12, 1),
                                 "frac_of_mfma_peak": round(fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}
    log(f"gdn in-proj: {t * 1e3:.3f} ms = {fl / t / 1e12:.0f} TFLOP/s")
    res["scale_harmonization_gdn_in_proj"] = harmonization_study(nv, torch, stream, log, gw, ag, wq, offs, sg, gate)
    del outg
    return res


def gdn_study(nv, W, torch, stream, log, dev):
    """The gated delta-rule recurrence of one synthetic GDN layer (32K tokens,
    48 value heads, 16 key heads, 128 wide; gate projections scaled to the
    pages' decay horizons): its time, and the pages' two recurrence
    measurements -- relS, the relative state error of
    the NVFP4-quantized layer against an unquantized (bf16 weights and
    activations, float32 products) in-projection, along the sequence; and the
    erasure of a state impulse (10 % of |S|) injected at token 8192, in steps
    until it falls below 1/e and 10 %, beside each head's pure-decay horizon
    1 / mean(-g), the keys' effective rank, and the same erasure with the
    keys replaced by isotropic random directions."""
    gw = W.gdn_layer()
    xg = gw.x.to(dev)
    T = xg.shape[0]
    segs = [t.to(dev) for _, t in gw.weights]
    wq = nv.empty_nvfp4(sum(t.shape[0] for t in segs), xg.shape[1], dev)
    sg = torch.empty(len(segs), dtype=torch.float32, device=dev)
    offs = [0]
    wsq = nv.workspace_for(max(t.shape[0] for t in segs), xg.shape[1], dev)
    for i, t in enumerate(segs):
        part = wq.row_slice(offs[-1], offs[-1] + t.shape[0])
        nv.nvfp4_quantize(t, nv.NVFP4Tensor(part.codes, part.scales, sg[i:i + 1], part.rows, part.cols),
                          nv.SCALE_DYNAMIC, wsq)
        offs.append(offs[-1] + t.shape[0])
    gate = dict(b_segment=4, a_segment=5, A_log=gw.extra["A_log"].to(dev), dt_bias=gw.extra["dt_bias"].to(dev))
    ag = nv.quantize(xg)
    hk, hv = (offs[1] - offs[0]) // 128, (offs[3] - offs[2]) // 128
    outq = nv.gemm_fused_segments(ag, wq, offs, sg, gate, out_dtype=torch.float32)
    cols = lambda o, s: o[:, offs[s]:offs[s + 1]]
    ws = torch.empty(nv.nvfp4_gdn_workspace_bytes(T, hv) // 4, dtype=torch.float32, device=dev)
    o = torch.empty((T, hv * 128), dtype=torch.float32, device=dev)
    run = lambda src: nv.nvfp4_gdn_recurrence(cols(src, 0), cols(src, 1), cols(src, 2), cols(src, 4), cols(src, 5),
                                              o, hk, hv, ws)
    ms = time_steps(torch, stream, lambda: run(outq), steps=3, warmup=1)
    flops = 8.0 * 128 * 128 * T * hv  # S k, two rank-1 updates, S q per token and head
    log(f"gdn recurrence {T} tokens x {hv} heads: {ms:.2f} ms = {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s (fp32)")

    # unquantized reference in-projection with the same gate formulas
    w = torch.cat(segs).float()
    del segs
    ref = xg.float() @ w.t()
    del w
    b0, a0 = offs[4], offs[5]
    a_log, dt_bias = gate["A_log"].float(), gate["dt_bias"].float()
    ref[:, b0:offs[5]] = torch.sigmoid(ref[:, b0:offs[5]])
    ref[:, a0:offs[6]] = -torch.exp(a_log) * torch.nn.functional.softplus(ref[:, a0:offs[6]] + dt_bias)

    def states(src, bounds, s_init=None, t_begin=0):
        """States after each prefix end in `bounds`, carrying the state across calls."""
        out, s = [], s_init
        t_prev = t_begin
        for t_end in bounds:
            sl = slice(t_prev, t_end)
            wsl = torch.empty(nv.nvfp4_gdn_workspace_bytes(t_end - t_prev, hv) // 4, dtype=torch.float32, device=dev)
            osl = torch.empty((t_end - t_prev, hv * 128), dtype=torch.float32, device=dev)
            s_new = torch.empty((hv, 128, 128), dtype=torch.float32, device=dev)
            nv.nvfp4_gdn_recurrence(cols(src, 0)[sl], cols(src, 1)[sl], cols(src, 2)[sl], cols(src, 4)[sl],
                                    cols(src, 5)[sl], osl, hk, hv, wsl, s0=s, s_final=s_new)
            out.append(s_new)
            s, t_prev = s_new, t_end
        return out

    marks = [256, 1024] + list(range(2048, T + 1, 2048))
    sq_, sr_ = states(outq, marks), states(ref, marks)
    rel = [((a - b).flatten(1).norm(dim=1) / b.flatten(1).norm(dim=1)) for a, b in zip(sq_, sr_)]
    rels = {str(m): {"mean": round(r.mean().item(), 4), "min": round(r.min().item(), 4), "max": round(r.max().item(), 4)}
            for m, r in zip(marks, rel)}
    log("relS mean: " + ", ".join(f"{m}:{v['mean']:.3f}" for m, v in rels.items()))

    # impulse erasure: a state impulse of 10 % of |S| injected at token
    # 8192, followed against the unperturbed run
    t0 = 8192
    ends = list(range(t0 + 16, t0 + 1025, 16)) + list(range(t0 + 1152, min(T, t0 + 8192) + 1, 128))
    steps = torch.tensor([e - t0 for e in ends], device=dev, dtype=torch.float32)

    def erasure(src, seed):
        s_t0 = states(src, [t0])[0]
        gen = torch.Generator(device=dev).manual_seed(seed)
        imp = torch.randn(s_t0.shape, device=dev, generator=gen)
        imp *= (0.1 * s_t0.flatten(1).norm(dim=1) / imp.flatten(1).norm(dim=1))[:, None, None]
        base = states(src, ends, s_init=s_t0, t_begin=t0)
        pert = states(src, ends, s_init=s_t0 + imp, t_begin=t0)
        norm0 = imp.flatten(1).norm(dim=1)
        ratio = torch.stack([(p_ - b_).flatten(1).norm(dim=1) / norm0 for p_, b_ in zip(pert, base)])  # [steps, hv]

        def first_below(th):
            below = ratio < th
            idx = torch.where(below.any(dim=0), below.float().argmax(dim=0), torch.full((hv,), len(ends) - 1, device=dev))
            return steps[idx]
        e1, e10 = first_below(float(torch.exp(torch.tensor(-1.0)))), first_below(0.1)
        return ({"median": e1.median().item(), "min": e1.min().item(), "max": e1.max().item()},
                {"median": e10.median().item(), "min": e10.min().item(), "max": e10.max().item()})

    def key_effective_rank(src):
        """Participation ratio (tr C)^2 / tr(C^2) of the unit keys' second
        moment C per key head: 128 for isotropic keys, r for keys spread
        evenly over r directions."""
        kn = cols(src, 1).reshape(T, hk, 128).permute(1, 0, 2)
        kn = kn / kn.norm(dim=2, keepdim=True).clamp_min(1e-30)
        c = torch.matmul(kn.transpose(1, 2).contiguous(), kn) / T  # [hk, 128, 128]
        pr = c.diagonal(dim1=1, dim2=2).sum(dim=1) ** 2 / (c * c).sum(dim=(1, 2))
        return {"median": round(pr.median().item(), 1), "min": round(pr.min().item(), 1),
                "max": round(pr.max().item(), 1)}

    e1, e10 = erasure(ref, 0)
    horizon = 1.0 / (-ref[:, a0:offs[6]].mean(dim=0))
    rank_layer = key_effective_rank(ref)
    # the same dynamics (beta, g, q, v) with the keys replaced by isotropic
    # random directions: how much of the erasure time the keys' spread sets
    iso = ref.clone()
    gen = torch.Generator(device=dev).manual_seed(1)
    iso[:, offs[1]:offs[2]] = torch.randn((T, offs[2] - offs[1]), device=dev, generator=gen)
    rank_iso = key_effective_rank(iso)
    e1_iso, e10_iso = erasure(iso, 0)
    del iso
    imp_res = {"steps_to_1_over_e": e1, "steps_to_10pct": e10,
               "pure_decay_horizon_tokens": {"median": round(horizon.median().item(), 1),
                                             "min": round(horizon.min().item(), 1),
                                             "max": round(horizon.max().item(), 1)},
               "key_effective_rank": rank_layer,
               "isotropic_keys": {"steps_to_1_over_e": e1_iso, "steps_to_10pct": e10_iso,
                                  "key_effective_rank": rank_iso},
               "resolution_tokens": "16 up to 1024 steps, then 128"}
    log(f"impulse: 1/e after median {e1['median']:.0f} steps "
        f"(pure-decay horizon median {imp_res['pure_decay_horizon_tokens']['median']:.0f} tokens); "
        f"keys' effective rank median {rank_layer['median']}; isotropic keys (rank {rank_iso['median']}): "
        f"1/e after median {e1_iso['median']:.0f} steps")
    del ref, outq
    return {"ms": round(ms, 3), "tflops_fp32": round(flops / (ms * 1e-3) / 1e12, 2),
            "algorithmic_flops": flops, "relS_vs_unquantized": rels, "impulse_erasure": imp_res,
            "note": "q and k L2-normalized straight from the in-projection (no short convolution)"}


def harmonization_study(nv, torch, stream, log, gw, ag, wq, offs, sg, gate):
    """The global-scale mismatch and its checkpoint-side repair on the 32K
    GDN in-projection with gates: per module, the relative error against the
    per-module-scale result (this library's fused epilogue) of (a) serving
    module q's scale for every column and (b) the harmonized weight served
    with one global scale; plus the harmonization kernel's time."""
    n = len(offs) - 1
    hw = nv.harmonize_scales(wq, offs, sg)
    hs_buf, g_buf = torch.empty_like(wq.scales), torch.empty(1, dtype=torch.float32, device=wq.codes.device)
    t_h = time_steps(torch, stream, lambda: nv.nvfp4_harmonize_scales(wq, offs, sg, hs_buf, g_buf), steps=20)
    ref = nv.gemm_fused_segments(ag, wq, offs, sg, gate, out_dtype=torch.float32)
    fixed = nv.gemm_fused_segments(ag, hw, offs, hw.global_scale.repeat(n), gate, out_dtype=torch.float32)
    bad = nv.gemm_fused_segments(ag, wq, offs, sg[:1].repeat(n), gate, out_dtype=torch.float32)
    torch.cuda.synchronize()
    names = [nm for nm, _ in gw.weights]
    per = {}
    for i, nm in enumerate(names):
        c = slice(offs[i], offs[i + 1])
        den = torch.linalg.vector_norm(ref[:, c].double()).item()
        per[nm] = {"harmonized": round(torch.linalg.vector_norm((fixed[:, c] - ref[:, c]).double()).item() / den, 6),
                   "mismatch": round(torch.linalg.vector_norm((bad[:, c] - ref[:, c]).double()).item() / den, 6)}
    del ref, fixed, bad
    log("harmonization: " + ", ".join(f"{k} {v['harmonized']:.4f}/{v['mismatch']:.4f}" for k, v in per.items()))
    return {"relative_error_vs_per_module_scales": per,
            "outputs": "b and a columns are the gate outputs (sigmoid, decay) of each variant",
            "harmonize_kernel_us": round(t_h * 1e3, 2)}


def cpu_baseline(nv, W, torch, np, wl, a, w_gu, gu_offs, gu_g, w_d, d_offs, d_g, rows, log):
    """The oracle, as it stands, on the first `rows` rows of the same MLP
    pair step (quantize X rows with the step's global scale, fused gate|up,
    SiLU*mul, quantize h rows, down), on the host's cores."""
    from threadpoolctl import threadpool_info

    from oracle import nvfp4_oracle as O

    torch.cuda.synchronize()
    k = a.cols
    inter = w_d.cols
    xs = W.bf16_to_f32_numpy(wl.x[:rows])
    g_x = np.float32(a.global_scale.cpu().numpy()[0])
    wgc = w_gu.codes[:, : k // 2].cpu().numpy()
    wgs = w_gu.scales[:, : k // 16].cpu().numpy()
    wdc = w_d.codes[:, : inter // 2].cpu().numpy()
    wds = w_d.scales[:, : inter // 16].cpu().numpy()
    gg = gu_g.cpu().numpy()
    dg = d_g.cpu().numpy()
    log(f"cpu oracle on {rows} rows of the step")
    t0 = time.perf_counter()
    ac, as_, ag = O.quantize(xs, g_x)
    gu, _ = O.fused_segments(ac, as_, ag, wgc, wgs, gu_offs, gg, k, with_tol=False)
    hh = O.silu_mul(O.round_bf16(gu[:, :inter]), O.round_bf16(gu[:, inter:]))
    hc, hs, hg = O.quantize(hh.astype(np.float32))
    out, _ = O.fused_segments(hc, hs, hg, wdc, wds, d_offs, dg, inter, with_tol=False)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * (2 * inter * k + k * inter)
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    log(f"cpu oracle: {dt:.1f} s")
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"first {rows} of 8192 rows of the MLP pair step (quantize X, fused gate|up, "
                      f"SiLU*mul, quantize h, down) in float64 numpy; weight dequantization inside "
                      f"each GEMM call as the oracle does it; host affinity {len(os.sched_getaffinity(0))} cpus"}


if __name__ == "__main__":
    main()
