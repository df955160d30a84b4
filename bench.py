#!/usr/bin/env python3
"""Benchmark: BitNet b1.58 BitLinear W1.58A8 decode through a 2B-shaped stack on one MI355X.

Workload: one token (M = 1) through 30 layers of the 2B-shaped BitLinears
(QKV 2560->3840, O 2560->2560, gate+up 2560->13824, down 6912->2560), 120
independent ternary matrices (N(0, 0.02) weights, absmean-ternarized and packed
once at 2 bits), each with its own seeded bf16 input row (N(0, 1) with 8
outlier channels x20).  A step is one pass over the stack: for every linear,
the per-token int8 quantization (bl_quant_act) and the packed-ternary product
with the bf16 rescale (bl_linear), which bl_bitlinear runs as one kernel.  Weights are prepared once (bl_ternarize_pack)
before timing, as a deployed model does; the packer's throughput is reported
separately.  All inputs are resident in HBM when timing starts; the packed
stack (521 MB) is larger than the 256 MB Infinity Cache, so every step streams
the weights from HBM.

Prints one JSON line.  value = decode tokens/s with the step replayed as a
captured HIP graph.  roofline = the decode GEMV kernel: algorithmic bytes per
launch / its average launch duration, measured with HIP events on the stream
the kernels run on.  cpu_baseline = the CPU oracle on a bounded sample of the
same stack (rank 0, N = 1 only).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BitLinear W1.58A8 decode weight GB/s & tokens/s; prefill int8 TOPS"
HBM_PEAK_GBPS = 8000.0


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--layers", type=int, default=30, help="layers of the 2B-shaped stack (30 = the full model)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="bound on the CPU-oracle timing sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(the BitLinear path runs on a single MI355X).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lib = bl.library()
    wl = datagen.WORKLOAD_STACK_2B
    proj = datagen.STACK_2B_PROJ
    m = 1

    # ------------------------------------------------------------ weights, once
    ws = torch.empty(bl.bl_ternarize_pack_workspace_bytes(2560, 2560), dtype=torch.uint8, device=dev)
    linears = []
    pack_ms = 0.0
    w_bytes = 0
    outliers = {k: datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS) for _, k, _ in proj}
    for layer in range(args.layers):
        for pi, (name, k, n) in enumerate(proj):
            w = datagen.weights(datagen.stream_id(wl, layer, pi, datagen.TENSOR_W), n, k)
            wd = torch.from_numpy(w).to(dev)
            packed = torch.empty(bl.bl_packed_bytes(n, k), dtype=torch.uint8, device=dev)
            gamma = torch.empty(1, dtype=torch.float32, device=dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bl.bl_ternarize_pack(wd, packed, gamma, ws)
            e1.record()
            e1.synchronize()
            pack_ms += e0.elapsed_time(e1)
            w_bytes += wd.numel() * 4
            del wd
            x = datagen.activations_bf16(datagen.stream_id(wl, layer, pi, datagen.TENSOR_X), m, k, outliers[k],
                                         datagen.STACK_2B_OUTLIER_MULT)
            xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
            linears.append(dict(name=name, n=n, k=k, packed=packed, gamma=gamma, x=xd,
                                xq=torch.empty((m, k), dtype=torch.int8, device=dev),
                                alpha=torch.empty(m, dtype=torch.float32, device=dev),
                                y=torch.empty((m, n), dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    print(f"[bench] packed {len(linears)} BitLinears ({sum(l['packed'].numel() for l in linears) / 1e6:.1f} MB)",
          file=sys.stderr, flush=True)

    vp = ctypes.c_void_p
    calls = []
    for lin in linears:
        calls.append((vp(lin["packed"].data_ptr()), vp(lin["gamma"].data_ptr()), vp(lin["x"].data_ptr()),
                      lin["n"], lin["k"], vp(lin["xq"].data_ptr()), vp(lin["alpha"].data_ptr()),
                      vp(lin["y"].data_ptr())))

    def step(select=None):
        """One token through the stack: bl_bitlinear (per-token int8 quantization,
        packed-ternary product, bf16 rescale) for every linear in order."""
        s = vp(torch.cuda.current_stream().cuda_stream)
        for i, (packed, gamma, x, n, k, xq, alpha, y) in enumerate(calls):
            if select is not None and i not in select:
                continue
            rc = lib.bl_bitlinear(packed, gamma, x, m, n, k, xq, alpha, None, y, s)
            if rc:
                raise RuntimeError(f"bl_bitlinear failed on linear {i}: {bl.bl_status_string(rc)}")

    def capture(select=None):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(select)
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            step(select)
        return g

    def time_graph(g, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # per-linear algorithmic bytes: packed W + bf16 x + int8 xq and alpha written + gamma + bf16 y
    layer_bytes = [bl.bl_packed_bytes(l["n"], l["k"]) + 2 * m * l["k"] + m * l["k"] + 4 * m + 4 + 2 * m * l["n"]
                   for l in linears]
    weight_bytes_step = sum(bl.bl_packed_bytes(l["n"], l["k"]) for l in linears)

    # ------------------------------------------------------------ eager (host-launched) reference
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eager_steps = max(1, min(args.steps, 50))
    t0.record()
    for _ in range(eager_steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1) / eager_steps

    # ------------------------------------------------------------ graph capture + timed region
    graph = capture()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms_per_step = time_graph(graph, args.steps)
    wall = time.perf_counter() - wall0
    tokens_per_s = m * 1000.0 / ms_per_step

    # ------------------------------------------------------------ per-kernel duration (live, HIP events)
    # The step is one kernel launch per linear, back to back in the graph, so the
    # timed region above is the dominant kernel's launches end to end: its
    # average duration is the step time over the launch count (gaps included).
    avg_us = 1000.0 * ms_per_step / len(linears)
    avg_bytes = sum(layer_bytes) / len(layer_bytes)
    gemv_gbps = avg_bytes / (avg_us * 1e-6) / 1e9

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, outliers)

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,0.02) weights absmean-ternarized; N(0,1) bf16 tokens, 8 outlier channels x20)",
        "config": {"workload": "bitnet-b1.58-2B-shaped decode stack, M=1",
                   "layers": args.layers, "linears_per_layer": 4,
                   "shapes_KxN": [f"{k}x{n}" for _, k, n in proj],
                   "launch": "HIP graph, one bl_bitlinear (fused quantize + product) per linear"},
        "decode_weight_GBps": round(weight_bytes_step / (ms_per_step * 1e-3) / 1e9, 1),
        "eager": {"ms_per_step": round(eager_ms, 4), "tokens_per_s": round(m * 1000.0 / eager_ms, 2)},
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": "k_gemv_lds<fused> (bl_bitlinear)", "achieved": round(gemv_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gemv_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "avg_launch_us": round(avg_us, 3),
                     "algorithmic_bytes_per_launch": round(avg_bytes, 1)},
        "packer": {"weights": len(linears), "fp32_GB": round(w_bytes / 1e9, 3), "ms": round(pack_ms, 3),
                   "GBps_fp32_read": round(w_bytes / (pack_ms * 1e-3) / 1e9, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline(args, outliers):
    """The CPU oracle (plain C, OpenMP over output rows) on a bounded sample:
    the first layer's four linears of the same stack, one token each,
    repeated until about --cpu-seconds of CPU time; scaled to tokens/s of the
    full stack.  The oracle packs its own weights (untimed, offline)."""
    import datagen
    import oracle

    wl = datagen.WORKLOAD_STACK_2B
    proj = datagen.STACK_2B_PROJ
    prepared = []
    for pi, (name, k, n) in enumerate(proj):
        w = datagen.weights(datagen.stream_id(wl, 0, pi, datagen.TENSOR_W), n, k)
        packed, gamma = oracle.ternarize_pack(w)
        x = datagen.activations_bf16(datagen.stream_id(wl, 0, pi, datagen.TENSOR_X), 1, k, outliers[k],
                                     datagen.STACK_2B_OUTLIER_MULT)
        prepared.append((packed, gamma, x, n))
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    done = 0
    t0 = time.perf_counter()
    while True:
        for packed, gamma, x, n in prepared:
            oracle.bitlinear_forward(packed, gamma, x, n)
        done += 1
        elapsed = time.perf_counter() - t0
        if elapsed >= args.cpu_seconds:
            break
    layers_per_s = done / elapsed
    return {"value": round(layers_per_s / args.layers, 4), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"layer 0 of the 2B-shaped stack (4 linears, M=1) run {done}x in {elapsed:.1f} s; "
                      f"tokens/s = layers/s / {args.layers}"}


if __name__ == "__main__":
    sys.exit(main())
