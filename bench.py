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
    p.add_argument("--no-extras", action="store_true",
                   help="skip the prefill, batched-decode and 70B-shaped measurements")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only copy a 1 GiB device buffer 3 times (counter calibration run)")
    p.add_argument("--profile", choices=sorted(PROFILE_CASES), default=None,
                   help="only run one workload a few times (a short program for rocprofv3)")
    p.add_argument("--reps", type=int, default=3, help="repetitions for --profile")
    p.add_argument("--summarize", metavar="NAME", default=None,
                   help="write profiles/NAME.md from rocprofv3 outputs (no GPU needed)")
    p.add_argument("--title", default="")
    p.add_argument("--workload", default="", help="workload the summary covers (key in profiles/traffic.json)")
    p.add_argument("--stats", default=None, help="rocprofv3 --kernel-trace --stats output directory")
    p.add_argument("--pmc", action="append", default=[], help="rocprofv3 --pmc output directory (repeatable)")
    p.add_argument("--calib", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                   help="FETCH_SIZE and WRITE_SIZE runs of --calibrate-copy")
    p.add_argument("--command", action="append", default=[], help="command that produced an input (repeatable)")
    p.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"), help="where --summarize writes")
    return p.parse_args()


def main() -> int:
    args = parse_args()
    if args.summarize:
        return summarize(args)
    if args.profile:
        if args.gpus != 1:
            print("--profile runs on one GPU", file=sys.stderr)
            return 2
        return PROFILE_CASES[args.profile](args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the BitLinear path runs on a single MI355X).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copied 3 x 1 GiB", flush=True)
        return 0

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
    layer0_w = []  # fp32 weights of layer 0, kept for the packer's timing
    outliers = {k: datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS) for _, k, _ in proj}
    for layer in range(args.layers):
        for pi, (name, k, n) in enumerate(proj):
            w = datagen.weights(datagen.stream_id(wl, layer, pi, datagen.TENSOR_W), n, k)
            wd = torch.from_numpy(w).to(dev)
            packed = torch.empty(bl.bl_packed_bytes(n, k), dtype=torch.uint8, device=dev)
            gamma = torch.empty(1, dtype=torch.float32, device=dev)
            bl.bl_ternarize_pack(wd, packed, gamma, ws)
            if layer == 0:
                layer0_w.append((wd, n, k))
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

    # each projection's launches alone (30 of one shape back to back in a graph)
    per_projection = {}
    for name, k, n in proj:
        sel = {i for i, l in enumerate(linears) if l["name"] == name}
        us = 1000.0 * time_graph(capture(sel), max(args.steps, 20)) / len(sel)
        wb = bl.bl_packed_bytes(n, k)
        per_projection[name] = {"KxN": f"{k}x{n}", "us_per_launch": round(us, 3),
                                "weight_GBps": round(wb / (us * 1e-6) / 1e9, 1),
                                "weights_MB": round(wb * len(sel) / 1e6, 1),
                                # the 30 matrices of one shape: below 256 MB the Infinity Cache can hold them
                                "cache_resident": wb * len(sel) <= INFINITY_CACHE_BYTES}

    extras = None
    if not args.no_extras:
        extras = measure_extras(args, linears, lib)
    stream = stream_reference(torch)
    floor_us = graph_node_floor_us(torch, len(linears))
    ceiling_us = floor_us + avg_bytes / (stream["read_GBps"] * 1e3)

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, outliers)

    # the packer (offline for decode): layer 0's four matrices re-packed,
    # timed as graph replays (launch gaps spread over 5 calls per replay)
    pk_out = [(torch.empty(bl.bl_packed_bytes(n, k), dtype=torch.uint8, device=dev),
               torch.empty(1, dtype=torch.float32, device=dev)) for _, n, k in layer0_w]

    def pack_layer0():
        s = vp(torch.cuda.current_stream().cuda_stream)
        for (wd, n, k), (pk, gm) in zip(layer0_w, pk_out):
            rc = lib.bl_ternarize_pack(vp(wd.data_ptr()), n, k, vp(pk.data_ptr()), vp(gm.data_ptr()),
                                       vp(ws.data_ptr()), ws.numel(), s)
            if rc:
                raise RuntimeError(bl.bl_status_string(rc))

    pack_ms = _graph_time_ms(torch, _repeat(pack_layer0, 5), 5) / 5
    w0_bytes = sum(4 * n * k for _, n, k in layer0_w)
    packer = {"matrices": len(layer0_w), "fp32_MB": round(w0_bytes / 1e6, 1), "ms": round(pack_ms, 4),
              "us_per_matrix": round(1000 * pack_ms / len(layer0_w), 2),
              "GBps_fp32_read": round(w0_bytes / (pack_ms * 1e-3) / 1e9, 1),
              "note": "layer 0 of the stack; each weight is read twice (absmean pass, ternarize pass)"}
    del layer0_w, pk_out

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
        "config": {"workload": STACK_WORKLOAD,
                   "layers": args.layers, "linears_per_layer": 4,
                   "shapes_KxN": [f"{k}x{n}" for _, k, n in proj],
                   "launch": "HIP graph, one bl_bitlinear (fused quantize + product) per linear"},
        "decode_weight_GBps": round(weight_bytes_step / (ms_per_step * 1e-3) / 1e9, 1),
        "eager": {"ms_per_step": round(eager_ms, 4), "tokens_per_s": round(m * 1000.0 / eager_ms, 2)},
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": f"{STACK_KERNEL} (bl_bitlinear, all {len(linears)} launches)",
                     "time_source": (f"HIP events around {args.steps} replays of the captured step ({len(linears)} "
                                     "launches back to back on one stream); per launch = step time / launches, "
                                     "the gap between dependent launches included"),
                     "achieved": round(gemv_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gemv_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": stored_traffic(STACK_WORKLOAD, STACK_KERNEL, avg_bytes),
                     "avg_launch_us": round(avg_us, 3),
                     "algorithmic_bytes_per_launch": round(avg_bytes, 1),
                     "measured_hbm_reference": stream,
                     "frac_of_measured_read": round(gemv_gbps / stream["read_GBps"], 4),
                     "graph_node_floor_us": floor_us,
                     # per-launch lower bound: the node floor plus the weight bytes at the measured read rate
                     "launch_bound_ceiling_us": round(ceiling_us, 3),
                     "frac_of_launch_bound_ceiling": round(ceiling_us / avg_us, 4),
                     "per_projection": per_projection},
        "packer": packer,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(result), flush=True)
    return 0


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
INFINITY_CACHE_BYTES = 256 * 1000 ** 2  # MI355X last-level (MALL) cache
MFMA_I8_PEAK_TOPS = 5000.0
CALIB_BYTES = 1 << 30
STACK_WORKLOAD = "bitnet-b1.58-2B-shaped decode stack, M=1"
STACK_KERNEL = "k_bitlinear_m1"
# kernel base name -> source file whose hash marks the stored counter figures as current
KERNEL_SOURCES = {"k_bitlinear_m1": "gemv.hip", "k_bitlinear_fused": "gemv.hip", "k_gemv_direct": "gemv.hip",
                  "k_bitlinear_tok": "gemv.hip", "k_bitlinear_b3": "b3.hip", "k_bitlinear_b3_band": "b3.hip",
                  "k_gemv_lds": "gemv.hip", "k_gemv_ring": "gemv.hip", "k_gemm": "gemm.hip", "k_quant_act": "quant.hip",
                  "k_bwd_x": "backward.hip", "k_bwd_w": "backward.hip", "k_bwd_w_prep": "backward.hip"}
# operations per MFMA instruction: int8 16 x 16 x 64 (the forward kernels),
# bf16 16 x 16 x 32 (the backward kernels), two per multiply-add
MFMA_OPS = {"k_bwd_x": 16384, "k_bwd_w": 16384}
MFMA_OPS_DEFAULT = 32768
CU_SIMDS = 256 * 4
CLOCK_GHZ = 2.4


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def _base_name(name: str) -> str:
    """'bl::(anonymous namespace)::k_gemm<8>(...)' -> 'k_gemm'."""
    short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0].replace("bl::", "")
    return short.split("<")[0].strip()


def _per_kernel(rows, counter):
    """Average per dispatch of `counter`, and mean dispatch duration (ns), per kernel base name."""
    import collections
    vals, durs = collections.defaultdict(list), collections.defaultdict(list)
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        base = _base_name(r["Kernel_Name"])
        vals[base].append(float(r["Counter_Value"]))
        durs[base].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return {b: (sum(v) / len(v), sum(durs[b]) / len(durs[b]), len(v)) for b, v in vals.items()}


def summarize(args):
    """profiles/NAME.md from rocprofv3 outputs: kernel durations (kernel-trace
    stats), per-dispatch counters of each --pmc run, and, with --calib, HBM
    bytes per launch from FETCH_SIZE + WRITE_SIZE scaled by what the same
    counters read for a 1 GiB device copy.  MFMA utilisation, when the
    counters are present: SQ_VALU_MFMA_BUSY_CYCLES over the dispatch's
    duration x 1024 SIMDs x 2.4 GHz."""
    import collections
    name = args.summarize
    lines = [f"# {args.title or name}", ""]
    if args.workload:
        lines += [f"Workload: {args.workload}", ""]
    lines += ["Commands (run from the repository root on one MI355X; `cd /tmp && export TMPDIR=/tmp` first):", "", "```"]
    lines += args.command + ["```", ""]
    stats_rows = _read_csv(_find(args.stats, "kernel_stats.csv")) if args.stats else []
    grouped = collections.OrderedDict()
    for r in stats_rows:
        base = _base_name(r["Name"])
        g = grouped.setdefault(base, {"calls": 0, "total": 0.0, "min": float("inf"), "max": 0.0})
        g["calls"] += int(r["Calls"])
        g["total"] += float(r["TotalDurationNs"])
        g["min"] = min(g["min"], float(r["MinNs"]))
        g["max"] = max(g["max"], float(r["MaxNs"]))
    # the later half of each kernel's dispatches (the timed steps, after the
    # warmup and the eager passes) from the per-dispatch trace
    late = {}
    try:
        trace = _find(args.stats, "kernel_trace.csv") if args.stats else None
    except FileNotFoundError:  # a stats directory without the per-dispatch trace
        trace = None
    s2s = {}
    if trace:
        per = collections.defaultdict(list)
        rows = sorted(_read_csv(trace), key=lambda r: int(r["Start_Timestamp"]))
        for r in rows:
            per[_base_name(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        late = {k: sum(v[len(v) // 2:]) / len(v[len(v) // 2:]) for k, v in per.items() if v}
        # start-to-start interval of consecutive dispatches of the same kernel
        # (graph replays: one launch after the other), gaps over 100 us
        # (between replays, or host work) left out
        gaps = collections.defaultdict(list)
        for a, b in zip(rows, rows[1:]):
            ka, kb = _base_name(a["Kernel_Name"]), _base_name(b["Kernel_Name"])
            d = int(b["Start_Timestamp"]) - int(a["Start_Timestamp"])
            if ka == kb and d < 100000:
                gaps[ka].append(d)
        for k, v in gaps.items():
            v = sorted(v)
            s2s[k] = (sum(v) / len(v), v[len(v) // 2], len(v))
    if grouped:
        lines += ["## Kernel durations (--kernel-trace --stats; template instances summed)", "",
                  "avg, later half: the later half of a kernel's dispatches.  start-to-start: the interval between "
                  "the starts of consecutive dispatches of the same kernel (launches back to back, e.g. within a "
                  "graph replay; intervals over 100 us left out), mean and median, and how many.", "",
                  "| kernel | calls | avg (us) | min (us) | max (us) | share of GPU time | avg, later half (us) "
                  "| start-to-start mean / median (us), intervals |",
                  "|---|---|---|---|---|---|---|---|"]
        total = sum(g["total"] for g in grouped.values())
        for base, g in grouped.items():
            lh = f"{late[base] / 1e3:.3f}" if base in late else "-"
            ss = f"{s2s[base][0] / 1e3:.3f} / {s2s[base][1] / 1e3:.3f}, {s2s[base][2]}" if base in s2s else "-"
            lines.append(f"| {base} | {g['calls']} | {g['total'] / g['calls'] / 1e3:.3f} | {g['min'] / 1e3:.3f} | "
                         f"{g['max'] / 1e3:.3f} | {100 * g['total'] / total:.1f}% | {lh} | {ss} |")
        lines.append("")
    counters = collections.OrderedDict()  # counter -> {kernel: (avg value, avg duration ns, dispatches)}
    for d in args.pmc:
        rows = _read_csv(_find(d, "counter_collection.csv"))
        for c in sorted({r["Counter_Name"] for r in rows}):
            counters[c] = _per_kernel(rows, c)
    kernels = sorted({k for per in counters.values() for k in per})
    if counters:
        lines += ["## Counters per dispatch (averages over the profiled dispatches)", "",
                  "| kernel | " + " | ".join(counters) + " | avg dispatch (us) |",
                  "|---|" + "---|" * (len(counters) + 1)]
        for k in kernels:
            vals = [counters[c].get(k) for c in counters]
            dur = next((v[1] for v in vals if v), 0.0)
            lines.append(f"| {k} | " + " | ".join("" if v is None else f"{v[0]:.1f}" for v in vals) +
                         f" | {dur / 1e3:.3f} |")
        lines.append("")
    traffic = {}
    if args.calib and "FETCH_SIZE" in counters and "WRITE_SIZE" in counters:
        cf = _per_kernel(_read_csv(_find(args.calib[0], "counter_collection.csv")), "FETCH_SIZE")
        cw = _per_kernel(_read_csv(_find(args.calib[1], "counter_collection.csv")), "WRITE_SIZE")
        copy_f = next(v[0] for k, v in cf.items() if "copy" in k.lower())
        copy_w = next(v[0] for k, v in cw.items() if "copy" in k.lower())
        f_fetch, f_write = CALIB_BYTES / (copy_f * 1024.0), CALIB_BYTES / (copy_w * 1024.0)
        lines += ["## HBM traffic", "",
                  f"Calibration: a 1 GiB device copy reads {copy_f:.0f} KiB (FETCH_SIZE) and writes {copy_w:.0f} KiB "
                  f"(WRITE_SIZE) per dispatch, so the counters are scaled by {f_fetch:.4f} and {f_write:.4f}.", "",
                  "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (calibrated) |", "|---|---|---|---|"]
        for k in kernels:
            fk, wk = counters["FETCH_SIZE"].get(k), counters["WRITE_SIZE"].get(k)
            if not fk or not wk:
                continue
            hbm = fk[0] * 1024.0 * f_fetch + wk[0] * 1024.0 * f_write
            lines.append(f"| {k} | {fk[0]:.1f} | {wk[0]:.1f} | {hbm:.0f} |")
            if k in KERNEL_SOURCES:
                traffic[k] = {"bytes_per_launch": round(hbm), "fetch_kib": round(fk[0], 1), "write_kib": round(wk[0], 1),
                              "calibration": {"fetch": round(f_fetch, 5), "write": round(f_write, 5)},
                              "source_sha256_16": source_hash(k), "dispatches": fk[2]}
        lines.append("")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
        lines += ["## MFMA utilisation", "",
                  "busy = SQ_VALU_MFMA_BUSY_CYCLES (all SIMDs) / (dispatch duration x 2.4 GHz x 1024 SIMDs); "
                  "ops = SQ_INSTS_MFMA x 32768 for v_mfma_i32_16x16x64_i8 (16 x 16 x 64 multiply-adds), "
                  "x 16384 for v_mfma_f32_16x16x32_bf16 (k_bwd_x, k_bwd_w).", "",
                  "| kernel | MFMA busy | MFMA instructions | ops per dispatch | T(FL)OPS over the dispatch |",
                  "|---|---|---|---|---|"]
        busy = counters["SQ_VALU_MFMA_BUSY_CYCLES"]
        insts = counters.get("SQ_INSTS_MFMA", {})
        for k, (b, dur, _) in busy.items():
            if b <= 0:
                continue
            util = b / (dur * CLOCK_GHZ * CU_SIMDS)
            n_inst = insts.get(k, (0.0, dur, 0))[0]
            ops = n_inst * MFMA_OPS.get(k, MFMA_OPS_DEFAULT)
            lines.append(f"| {k} | {100 * util:.1f}% | {n_inst:.0f} | {ops:.4g} | "
                         f"{ops / (insts.get(k, (0, dur, 0))[1] * 1e-9) / 1e12 if n_inst else 0:.1f} |")
        lines.append("")
    if "SQ_INSTS_VALU" in counters or "SQ_WAIT_INST_ANY" in counters:
        lines += ["## Where the waves' time goes", "",
                  "VALU issue = SQ_INSTS_VALU x 4 cycles (a wave64 instruction on a 16-lane SIMD) / (dispatch "
                  "duration x 2.4 GHz x 1024 SIMDs); MFMA busy as above; waiting = SQ_WAIT_INST_ANY / "
                  "SQ_WAVE_CYCLES (share of resident wave time spent waiting on a dependency or counter); LDS "
                  "conflict cycles per LDS instruction = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS.", "",
                  "| kernel | VALU issue | MFMA busy | waiting | VALU per MFMA | LDS conflict cycles per LDS instr |",
                  "|---|---|---|---|---|---|"]
        def avg(c, k):
            v = counters.get(c, {}).get(k)
            return (v[0], v[1]) if v else (None, None)
        for k in kernels:
            valu, dur = avg("SQ_INSTS_VALU", k)
            mfma, _ = avg("SQ_INSTS_MFMA", k)
            busy, dur_b = avg("SQ_VALU_MFMA_BUSY_CYCLES", k)
            wait, _ = avg("SQ_WAIT_INST_ANY", k)
            wave, _ = avg("SQ_WAVE_CYCLES", k)
            lds, _ = avg("SQ_INSTS_LDS", k)
            conf, _ = avg("SQ_LDS_BANK_CONFLICT", k)
            dur = dur or dur_b
            if not dur:
                continue
            cyc = dur * 1e-9 * CLOCK_GHZ * 1e9
            cells = [f"{100 * valu * 4 / (cyc * CU_SIMDS):.1f}%" if valu is not None else "-",
                     f"{100 * busy / (cyc * CU_SIMDS):.1f}%" if busy is not None else "-",
                     f"{100 * wait / wave:.1f}%" if wait is not None and wave else "-",
                     f"{valu / mfma:.2f}" if valu is not None and mfma else "-",
                     f"{conf / lds:.3f}" if conf is not None and lds else "-"]
            lines.append(f"| {k} | " + " | ".join(cells) + " |")
        lines.append("")
    os.makedirs(args.out_dir, exist_ok=True)
    if traffic and args.workload:
        path = os.path.join(args.out_dir, "traffic.json")
        try:
            with open(path) as f:
                stored = json.load(f)
        except (OSError, ValueError):
            stored = {}
        stored = {k: v for k, v in stored.items() if isinstance(v, dict) and all(isinstance(x, dict) for x in v.values())}
        stored[args.workload] = traffic
        with open(path, "w") as f:
            json.dump(stored, f, indent=1, sort_keys=True)
            f.write("\n")
    with open(os.path.join(args.out_dir, f"{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def source_hash(kernel: str) -> str:
    """Hash of the kernel's source file and the device helpers it includes."""
    import hashlib
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[kernel], "device_util.h"):
        with open(os.path.join(ROOT, "ternary_weight_absmean_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str, algorithmic_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when there is none or the kernel's source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload, {}).get(kernel)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(kernel):
        return None
    return {"bytes_per_launch": rec["bytes_per_launch"],
            "ratio_to_algorithmic": round(rec["bytes_per_launch"] / algorithmic_bytes, 3),
            "workload": workload}


# ---------------------------------------------------------------- short programs for rocprofv3


def _profile_stack_2b_m1(args):
    """The benchmark's step alone: the 30-layer 2B-shaped stack packed, the
    step captured as a HIP graph (120 bl_bitlinear launches at one token),
    5 warm replays, then --reps timed replays back to back."""
    import numpy as np
    import torch
    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    wl = datagen.WORKLOAD_STACK_2B
    vp = ctypes.c_void_p
    lib = bl.library()
    calls, keep = [], []
    for layer in range(datagen.STACK_2B_LAYERS):
        for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
            w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, layer, pi, datagen.TENSOR_W), n, k)).to(dev)
            packed, gamma = bl.bl_ternarize_pack(w)
            del w
            cols = datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS)
            x = datagen.activations_bf16(datagen.stream_id(wl, layer, pi, datagen.TENSOR_X), 1, k, cols,
                                         datagen.STACK_2B_OUTLIER_MULT)
            xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
            xq = torch.empty((1, k), dtype=torch.int8, device=dev)
            alpha = torch.empty(1, dtype=torch.float32, device=dev)
            y = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
            keep.append((packed, gamma, xd, xq, alpha, y))
            calls.append((vp(packed.data_ptr()), vp(gamma.data_ptr()), vp(xd.data_ptr()), n, k, vp(xq.data_ptr()),
                          vp(alpha.data_ptr()), vp(y.data_ptr())))
    torch.cuda.synchronize()
    print(f"[profile] stack_2b_m1: {len(calls)} linears packed", flush=True)

    def step():
        s = vp(torch.cuda.current_stream().cuda_stream)
        for packed, gamma, x, n, k, xq, alpha, y in calls:
            rc = lib.bl_bitlinear(packed, gamma, x, 1, n, k, xq, alpha, None, y, s)
            if rc:
                raise RuntimeError(bl.bl_status_string(rc))

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        step()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.reps
    print(f"[profile] stack_2b_m1: {args.reps} replays, {ms:.4f} ms per step, "
          f"{1000 * ms / len(calls):.3f} us per launch (HIP events)", flush=True)
    return 0


def _profile_prefill_2b(args):
    """Layer-0 gate+up and down of the 2B-shaped stack at M = 2048: bl_bitlinear
    (quantizer + GEMM) --reps times each."""
    import numpy as np
    import torch
    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    wl = datagen.WORKLOAD_STACK_2B
    m = 2048
    for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
        if name not in ("gate_up", "down"):
            continue
        w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, 0, pi, datagen.TENSOR_W), n, k)).to(dev)
        packed, gamma = bl.bl_ternarize_pack(w)
        del w
        cols = datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS)
        x = datagen.activations_bf16(datagen.stream_id(wl, 0, pi, datagen.TENSOR_X) + m, m, k, cols,
                                     datagen.STACK_2B_OUTLIER_MULT)
        xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        for _ in range(args.reps):
            bl.bl_bitlinear(packed, gamma, xd, n, acc=False)
        torch.cuda.synchronize()
        print(f"[profile] prefill_2b {name} M={m} K={k} N={n} x{args.reps}", flush=True)
    return 0


def _profile_batched_2b(args, m):
    """The first 16 layers of the 2B-shaped stack (64 linears, 278 MB packed:
    more than the 256 MB Infinity Cache, so each pass streams from HBM) at M
    tokens: bl_bitlinear on every linear in order, --reps passes."""
    import numpy as np
    import torch
    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    wl = datagen.WORKLOAD_STACK_2B
    linears = []
    for layer in range(16):
        for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
            w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, layer, pi, datagen.TENSOR_W), n, k)).to(dev)
            packed, gamma = bl.bl_ternarize_pack(w)
            del w
            cols = datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS)
            x = datagen.activations_bf16(datagen.stream_id(wl, layer, pi, datagen.TENSOR_X) + m, m, k, cols,
                                         datagen.STACK_2B_OUTLIER_MULT)
            linears.append((packed, gamma, torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16), n))
    torch.cuda.synchronize()
    print(f"[profile] batched_2b M={m}: {len(linears)} linears packed", flush=True)
    for r in range(args.reps):
        for packed, gamma, xd, n in linears:
            bl.bl_bitlinear(packed, gamma, xd, n, acc=False)
        torch.cuda.synchronize()
        print(f"[profile] batched_2b M={m} pass {r + 1}/{args.reps}", flush=True)
    return 0


def _profile_70b(args, ms):
    import numpy as np
    import torch
    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    wl = datagen.WORKLOAD_70B
    layer = []
    for pi, (name, k, n) in enumerate(datagen.LAYER_70B_PROJ):
        w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, 0, pi, datagen.TENSOR_W), n, k)).to(dev)
        packed, gamma = bl.bl_ternarize_pack(w)
        del w
        # two copies (2 x 176 MB > the 256 MB Infinity Cache): consecutive launches stream from HBM
        layer.append((name, k, n, [packed, packed.clone()], gamma))
    torch.cuda.synchronize()
    for m in ms:
        for pi, (name, k, n, copies, gamma) in enumerate(layer):
            cols = datagen.outlier_columns(wl, k, datagen.n_outliers_70b(k))
            x = datagen.activations_bf16(datagen.stream_id(wl, 0, pi, datagen.TENSOR_X) + m, m, k, cols,
                                         datagen.LAYER_70B_OUTLIER_MULT)
            xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
            for r in range(args.reps):
                bl.bl_bitlinear(copies[r % 2], gamma, xd, n, acc=False)
            torch.cuda.synchronize()
            print(f"[profile] 70b {name} M={m} K={k} N={n} x{args.reps}", flush=True)
    return 0


def _profile_training_2b(args):
    """Layer-0 gate+up and down of the 2B-shaped stack at M = 2048, training
    side: re-ternarization with the transposed packing, the input gradient and
    the weight gradient, --reps times each."""
    import numpy as np
    import torch
    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    wl = datagen.WORKLOAD_STACK_2B
    m = 2048
    for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
        if name not in ("gate_up", "down"):
            continue
        w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, 0, pi, datagen.TENSOR_W), n, k)).to(dev)
        g = torch.Generator(device="cpu").manual_seed(n * 31 + k)
        dy = (torch.randn((m, n), generator=g) * 0.01).to(torch.bfloat16).to(dev)
        cols = datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS)
        x = datagen.activations_bf16(datagen.stream_id(wl, 0, pi, datagen.TENSOR_X) + 8192, m, k, cols,
                                     datagen.STACK_2B_OUTLIER_MULT)
        xq, alpha = bl.bl_quant_act(torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16))
        ws = torch.empty(bl.bl_backward_w_workspace_bytes(m, n, k), dtype=torch.uint8, device=dev)
        for _ in range(args.reps):
            packed, gamma = bl.bl_ternarize_pack(w)
            packed_t = bl.bl_pack_transposed(packed, n, k)
            bl.bl_bitlinear_backward_x(packed_t, gamma, dy, k)
            bl.bl_bitlinear_backward_w(dy, xq, alpha, workspace=ws)
        torch.cuda.synchronize()
        print(f"[profile] training_2b {name} M={m} K={k} N={n} x{args.reps}", flush=True)
    return 0


def _profile_b3(args):
    """Five-trits-per-byte weights at one token: the 70B-shaped layer's gate+up
    and down (two copies each, 2 x 143 MB for gate+up), then the first 16
    layers of the 2B-shaped stack; bl_bitlinear_b3, --reps passes each."""
    import numpy as np
    import torch
    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    wl = datagen.WORKLOAD_70B
    for pi, (name, k, n) in enumerate(datagen.LAYER_70B_PROJ):
        w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, 0, pi, datagen.TENSOR_W), n, k)).to(dev)
        p3, g3 = bl.bl_ternarize_pack_b3(w)
        del w
        copies = [p3, p3.clone()]
        cols = datagen.outlier_columns(wl, k, datagen.n_outliers_70b(k))
        x = datagen.activations_bf16(datagen.stream_id(wl, 0, pi, datagen.TENSOR_X) + 1, 1, k, cols,
                                     datagen.LAYER_70B_OUTLIER_MULT)
        xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        for r in range(args.reps):
            bl.bl_bitlinear_b3(copies[r % 2], g3, xd, n, acc=False)
        torch.cuda.synchronize()
        print(f"[profile] b3 70b {name} K={k} N={n} x{args.reps}", flush=True)
        del copies, p3
    wl = datagen.WORKLOAD_STACK_2B
    linears = []
    for layer in range(16):
        for pi, (name, k, n) in enumerate(datagen.STACK_2B_PROJ):
            w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, layer, pi, datagen.TENSOR_W), n, k)).to(dev)
            p3, g3 = bl.bl_ternarize_pack_b3(w)
            del w
            cols = datagen.outlier_columns(wl, k, datagen.STACK_2B_OUTLIERS)
            x = datagen.activations_bf16(datagen.stream_id(wl, layer, pi, datagen.TENSOR_X), 1, k, cols,
                                         datagen.STACK_2B_OUTLIER_MULT)
            linears.append((p3, g3, torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16), n))
    torch.cuda.synchronize()
    for r in range(args.reps):
        for p3, g3, xd, n in linears:
            bl.bl_bitlinear_b3(p3, g3, xd, n, acc=False)
        torch.cuda.synchronize()
        print(f"[profile] b3 2B stack pass {r + 1}/{args.reps}", flush=True)
    return 0


PROFILE_CASES = {
    "decode_b3": _profile_b3,
    "stack_2b_m1": _profile_stack_2b_m1,
    "prefill_2b": _profile_prefill_2b,
    "training_2b": _profile_training_2b,
    "decode_70b": lambda args: _profile_70b(args, (1, 16)),
    "prefill_70b": lambda args: _profile_70b(args, (1024,)),
    "batched_2b_m4": lambda args: _profile_batched_2b(args, 4),
    "batched_2b_m16": lambda args: _profile_batched_2b(args, 16),
    "batched_2b_m64": lambda args: _profile_batched_2b(args, 64),
}


def _repeat(fn, inner):
    """fn called `inner` times: one graph replay then holds that many calls, so
    that the per-replay launch gap is spread over them (time / inner)."""
    def run():
        for _ in range(inner):
            fn()
    return run


def _graph_time_ms(torch, fn, reps, warm=2):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        fn()
    for _ in range(warm):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_extras(args, linears, lib):
    """Other workloads of the metric, each timed as HIP-graph replays:
    prefill (M = 2048) on the 2B stack's layer-0 gate+up and down, batched
    decode (M = 4, 16, 64) through the whole 2B stack, and the 70B-shaped
    layer (80 distinct copies of one layer's packed weights, looped) at M = 1,
    16 and 1024.  Inputs are seeded synthetic activations of each shape."""
    import numpy as np
    import torch

    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    vp = ctypes.c_void_p
    out = {}

    def act(stream, m, k, wl, n_out, mult):
        cols = datagen.outlier_columns(wl, k, n_out)
        x = datagen.activations_bf16(stream, m, k, cols, mult)
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    def layer_fn(items, m):
        """items: list of (packed, gamma, x, n, k, xq, alpha, y) tensors."""
        def fn():
            s = vp(torch.cuda.current_stream().cuda_stream)
            for packed, gamma, x, n, k, xq, alpha, y in items:
                rc = lib.bl_bitlinear(vp(packed.data_ptr()), vp(gamma.data_ptr()), vp(x.data_ptr()), m, n, k,
                                      vp(xq.data_ptr()), vp(alpha.data_ptr()), None, vp(y.data_ptr()), s)
                if rc:
                    raise RuntimeError(bl.bl_status_string(rc))
        return fn

    def bufs(m, n, k):
        return (torch.empty((m, k), dtype=torch.int8, device=dev), torch.empty(m, dtype=torch.float32, device=dev),
                torch.empty((m, n), dtype=torch.bfloat16, device=dev))

    # ---- prefill, 2B layer 0 gate+up and down, M = 2048 (per-token quantize + GEMM)
    wl = datagen.WORKLOAD_STACK_2B
    prefill = {}
    for name in ("gate_up", "down"):
        lin = next(l for l in linears if l["name"] == name)
        m, n, k = 2048, lin["n"], lin["k"]
        x = act(datagen.stream_id(wl, 0, 2 if name == "gate_up" else 3, datagen.TENSOR_X) + 2048, m, k, wl,
                datagen.STACK_2B_OUTLIERS, datagen.STACK_2B_OUTLIER_MULT)
        xq, alpha, y = bufs(m, n, k)
        # ten calls per graph replay (a replay of a single ~60 us kernel would
        # also time the gap between graph launches)
        inner = 10
        ms = _graph_time_ms(torch, _repeat(layer_fn([(lin["packed"], lin["gamma"], x, n, k, xq, alpha, y)], m),
                                           inner), 10) / inner
        # the product alone (quantized activations already in place)
        def gemm_only():
            s = vp(torch.cuda.current_stream().cuda_stream)
            rc = lib.bl_linear(vp(lin["packed"].data_ptr()), vp(lin["gamma"].data_ptr()), vp(xq.data_ptr()),
                               vp(alpha.data_ptr()), m, n, k, None, vp(y.data_ptr()), s)
            if rc:
                raise RuntimeError(bl.bl_status_string(rc))
        ms_gemm = _graph_time_ms(torch, _repeat(gemm_only, inner), 10) / inner
        ops = 2.0 * m * n * k
        prefill[f"{name} M={m} K={k} N={n}"] = {
            "layer_ms": round(ms, 4), "layer_TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
            "gemm_ms": round(ms_gemm, 4), "gemm_TOPS": round(ops / (ms_gemm * 1e-3) / 1e12, 1),
            "gemm_frac_of_int8_mfma_peak": round(ops / (ms_gemm * 1e-3) / 1e12 / MFMA_I8_PEAK_TOPS, 4)}
    out["prefill_2b"] = prefill

    # ---- gated feed-forward of the 2B layer 0: gate+up with squared-ReLU
    # gating fused (packed with alternating gate/up tiles), then down
    gu = next(l for l in linears if l["name"] == "gate_up")
    dn = next(l for l in linears if l["name"] == "down")
    f = gu["n"] // 2
    w_gu = torch.from_numpy(datagen.weights(datagen.stream_id(wl, 0, 2, datagen.TENSOR_W), gu["n"], gu["k"])).to(dev)
    packed_glu, gamma_glu = bl.bl_ternarize_pack_glu(w_gu)
    del w_gu
    ffn = {}
    for m in (1, 2048):
        x = act(datagen.stream_id(wl, 0, 2, datagen.TENSOR_X) + 4096 + m, m, gu["k"], wl,
                datagen.STACK_2B_OUTLIERS, datagen.STACK_2B_OUTLIER_MULT)
        xq = torch.empty((m, gu["k"]), dtype=torch.int8, device=dev)
        alpha = torch.empty(m, dtype=torch.float32, device=dev)
        h = torch.empty((m, f), dtype=torch.bfloat16, device=dev)
        xq2, alpha2, y2 = bufs(m, dn["n"], dn["k"])

        def glu_only():
            s = vp(torch.cuda.current_stream().cuda_stream)
            rc = lib.bl_bitlinear_glu(vp(packed_glu.data_ptr()), vp(gamma_glu.data_ptr()), vp(x.data_ptr()), m, f,
                                      gu["k"], vp(xq.data_ptr()), vp(alpha.data_ptr()), vp(h.data_ptr()), s)
            if rc:
                raise RuntimeError(bl.bl_status_string(rc))

        def chain():
            glu_only()
            s = vp(torch.cuda.current_stream().cuda_stream)
            rc = lib.bl_bitlinear(vp(dn["packed"].data_ptr()), vp(dn["gamma"].data_ptr()), vp(h.data_ptr()), m,
                                  dn["n"], dn["k"], vp(xq2.data_ptr()), vp(alpha2.data_ptr()), None,
                                  vp(y2.data_ptr()), s)
            if rc:
                raise RuntimeError(bl.bl_status_string(rc))

        # several calls per graph replay, so that the gap between graph
        # launches is spread over them
        inner = 50 if m == 1 else 10
        ms_glu = _graph_time_ms(torch, _repeat(glu_only, inner), 10) / inner
        ms_chain = _graph_time_ms(torch, _repeat(chain, inner), 10) / inner
        ops = 2.0 * m * gu["n"] * gu["k"]
        e = {"gate_up_glu_us": round(ms_glu * 1e3, 2), "ffn_gate_up_glu_down_us": round(ms_chain * 1e3, 2)}
        if m == 1:
            e["gate_up_glu_weight_GBps"] = round(packed_glu.numel() / (ms_glu * 1e-3) / 1e9, 1)
            # one 8.8 MB matrix re-read by every call: served by the caches, not an HBM figure
            e["cache_resident"] = True
        else:
            e["gate_up_glu_TOPS"] = round(ops / (ms_glu * 1e-3) / 1e12, 1)
            e["gate_up_glu_frac_of_int8_mfma_peak"] = round(ops / (ms_glu * 1e-3) / 1e12 / MFMA_I8_PEAK_TOPS, 4)
        ffn[f"M={m}"] = e
        del x, xq, alpha, h, xq2, alpha2, y2
    out["ffn_glu_2b_layer0"] = ffn
    del packed_glu, gamma_glu

    # ---- chained feed-forward through the 30 layers: h = bl_bitlinear_glu(x)
    # with layer l's gate+up (squared-ReLU gated), then x' = bl_bitlinear(h)
    # with its down projection feeding layer l + 1 (60 dependent launches per
    # token; 398 MB of weights, more than the Infinity Cache)
    out["ffn_chain_2b"] = measure_ffn_chain(args, linears, lib)

    # ---- config-1 decode (2560 x 2560, one token) over 320 distinct copies
    # of the packed matrix (524 MB), so that each launch streams from HBM
    out["single_2560_rotated"] = measure_single_rotated(args, lib)

    # ---- training side, 2B layer 0 gate+up and down at M = 2048: the
    # straight-through gradients and the per-step re-ternarization
    train = {}
    for name in ("gate_up", "down"):
        lin = next(l for l in linears if l["name"] == name)
        m, n, k = 2048, lin["n"], lin["k"]
        w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, 0, 2 if name == "gate_up" else 3,
                                                               datagen.TENSOR_W), n, k)).to(dev)
        packed = torch.empty(bl.bl_packed_bytes(n, k), dtype=torch.uint8, device=dev)
        gamma = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(bl.bl_ternarize_pack_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
        packed_t = torch.empty(bl.bl_packed_bytes(k, n), dtype=torch.uint8, device=dev)
        g = torch.Generator(device="cpu").manual_seed(n * 31 + k)
        dy = (torch.randn((m, n), generator=g) * 0.01).to(torch.bfloat16).to(dev)
        x = act(datagen.stream_id(wl, 0, 2 if name == "gate_up" else 3, datagen.TENSOR_X) + 8192, m, k, wl,
                datagen.STACK_2B_OUTLIERS, datagen.STACK_2B_OUTLIER_MULT)
        xq, alpha = bl.bl_quant_act(x)
        dx = torch.empty((m, k), dtype=torch.float32, device=dev)
        dw = torch.empty((n, k), dtype=torch.float32, device=dev)
        wws = torch.empty(bl.bl_backward_w_workspace_bytes(m, n, k), dtype=torch.uint8, device=dev)

        def repack():
            s = vp(torch.cuda.current_stream().cuda_stream)
            rc = lib.bl_ternarize_pack(vp(w.data_ptr()), n, k, vp(packed.data_ptr()), vp(gamma.data_ptr()),
                                       vp(ws.data_ptr()), ws.numel(), s)
            rc = rc or lib.bl_pack_transposed(vp(packed.data_ptr()), n, k, vp(packed_t.data_ptr()), s)
            if rc:
                raise RuntimeError(bl.bl_status_string(rc))

        def grad_x():
            s = vp(torch.cuda.current_stream().cuda_stream)
            rc = lib.bl_bitlinear_backward_x(vp(packed_t.data_ptr()), vp(gamma.data_ptr()), vp(dy.data_ptr()), m, n,
                                             k, vp(dx.data_ptr()), s)
            if rc:
                raise RuntimeError(bl.bl_status_string(rc))

        def grad_w():
            s = vp(torch.cuda.current_stream().cuda_stream)
            rc = lib.bl_bitlinear_backward_w(vp(dy.data_ptr()), vp(xq.data_ptr()), vp(alpha.data_ptr()), m, n, k,
                                             vp(dw.data_ptr()), vp(wws.data_ptr()), wws.numel(), s)
            if rc:
                raise RuntimeError(bl.bl_status_string(rc))

        repack()
        inner = 5
        ms_pack = _graph_time_ms(torch, _repeat(repack, inner), 5) / inner
        ms_x = _graph_time_ms(torch, _repeat(grad_x, inner), 5) / inner
        ms_w = _graph_time_ms(torch, _repeat(grad_w, inner), 5) / inner
        flops = 2.0 * m * n * k
        train[f"{name} M={m} K={k} N={n}"] = {
            "repack_ms": round(ms_pack, 4), "repack_fp32_GBps": round(4.0 * n * k / (ms_pack * 1e-3) / 1e9, 1),
            "grad_x_ms": round(ms_x, 4), "grad_x_TFLOPS": round(flops / (ms_x * 1e-3) / 1e12, 1),
            "grad_x_frac_of_bf16_mfma_peak": round(flops / (ms_x * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "grad_w_ms": round(ms_w, 4), "grad_w_TFLOPS": round(flops / (ms_w * 1e-3) / 1e12, 1),
            "grad_w_frac_of_bf16_mfma_peak": round(flops / (ms_w * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        del w, packed, packed_t, ws, dy, x, xq, alpha, dx, dw, wws
    out["training_2b_layer0"] = train

    # ---- batched decode through the whole 2B stack, M = 4, 16, 64
    batched = {}
    weight_bytes = sum(l["packed"].numel() for l in linears)
    for m in (4, 16, 64):
        items = []
        for i, lin in enumerate(linears):
            x = act(datagen.stream_id(wl, i // 4, i % 4, datagen.TENSOR_X) + 7 * m, m, lin["k"], wl, 0, 1.0)
            items.append((lin["packed"], lin["gamma"], x, lin["n"], lin["k"], *bufs(m, lin["n"], lin["k"])))
        ms = _graph_time_ms(torch, layer_fn(items, m), max(5, args.steps // 10))
        ops = 2.0 * m * sum(lin["n"] * lin["k"] for lin in linears)
        batched[f"M={m}"] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(m * 1000.0 / ms, 1),
                             "weight_GBps": round(weight_bytes / (ms * 1e-3) / 1e9, 1),
                             "frac_of_hbm_peak": round(weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                             "TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
                             "frac_of_int8_mfma_peak": round(ops / (ms * 1e-3) / 1e12 / MFMA_I8_PEAK_TOPS, 4)}
        del items
    out["batched_decode_2b_stack"] = batched

    # ---- 70B-shaped layer: 80 distinct copies of one layer's packed weights
    wl70 = datagen.WORKLOAD_70B
    layer = []
    for pi, (name, k, n) in enumerate(datagen.LAYER_70B_PROJ):
        w = torch.from_numpy(datagen.weights(datagen.stream_id(wl70, 0, pi, datagen.TENSOR_W), n, k)).to(dev)
        packed, gamma = bl.bl_ternarize_pack(w)
        del w
        layer.append((name, k, n, packed, gamma))
    torch.cuda.synchronize()
    n_layers = datagen.LAYER_70B_LAYERS
    copies = [[(name, k, n, packed.clone(), gamma) for name, k, n, packed, gamma in layer] for _ in range(n_layers)]
    torch.cuda.synchronize()
    layer_bytes = sum(packed.numel() for _, _, _, packed, _ in layer)
    r70 = {"packed_bytes_per_layer": layer_bytes, "layers": n_layers}
    for m in (1, 16, 1024):
        xs = {k: act(datagen.stream_id(wl70, 0, pi, datagen.TENSOR_X) + m, m, k, wl70, datagen.n_outliers_70b(k),
                     datagen.LAYER_70B_OUTLIER_MULT) for pi, (_, k, _) in enumerate(datagen.LAYER_70B_PROJ)}
        scratch = {(n, k): bufs(m, n, k) for _, k, n, _, _ in layer}
        items = [(packed, gamma, xs[k], n, k, *scratch[(n, k)]) for c in copies for (_, k, n, packed, gamma) in c]
        ms = _graph_time_ms(torch, layer_fn(items, m), 3 if m == 1024 else 10)
        entry = {"ms_per_80_layers": round(ms, 3), "tokens_per_s": round(m * 1000.0 / ms, 1),
                 "weight_GBps": round(layer_bytes * n_layers / (ms * 1e-3) / 1e9, 1)}
        if m == 1024:
            ops = 2.0 * m * sum(n * k for _, k, n, _, _ in layer) * n_layers
            entry["TOPS"] = round(ops / (ms * 1e-3) / 1e12, 1)
            entry["frac_of_int8_mfma_peak"] = round(ops / (ms * 1e-3) / 1e12 / MFMA_I8_PEAK_TOPS, 4)
        else:
            entry["frac_of_hbm_peak"] = round(layer_bytes * n_layers / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
            # each projection alone over the 80 copies (same launches, same copies)
            per = {}
            for name_p, k_p, n_p, packed_p, _ in layer:
                sel = [it for c in copies for it, (nm, _, _, _, _) in
                       zip([(packed, gamma, xs[k], n, k, *scratch[(n, k)]) for (_, k, n, packed, gamma) in c], c)
                       if nm == name_p]
                ms_p = _graph_time_ms(torch, layer_fn(sel, m), 10)
                gbps = packed_p.numel() * n_layers / (ms_p * 1e-3) / 1e9
                per[name_p] = {"us_per_layer": round(1000.0 * ms_p / n_layers, 2), "weight_GBps": round(gbps, 1),
                               "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            entry["per_projection"] = per
        r70[f"M={m}"] = entry
        del items, scratch
    out["layer_70b"] = r70
    del copies, layer
    torch.cuda.empty_cache()

    # ---- the same decode with five-trits-per-byte weights
    out["b3"] = measure_b3(args, linears, lib)
    return out


def measure_ffn_chain(args, linears, lib):
    import numpy as np
    import torch

    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    vp = ctypes.c_void_p
    wl = datagen.WORKLOAD_STACK_2B
    gus = [l for l in linears if l["name"] == "gate_up"]
    dns = [l for l in linears if l["name"] == "down"]
    f = gus[0]["n"] // 2
    k_in = gus[0]["k"]
    glu = []
    for layer, gu in enumerate(gus):
        w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, layer, 2, datagen.TENSOR_W), gu["n"], gu["k"])).to(dev)
        glu.append(bl.bl_ternarize_pack_glu(w))
        del w
    torch.cuda.synchronize()
    weight_bytes = sum(p.numel() for p, _ in glu) + sum(d["packed"].numel() for d in dns)
    res = {"layers": len(gus), "weights_MB": round(weight_bytes / 1e6, 1),
           "launch": "per layer: bl_bitlinear_glu (gate+up, squared ReLU) then bl_bitlinear (down), chained"}
    for m in (1, 16):
        cols = datagen.outlier_columns(wl, k_in, datagen.STACK_2B_OUTLIERS)
        x0 = datagen.activations_bf16(datagen.stream_id(wl, 0, 2, datagen.TENSOR_X) + 9000 + m, m, k_in, cols,
                                      datagen.STACK_2B_OUTLIER_MULT)
        xs = [torch.from_numpy(x0.view(np.int16)).to(dev).view(torch.bfloat16)]
        xs += [torch.empty((m, k_in), dtype=torch.bfloat16, device=dev) for _ in gus]
        h = torch.empty((m, f), dtype=torch.bfloat16, device=dev)
        xq1 = torch.empty((m, k_in), dtype=torch.int8, device=dev)
        xq2 = torch.empty((m, f), dtype=torch.int8, device=dev)
        a1 = torch.empty(m, dtype=torch.float32, device=dev)
        a2 = torch.empty(m, dtype=torch.float32, device=dev)

        def chain():
            s = vp(torch.cuda.current_stream().cuda_stream)
            for layer, ((pk, gm), dn) in enumerate(zip(glu, dns)):
                rc = lib.bl_bitlinear_glu(vp(pk.data_ptr()), vp(gm.data_ptr()), vp(xs[layer].data_ptr()), m, f, k_in,
                                          vp(xq1.data_ptr()), vp(a1.data_ptr()), vp(h.data_ptr()), s)
                rc = rc or lib.bl_bitlinear(vp(dn["packed"].data_ptr()), vp(dn["gamma"].data_ptr()), vp(h.data_ptr()),
                                            m, dn["n"], dn["k"], vp(xq2.data_ptr()), vp(a2.data_ptr()), None,
                                            vp(xs[layer + 1].data_ptr()), s)
                if rc:
                    raise RuntimeError(bl.bl_status_string(rc))

        ms = _graph_time_ms(torch, chain, max(5, args.steps // 10))
        res[f"M={m}"] = {"ms_per_token_pass": round(ms, 4), "tokens_per_s": round(m * 1000.0 / ms, 1),
                         "weight_GBps": round(weight_bytes / (ms * 1e-3) / 1e9, 1),
                         "frac_of_hbm_peak": round(weight_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "us_per_launch": round(1000.0 * ms / (2 * len(gus)), 3)}
        del xs, h, xq1, xq2, a1, a2
    del glu
    torch.cuda.empty_cache()
    return res


def measure_single_rotated(args, lib, copies=320):
    """The single 2560 x 2560 BitLinear at one token (config 1): one
    bl_bitlinear per launch, each on its own copy of the packed matrix
    (320 x 1.64 MB = 524 MB, twice the Infinity Cache), replayed as a graph."""
    import numpy as np
    import torch

    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    vp = ctypes.c_void_p
    n = k = 2560
    w = torch.from_numpy(datagen.weights(datagen.stream_id(datagen.WORKLOAD_SINGLE, 0, 0, datagen.TENSOR_W), n, k)).to(dev)
    packed, gamma = bl.bl_ternarize_pack(w)
    del w
    bank = packed.repeat(copies)  # copies back to back
    nb = packed.numel()
    x = datagen.activations_bf16(datagen.stream_id(datagen.WORKLOAD_SINGLE, 0, 0, datagen.TENSOR_X), 1, k)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    xq = torch.empty((1, k), dtype=torch.int8, device=dev)
    alpha = torch.empty(1, dtype=torch.float32, device=dev)
    y = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def run():
        s = vp(torch.cuda.current_stream().cuda_stream)
        base = bank.data_ptr()
        for c in range(copies):
            rc = lib.bl_bitlinear(vp(base + c * nb), vp(gamma.data_ptr()), vp(xd.data_ptr()), 1, n, k,
                                  vp(xq.data_ptr()), vp(alpha.data_ptr()), None, vp(y.data_ptr()), s)
            if rc:
                raise RuntimeError(bl.bl_status_string(rc))

    ms = _graph_time_ms(torch, run, max(5, args.steps // 10))
    us = 1000.0 * ms / copies
    total = nb + 2 * k + k + 4 + 4 + 2 * n
    res = {"copies": copies, "weights_MB": round(nb * copies / 1e6, 1), "us_per_launch": round(us, 3),
           "weight_GBps": round(nb / (us * 1e-6) / 1e9, 1),
           "frac_of_hbm_peak": round(total / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "algorithmic_bytes_per_launch": total}
    del bank, packed
    torch.cuda.empty_cache()
    return res


def measure_b3(args, linears, lib):
    """Five-trits-per-byte weights (bl_ternarize_pack_b3 / bl_bitlinear_b3)
    against the 2-bit code on the same matrices: the 2B-shaped stack at one
    token (120 launches in a graph) and the 70B-shaped layer at one token
    (80 distinct copies, looped)."""
    import numpy as np
    import torch

    import datagen
    import ternary_weight_absmean_amd as bl

    dev = torch.device("cuda", 0)
    vp = ctypes.c_void_p
    wl = datagen.WORKLOAD_STACK_2B
    out = {}

    def run_fn(items):
        def fn():
            s = vp(torch.cuda.current_stream().cuda_stream)
            for packed, gamma, x, n, k, xq, alpha, y in items:
                rc = lib.bl_bitlinear_b3(vp(packed.data_ptr()), vp(gamma.data_ptr()), vp(x.data_ptr()), 1, n, k,
                                         vp(xq.data_ptr()), vp(alpha.data_ptr()), None, vp(y.data_ptr()), s)
                if rc:
                    raise RuntimeError(bl.bl_status_string(rc))
        return fn

    items = []
    for i, lin in enumerate(linears):
        layer, pi = i // 4, i % 4
        w = torch.from_numpy(datagen.weights(datagen.stream_id(wl, layer, pi, datagen.TENSOR_W), lin["n"], lin["k"])).to(dev)
        p3, g3 = bl.bl_ternarize_pack_b3(w)
        del w
        items.append((p3, g3, lin["x"], lin["n"], lin["k"], lin["xq"], lin["alpha"], lin["y"]))
    torch.cuda.synchronize()
    b3_bytes = sum(it[0].numel() for it in items)
    two_bit = sum(lin["packed"].numel() for lin in linears)
    ms = _graph_time_ms(torch, run_fn(items), max(10, args.steps // 4))
    out["decode_stack_2b_m1"] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(1000.0 / ms, 1),
                                 "weights_MB": round(b3_bytes / 1e6, 1), "weights_MB_2bit": round(two_bit / 1e6, 1),
                                 "weight_GBps": round(b3_bytes / (ms * 1e-3) / 1e9, 1),
                                 "us_per_launch": round(1000.0 * ms / len(items), 3)}
    del items
    torch.cuda.empty_cache()

    wl70 = datagen.WORKLOAD_70B
    layer = []
    for pi, (name, k, n) in enumerate(datagen.LAYER_70B_PROJ):
        w = torch.from_numpy(datagen.weights(datagen.stream_id(wl70, 0, pi, datagen.TENSOR_W), n, k)).to(dev)
        p3, g3 = bl.bl_ternarize_pack_b3(w)
        del w
        cols = datagen.outlier_columns(wl70, k, datagen.n_outliers_70b(k))
        x = datagen.activations_bf16(datagen.stream_id(wl70, 0, pi, datagen.TENSOR_X) + 1, 1, k, cols,
                                     datagen.LAYER_70B_OUTLIER_MULT)
        xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        layer.append((name, n, k, p3, g3, xd, torch.empty((1, k), dtype=torch.int8, device=dev),
                      torch.empty(1, dtype=torch.float32, device=dev), torch.empty((1, n), dtype=torch.bfloat16, device=dev)))
    n_layers = datagen.LAYER_70B_LAYERS
    copies = [[p3.clone() for (_, _, _, p3, _, _, _, _, _) in layer] for _ in range(n_layers)]
    torch.cuda.synchronize()
    lb = sum(l[3].numel() for l in layer)
    r70 = {"packed_bytes_per_layer": lb, "packed_bytes_per_layer_2bit": sum(
        bl.bl_packed_bytes(n, k) for _, k, n in datagen.LAYER_70B_PROJ), "layers": n_layers}
    allitems = [(c[i], l[4], l[5], l[1], l[2], l[6], l[7], l[8]) for c in copies for i, l in enumerate(layer)]
    ms = _graph_time_ms(torch, run_fn(allitems), 10)
    r70["M=1"] = {"ms_per_80_layers": round(ms, 3), "tokens_per_s": round(1000.0 / ms, 1),
                  "weight_GBps": round(lb * n_layers / (ms * 1e-3) / 1e9, 1),
                  "frac_of_hbm_peak": round(lb * n_layers / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                  "trits_per_ns": round(sum(n * k for _, k, n in datagen.LAYER_70B_PROJ) * n_layers / (ms * 1e6), 1)}
    per = {}
    for i, l in enumerate(layer):
        sel = [it for j, it in enumerate(allitems) if j % len(layer) == i]
        ms_p = _graph_time_ms(torch, run_fn(sel), 10)
        per[l[0]] = {"us_per_layer": round(1000.0 * ms_p / n_layers, 2),
                     "weight_GBps": round(l[3].numel() * n_layers / (ms_p * 1e-3) / 1e9, 1)}
    r70["M=1"]["per_projection"] = per
    out["layer_70b"] = r70
    del copies, layer, allitems
    torch.cuda.empty_cache()
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, outliers):
    """The CPU oracle (plain C, OpenMP over output rows) on a bounded sample:
    the first layer's four linears of the same stack, one token each,
    repeated for about --cpu-seconds at all threads and half that at one
    thread; scaled to tokens/s of the full stack.  The oracle packs its own
    weights (untimed, offline)."""
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

    def layers_per_s(seconds):
        done = 0
        t0 = time.perf_counter()
        while True:
            for packed, gamma, x, n in prepared:
                oracle.bitlinear_forward(packed, gamma, x, n)
            done += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= seconds:
                return done, elapsed

    all_threads = oracle.set_threads(int(os.environ.get("OMP_NUM_THREADS", "0") or 0))
    done, elapsed = layers_per_s(args.cpu_seconds)
    oracle.set_threads(1)
    done1, elapsed1 = layers_per_s(args.cpu_seconds / 2)
    oracle.set_threads(all_threads)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"value": round(done / elapsed / args.layers, 4), "unit": "tokens/s", "cores": all_threads,
            "kind": "oracle",
            "sample": f"layer 0 of the 2B-shaped stack (4 linears, M=1) run {done}x in {elapsed:.1f} s at "
                      f"{all_threads} threads; tokens/s = layers/s / {args.layers}",
            "value_1_thread": round(done1 / elapsed1 / args.layers, 4),
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": affinity}


def graph_node_floor_us(torch, nodes):
    """Time per node of a captured graph of `nodes` one-element kernels (torch's
    in-place add on a single int32), replayed back to back: the launch cost that
    each kernel node of the decode step pays before it moves any data."""
    t = torch.zeros(1, dtype=torch.int32, device="cuda")
    ms = _graph_time_ms(torch, _repeat(lambda: t.add_(1), nodes), 20)
    return round(1000.0 * ms / nodes, 3)


def stream_reference(torch):
    """Measured HBM ceilings on this machine for context: a 1 GiB device copy
    (read + write, torch) and a 1 GiB read by blmeasure_stream_read (the
    library's reference kernel: non-temporal 16-byte loads, a wave's load
    1 KiB contiguous, eight in flight per lane, as the decode kernels read
    weights), each timed over 5 runs after one warm run."""
    from ternary_weight_absmean_amd._build import MEASURE_LIB_PATH

    mlib = ctypes.CDLL(MEASURE_LIB_PATH)
    mlib.blmeasure_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    mlib.blmeasure_stream_read_sink_words.argtypes = [ctypes.c_size_t]
    mlib.blmeasure_stream_read_sink_words.restype = ctypes.c_size_t
    dev = torch.device("cuda", 0)
    nbytes = 1 << 30
    src = torch.ones(nbytes // 8, dtype=torch.int64, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(mlib.blmeasure_stream_read_sink_words(nbytes), dtype=torch.int32, device=dev)

    def read():
        rc = mlib.blmeasure_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc:
            raise RuntimeError(f"blmeasure_stream_read failed ({rc})")

    out = {}
    for name, fn, moved in (("copy_GBps", lambda: dst.copy_(src), 2 * nbytes), ("read_GBps", read, nbytes)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(moved * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    out["read_kernel"] = "blmeasure_stream_read (non-temporal 16-byte loads, 1 GiB)"
    # the same read at the sizes of the 70B-shaped layer's packed matrices
    # (down 58.7 MB, gate+up 117.4 MB): consecutive windows of the 1 GiB
    # buffer, one launch each, in a graph (every pass touches the whole GiB,
    # past the Infinity Cache)
    sink_ptr = ctypes.c_void_p(sink.data_ptr())
    for label, size in (("read_GBps_58.7MB", 58720256), ("read_GBps_117.4MB", 117440512)):
        wins = nbytes // size

        def windows(size=size, wins=wins):
            s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for w in range(wins):
                rc = mlib.blmeasure_stream_read(ctypes.c_void_p(src.data_ptr() + w * size), size, sink_ptr, s)
                if rc:
                    raise RuntimeError(f"blmeasure_stream_read failed ({rc})")

        ms = _graph_time_ms(torch, windows, 5)
        out[label] = round(size * wins / (ms * 1e-3) / 1e9, 1)
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    sys.exit(main())
