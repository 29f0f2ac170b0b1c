#!/usr/bin/env python3
"""Benchmark of the block-scaled GEMM on one MI355X.

Headline: MXFP8 GEMM M=N=K=4096 (inputs ~N(0,1) fp32, 5% of rows of A and of B scaled x1000,
quantised per 32-K block to E4M3 with E8M0 scale 2^ceil(log2(amax/448))), fp32 accumulation,
BF16 output, alpha = 0.5.  One step = one bsg_run call (plan created once; inputs resident in HBM).
Reported value: whole-job TFLOP/s = 2*M*N*K / host wall time per step.

Also reported, in "extra": the other workloads (MXFP8 8192^3 fp16 with bias+SiLU, NVFP4
128x8192x8192 bias+SiLU, MXFP8 256^3) and the looped small-M NVFP4 GEMM (M=256, N=K=4096, 10 input
sets x 100 calls) as host wall time per call vs GPU time per call, direct and from HIP graphs.

The CPU baseline is the fp64 oracle (test infrastructure) timed on the host cores on a bounded sample
of rows of the headline workload.

Scales are row-major by default (the ABI default).  --scale-layout ktile runs every workload on the
library's K-tile-major scale layout instead (BSG_SCALES_KTILE; scales converted by bsg_pack_scales
before timing, as the MXFP8 page's test swizzles its scales before the GEMM); the default run also
reports the headline and the NVFP4 128x8192x8192 workload on that layout in "extra".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only-main] [--calibration-copy]
                       [--scale-layout linear|ktile]
       python bench.py --counters-from FETCH_CSV WRITE_CSV   (records HBM traffic from rocprofv3 passes)
       python bench.py --api-loop N   (N direct calls per workload only, for rocprofv3 --hip-trace)
       python bench.py --only-workload NAME [--steps K --warmup W]   (one workload only, for
                      rocprofv3 counter passes; prints its timing, not the benchmark line)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"mxfp8": 5000.0, "nvfp4_fp4": 10100.0, "bf16": 2500.0}  # MI355X dense, published
HBM_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "mxfp8_4096_counters.json")


# Sources of the headline kernel (mxfp8_pp): committed counters are valid only for these bytes.
HEADLINE_SOURCES = ("mxfp8_pp.hip", "common.h", "epilogue.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in HEADLINE_SOURCES:
        with open(os.path.join(ROOT, "block_scaled_precision_gemm_amd", "csrc", name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def write_counters(fetch_csv: str, write_csv: str) -> int:
    """Turn two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE; each over `bench.py --only-main
    --calibration-copy`) into profiles/mxfp8_4096_counters.json.  FETCH_SIZE / WRITE_SIZE are scaled by
    what they read for the 256 MiB device copy of known size."""
    import csv
    import statistics

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: statistics.mean(v) for k, v in vals.items()}

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    gemm = [k for k in fetch if "mxfp8_pp_kernel" in k]
    copy = [k for k in fetch if "copyBuffer" in k]
    if len(gemm) != 1 or len(copy) != 1:
        print(f"expected one GEMM and one copy kernel, got {list(fetch)}", file=sys.stderr)
        return 1
    g, c = gemm[0], copy[0]
    n = float(1 << 28)
    rf, wf = n / (fetch[c] * 1024), n / (write[c] * 1024)
    traffic = fetch[g] * 1024 * rf + write[g] * 1024 * wf
    M = N = K = 4096
    out = {
        "kernel": g, "workload": "MXFP8 4096^3 bf16 alpha 0.5",
        "fetch_kib_per_dispatch": fetch[g], "write_kib_per_dispatch": write[g],
        "copy_calibration": {"bytes_read": n, "bytes_written": n, "fetch_kib": fetch[c], "write_kib": write[c],
                             "read_factor": rf, "write_factor": wf},
        "traffic_bytes_per_launch": traffic,
        "algorithmic_bytes_per_launch": M * K + N * K + (M + N) * K // 32 + 2 * M * N,
        "source_hash": kernel_source_hash(),
        "commands": [f"rocprofv3 --pmc {x} -f csv -d <repo>/gpurun_out/pmc_{x.lower()} -o run -- python3 <repo>/bench.py "
                     "--only-main --steps 20 --warmup 5 --calibration-copy" for x in ("FETCH_SIZE", "WRITE_SIZE")],
    }
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def device_inputs(p: dict, scale_layout: str = "linear"):
    import numpy as np
    import torch
    import block_scaled_precision_gemm_amd as bsg
    d = {k: torch.from_numpy(np.ascontiguousarray(p[k])).cuda() for k in ("A", "B", "sA", "sB")}
    if scale_layout == "ktile":  # one-time layout conversion, outside any timed region
        for key, rows in (("sA", p["M"]), ("sB", p["N"])):
            kb = p[key].shape[1]
            packed = torch.empty(bsg.scales_ktile_bytes(rows, kb), dtype=torch.uint8, device="cuda")
            bsg.pack_scales(d[key], packed, rows, kb)
            d[key] = packed
        torch.cuda.synchronize()
    d["bias"] = None if p["bias"] is None else torch.from_numpy(np.ascontiguousarray(p["bias"])).cuda()
    d["D"] = torch.empty((p["M"], p["N"]), dtype=torch.int16, device="cuda")
    return d


def time_gemm(p: dict, steps: int, warmup: int, stream, scale_layout: str = "linear") -> dict:
    """Warm up, then time `steps` back-to-back calls on `stream` (host wall and HIP events)."""
    import torch
    import block_scaled_precision_gemm_amd as bsg
    plan = bsg.Plan(p["fmt"], p["M"], p["N"], p["K"], out=p["out"], bias=p["bias"] is not None, silu=p["silu"],
                    scale_layout=scale_layout)
    d = device_inputs(p, scale_layout)
    args = (d["A"], d["B"], d["sA"], d["sB"], d["D"])
    kw = dict(alpha=float(p["alpha"]), bias=d["bias"], stream=stream)
    for _ in range(warmup):
        plan.run(*args, **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        plan.run(*args, **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    flops = 2.0 * p["M"] * p["N"] * p["K"]
    wall_ms = (t1 - t0) * 1e3 / steps
    gpu_ms = e0.elapsed_time(e1) / steps
    info = plan.info()
    plan.close()
    return dict(variant=info["variant"], grid=info["grid"], wall_ms=wall_ms, gpu_ms=gpu_ms,
                tflops_wall=flops / (wall_ms * 1e-3) / 1e12, tflops_gpu=flops / (gpu_ms * 1e-3) / 1e12, flops=flops)


def loop_bench(stream, n_sets: int = 10, calls: int = 100, scale_layout: str = "linear") -> dict:
    """Looped small-M NVFP4 GEMM: n_sets fresh seeded input sets x `calls` back-to-back calls."""
    import torch
    import block_scaled_precision_gemm_amd as bsg
    import seeded_inputs as si
    sets_host = [si.workload("nvfp4_256x4096x4096_loop", set_id=s) for s in range(n_sets)]
    p0 = sets_host[0]
    plan = bsg.Plan("nvfp4", p0["M"], p0["N"], p0["K"], out="bf16", scale_layout=scale_layout)
    sets = []
    for p in sets_host:
        d = device_inputs(p, scale_layout)
        d["alpha"] = float(p["alpha"])
        sets.append(d)
    # warm-up (first-launch costs, caches)
    bsg.bench_loop(plan, sets, 5, 0, stream)
    direct_us = bsg.bench_loop(plan, sets, calls, 0, stream)
    graph_us = bsg.bench_loop(plan, sets, calls, 1, stream)
    # GPU time per call: HIP events around 1000 back-to-back calls on the same stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for d in sets:
        for _ in range(calls):
            plan.run(d["A"], d["B"], d["sA"], d["sB"], d["D"], alpha=d["alpha"], stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    n = n_sets * calls
    gpu_us = e0.elapsed_time(e1) * 1e3 / n
    flops = 2.0 * p0["M"] * p0["N"] * p0["K"]
    info = plan.info()
    plan.close()
    return dict(variant=info["variant"], calls=n, gpu_us_per_call=gpu_us,
                wall_us_per_call_direct=direct_us / n, wall_us_per_call_graph=graph_us / n,
                overhead_pct_direct=100.0 * (direct_us / n - gpu_us) / gpu_us,
                overhead_pct_graph=100.0 * (graph_us / n - gpu_us) / gpu_us,
                tflops_gpu=flops / (gpu_us * 1e-6) / 1e12)


def api_loop(n: int, stream) -> int:
    """N direct calls per workload from the native loop and nothing else timed: run twice under
    `rocprofv3 --hip-trace --stats` with different N, the difference of the HIP API call counts is
    what N calls of bsg_run cost (setup, uploads and plan creation cancel)."""
    import torch
    import block_scaled_precision_gemm_amd as bsg
    import seeded_inputs as si
    for name in ("nvfp4_256x4096x4096_loop", "mxfp8_4096"):
        p = si.workload(name)
        plan = bsg.Plan(p["fmt"], p["M"], p["N"], p["K"], out=p["out"], bias=p["bias"] is not None, silu=p["silu"])
        d = device_inputs(p)
        d["alpha"] = float(p["alpha"])
        torch.cuda.synchronize()
        us = bsg.bench_loop(plan, [d], n, 0, stream)
        log(f"api loop {name}: {n} calls, {us / n:.2f} us per call, variant {plan.info()['variant']}")
        plan.close()
    return 0


def cpu_baseline(p: dict, budget_s: float = 12.0) -> dict:
    """The oracle as it stands, timed on host cores over row chunks of the workload until the budget."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import oracle
    chunk = 256
    rows_done, t_total = 0, 0.0
    while t_total < budget_s and rows_done < p["M"]:
        rows = np.arange(rows_done, min(rows_done + chunk, p["M"]))
        t0 = time.perf_counter()
        oracle.reference(p, rows=rows)
        t_total += time.perf_counter() - t0
        rows_done += len(rows)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    flops = 2.0 * rows_done * p["N"] * p["K"]
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle (dequantise, A x B^T and sum|ab| via numpy/BLAS, epilogue, bf16 rounding) "
                      f"on rows 0..{rows_done - 1} of the {p['M']}x{p['N']}x{p['K']} workload, "
                      f"{t_total:.1f} s in {rows_done // chunk + (rows_done % chunk > 0)} chunks of {chunk} rows"}


def traffic_from_counters(gpu_ms: float) -> dict | None:
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if taken on the current kernels."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        c = json.load(f)
    if c.get("source_hash") != kernel_source_hash():
        return None
    return dict(bytes=c["traffic_bytes_per_launch"], gbs=c["traffic_bytes_per_launch"] / (gpu_ms * 1e-3) / 1e9)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--only-main", action="store_true", help="time the headline workload only (for profiling)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="after timing, run a device copy of known size (HBM counter calibration)")
    ap.add_argument("--api-loop", type=int, metavar="N",
                    help="only run N direct bsg_run calls per workload (NVFP4 256x4096x4096 split-K, MXFP8 "
                         "4096^3) from the native loop, for counting HIP API calls under rocprofv3 --hip-trace")
    ap.add_argument("--only-workload", metavar="NAME",
                    help="time one workload only (mxfp8_256, mxfp8_4096, mxfp8_8192_silu, nvfp4_128x8192x8192_silu, "
                         "nvfp4_256x4096x4096_loop) and print its timing (for profiling)")
    ap.add_argument("--scale-layout", choices=("linear", "ktile"), default="linear",
                    help="scale layout of every workload (default: row-major, the ABI default)")
    ap.add_argument("--counters-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: write the headline kernel's HBM-traffic record from two rocprofv3 passes")
    args = ap.parse_args()
    if args.counters_from:
        return write_counters(*args.counters_from)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import block_scaled_precision_gemm_amd as bsg
    import seeded_inputs as si
    bsg.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    if args.api_loop:
        return api_loop(args.api_loop, stream)
    if args.only_workload:
        r = time_gemm(si.workload(args.only_workload), args.steps, args.warmup, stream, args.scale_layout)
        print(json.dumps({"workload": args.only_workload, "scale_layout": args.scale_layout,
                          **{k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items()}}), flush=True)
        return 0

    log("generating the headline workload (MXFP8 4096^3)")
    p = si.workload("mxfp8_4096")
    lay = args.scale_layout
    main_r = time_gemm(p, args.steps, args.warmup, stream, lay)
    log(f"main: {main_r}")
    if args.calibration_copy:
        n = 1 << 28  # 256 MiB read + 256 MiB written per copy
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: 5 x {n} bytes")

    extra = {}
    if not args.only_main:
        # warm-up lengths cover the clock / power transient of the first few hundred calls
        for name, steps, warm in (("mxfp8_8192_silu", 30, 60), ("nvfp4_128x8192x8192_silu", 200, 400),
                                  ("mxfp8_256", 500, 500)):
            log(f"workload {name}")
            q = si.workload(name)
            r = time_gemm(q, steps, warm, stream, lay)
            peak = PEAK_TFLOPS["mxfp8"] if q["fmt"] == "mxfp8" else PEAK_TFLOPS["nvfp4_fp4"]
            r["frac_of_mx_peak"] = r["tflops_gpu"] / peak
            if q["fmt"] == "nvfp4":
                r["frac_of_bf16_peak"] = r["tflops_gpu"] / PEAK_TFLOPS["bf16"]
            extra[name] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items() if k != "flops"}
            log(f"{name}: {extra[name]}")
        log("looped NVFP4 256x4096x4096, 10 sets x 100 calls")
        extra["nvfp4_256x4096x4096_loop"] = {k: (round(v, 3) if isinstance(v, float) else v)
                                             for k, v in loop_bench(stream, scale_layout=lay).items()}
        log(f"loop: {extra['nvfp4_256x4096x4096_loop']}")
        if lay == "linear":
            for name, steps, warm in (("mxfp8_4096", args.steps, 100), ("nvfp4_128x8192x8192_silu", 200, 100)):
                q = p if name == "mxfp8_4096" else si.workload(name)
                r = time_gemm(q, steps, warm, stream, "ktile")
                extra[name + "_ktile_scales"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                                 for k, v in r.items() if k != "flops"}
                log(f"{name} on K-tile-major scales: {extra[name + '_ktile_scales']}")

    cpu = None
    if not args.only_main:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(p)

    achieved = main_r["tflops_gpu"]
    peak = PEAK_TFLOPS["mxfp8"]
    tr = traffic_from_counters(main_r["gpu_ms"])
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None if tr is None else tr["bytes"],
                "kernel": main_r["variant"], "kernel_ms": round(main_r["gpu_ms"], 5),
                "flops_per_launch": main_r["flops"]}
    line = {
        "metric": "block-scaled GEMM TFLOPS (% of MX MFMA peak) + per-call loop us vs kernel us",
        "value": round(main_r["tflops_wall"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_r["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8_e4m3",
        "data": "synthetic (seeded N(0,1), 5% rows x1000, quantised to MXFP8 on the host)",
        "config": {"workload": "MXFP8 GEMM M=N=K=4096, E4M3 + E8M0/32, alpha=0.5, bf16 out, 5% outlier rows",
                   "M": p["M"], "N": p["N"], "K": p["K"], "out": "bf16", "alpha": 0.5,
                   "scale_layout": "row-major" if lay == "linear" else "K-tile-major (packed before timing)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
