#!/usr/bin/env python3
"""Benchmark of the NVFP4 block-scaled grouped GEMM on one MI355X.

One step = one nvfp4_group_gemm call over all groups of the workload (the
whole hot path: dequantisation, MFMA contraction and fp16 epilogue run in the
one kernel launch).  The default workload is the g=8, K=7168, N=4096 grouped
GEMM (M = 80,176,128,72,64,248,96,160), with synthetic seeded inputs resident
in HBM before timing starts.

Infinity-Cache hygiene: B alone is 117 MB and the MI355X's 256 MB MALL would
hold it between back-to-back calls, so the timed loop rotates through several
independent input sets (435 MB for three) and each call reads inputs the
previous calls did not touch.

Prints ONE JSON line (rank 0) with the metric, µs/call, HBM GB/s and TFLOP/s,
the roofline of the kernel and the CPU oracle's time on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "µs/call + achieved HBM GB/s & TFLOP/s, NVFP4 grouped GEMM g=8 K=7168 N=4096"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=workloads.HEADLINE["name"],
                    help="workload name (default: the g=8 K=7168 N=4096 grouped GEMM)")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets rotated through (0: enough to exceed 384 MB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run one device copy of this many MB (counter calibration)")
    return ap.parse_args()


def make_device_sets(cfg, nsets, torch):
    sets = []
    for v in range(nsets):
        A, B, SA, SB = workloads.config_inputs(cfg, variant=v)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        sets.append(dict(A=[dev(a) for a in A], B=[dev(b) for b in B],
                         SA=[dev(s) for s in SA], SB=[dev(s) for s in SB],
                         C=[torch.empty((m, n), dtype=torch.float16, device="cuda")
                            for m, n in zip(cfg["M"], cfg["N"])]))
    return sets


def cpu_baseline(cfg, target_s):
    """The oracle, as it is, on the first rows of group 0 (all N, all K),
    scaled to the whole workload by multiply-add count."""
    import oracle
    oracle.build(force=False)
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    A, B, SA, SB = workloads.make_group(cfg["seed"], 0, M[0], N[0], K[0])
    total_macs = sum(m * n * k for m, n, k in zip(M, N, K))
    threads = oracle.max_threads()

    def run(rows):
        t0 = time.perf_counter()
        oracle.group_gemm([rows], [N[0]], [K[0]], [A[:rows]], [B], [SA[:rows]], [SB],
                          nthreads=threads)
        return time.perf_counter() - t0

    rows = max(1, min(M[0], threads))
    t = run(rows)
    while t < target_s / 4 and rows < M[0]:
        rows = min(M[0], rows * 2)
        t = run(rows)
    if t < target_s and rows < M[0]:
        rows = min(M[0], max(rows, int(rows * target_s / max(t, 1e-3))))
        t = run(rows)
    macs = rows * N[0] * K[0]
    us_per_call = t * 1e6 * total_macs / macs
    return {"value": us_per_call, "unit": "µs/call", "cores": threads, "kind": "oracle",
            "sample": "group 0 rows 0..%d (all %d columns, K=%d): %d of %d multiply-adds, %.1f s, "
                      "scaled to the whole workload" % (rows - 1, N[0], K[0], macs, total_macs, t)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(the grouped GEMM would shard whole groups or N-slices across GPUs with no "
              "exchange step; that path is not built)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_block_scaled_grouped_amd as nv
    nv.load()
    cfg = next(c for c in workloads.CONFIGS if c["name"] == args.config)
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    abytes = workloads.algorithmic_bytes(M, N, K)
    flops = workloads.algorithmic_flops(M, N, K)
    nsets = args.sets or max(1, -(-384 * 2 ** 20 // abytes))
    sets = make_device_sets(cfg, nsets, torch)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    ptrs = [dict(A=[t.data_ptr() for t in s["A"]], B=[t.data_ptr() for t in s["B"]],
                 SA=[t.data_ptr() for t in s["SA"]], SB=[t.data_ptr() for t in s["SB"]],
                 C=[t.data_ptr() for t in s["C"]]) for s in sets]

    def step(i):
        p = ptrs[i % nsets]
        rc = nv.group_gemm_ptrs(M, N, K, p["A"], p["B"], p["SA"], p["SB"], p["C"], sh)
        if rc != nv.OK:
            raise RuntimeError(nv.last_error())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(args.steps)])  # µs
    us = float(per.mean())

    if args.calib_copy_mb > 0:
        src = torch.empty(args.calib_copy_mb * 2 ** 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    gbps = abytes / us / 1e3
    tflops = flops / us / 1e6
    out = {
        "metric": METRIC,
        "value": round(us, 3),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "g": len(M), "M": M, "N": N[0], "K": K[0],
                   "input_sets_rotated": nsets},
        "us_per_call": {"mean": round(us, 3), "std": round(float(per.std()), 3),
                        "min": round(float(per.min()), 3), "max": round(float(per.max()), 3),
                        "wall_mean": round(wall / args.steps * 1e6, 3)},
        "achieved_hbm_GBps": round(gbps, 1),
        "achieved_TFLOPs": round(tflops, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": None,
                     "hbm": {"achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(gbps / HBM_PEAK_GBPS, 4)}},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
