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

Prints ONE JSON line with the metric, µs/call, HBM GB/s and TFLOP/s, the
roofline of the kernel and the CPU oracle's time on a bounded sample.

Counter mode: ``python bench.py --traffic-from FETCH_CSV WRITE_CSV`` reads the
rocprofv3 counter_collection.csv files of a FETCH_SIZE run and a WRITE_SIZE
run of ``bench.py --calib-copy-mb N`` and prints the HBM traffic per launch of
the GEMM kernel, each counter scaled by what it reads for the plain device
copy of known size that the same run performed.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
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
KERNEL = "nvfp4_group_gemm_kernel"
MX_KERNEL = "mxfp4_group_gemm_kernel"
BLOCKED_KERNEL = "nvfp4_blocked_sf_gemm_kernel"
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 MFMA
CALIB_KERNEL = "neg"            # torch.neg's elementwise kernel: reads and writes the copy size
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_grouped_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=workloads.HEADLINE["name"],
                    help="workload name (default: the g=8 K=7168 N=4096 grouped GEMM)")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets rotated through (0: enough to exceed 384 MB, at most 64)")
    ap.add_argument("--format", choices=("nvfp4", "mxfp4"), default="nvfp4",
                    help="nvfp4 (E4M3 scale per 16 K, the headline) or mxfp4 (E8M0 scale per 32 K, "
                         "mxfp4_group_gemm on the block-scaled FP4 MFMA)")
    ap.add_argument("--batch", type=int, default=1,
                    help="L > 1: every group a batch of L independent products (nvfp4_group_gemm_batched)")
    ap.add_argument("--sf-layout", choices=("row-major", "blocked"), default="row-major",
                    help="scale layout: row-major (nvfp4_group_gemm) or the blocked 128 x 4 atom "
                         "layout (nvfp4_group_gemm_blocked)")
    ap.add_argument("--launch-per-group", action="store_true",
                    help="one launch per group instead of one grouped launch (for comparison)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run 3 device copies of this many MiB (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the counter-derived traffic per launch and exit (no GPU use)")
    ap.add_argument("--counters-from", nargs="+", metavar="CSV",
                    help="print the GEMM kernel's per-dispatch counter means from rocprofv3 "
                         "counter_collection.csv files and exit (no GPU use)")
    ap.add_argument("--stats-from", metavar="CSV",
                    help="print the GEMM kernel's row of a rocprofv3 kernel_stats.csv and exit (no GPU use)")
    return ap.parse_args()


def kernel_name(args) -> str:
    """The GEMM kernel a run launches."""
    if args.format == "mxfp4":
        return MX_KERNEL
    return BLOCKED_KERNEL if args.sf_layout == "blocked" else KERNEL


def source_digest() -> str:
    """sha256 over the kernel sources, so stored counter figures are only
    used for the kernel they were taken on."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_file(workload: str, kernel: str = KERNEL) -> str:
    return os.path.join(PROFILES, "%s_%s_traffic.txt" % (kernel, workload))


def read_traffic(workload: str, kernel: str = KERNEL):
    """Bytes per launch from the stored counter summary, or None when there
    is none or it was taken on other kernel sources."""
    path = traffic_file(workload, kernel)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#", "|")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def counter_means(path: str):
    """{kernel name: (dispatches, mean counter value)} of a counter_collection.csv."""
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in acc.items()}


def traffic_from(fetch_csv: str, write_csv: str, copy_mb: int, kernel: str = KERNEL):
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        means = counter_means(path)
        gemm = [v for k, v in means.items() if kernel in k]
        calib = [v for k, v in means.items() if CALIB_KERNEL in k and kernel not in k]
        if len(gemm) != 1 or len(calib) != 1:
            raise SystemExit("%s: expected one GEMM and one copy kernel, found %s" % (path, list(means)))
        known_kib = copy_mb * 1024.0
        factor = known_kib / calib[0][1]
        out[counter] = dict(gemm_kib=gemm[0][1], gemm_dispatches=gemm[0][0], copy_kib=calib[0][1],
                            factor=factor, bytes=gemm[0][1] * factor * 1024.0)
    return out


def make_device_sets(cfg, nsets, torch, blocked=False, blocked_bytes=None, fmt="nvfp4"):
    """Device copies of nsets input sets.  With blocked scales, each scale
    array is a fresh draw of scale codes of the blocked array's size (the
    timing does not depend on which valid scale sits where)."""
    sets = []
    for v in range(nsets):
        if fmt == "mxfp4":
            A, B, SA, SB = workloads.make_mx_inputs(cfg["M"], cfg["N"], cfg["K"], cfg["seed"], variant=v)
        else:
            A, B, SA, SB = workloads.config_inputs(cfg, variant=v)
        if blocked:
            kk = cfg["K"]
            SA = [workloads.scale_codes(workloads.stream_key(cfg["seed"], v, i, 101), blocked_bytes(m, k))
                  for i, (m, k) in enumerate(zip(cfg["M"], kk))]
            SB = [workloads.scale_codes(workloads.stream_key(cfg["seed"], v, i, 102), blocked_bytes(n, k))
                  for i, (n, k) in enumerate(zip(cfg["N"], kk))]
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        sets.append(dict(A=[dev(a) for a in A], B=[dev(b) for b in B],
                         SA=[dev(s) for s in SA], SB=[dev(s) for s in SB],
                         C=[torch.empty((m, n), dtype=torch.float16, device="cuda")
                            for m, n in zip(cfg["M"], cfg["N"])]))
    return sets


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, target_s, fmt="nvfp4"):
    """The oracle, as it is (plain C, -O3, OpenMP over output rows), timed on
    a bounded sample of the workload: the first r_i rows of every group (all
    N_i columns, all K_i), r_i the same fraction of M_i in each group, sized
    so that one run on all host threads takes about target_s / 3.  That run
    is repeated three times (the median is reported), and 1/threads of the
    rows is run once on one thread.  Both are extrapolated to the whole
    workload by multiply-add count (the oracle's cost per multiply-add does
    not depend on which rows it computes)."""
    import oracle
    oracle.build(force=False)
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    g = len(M)
    if fmt == "mxfp4":
        mx = workloads.make_mx_inputs(M, N, K, cfg["seed"])
        inputs = [tuple(x[i] for x in mx) for i in range(g)]
        run_oracle = oracle.mx_group_gemm
    else:
        inputs = [workloads.make_group(cfg["seed"], i, M[i], N[i], K[i]) for i in range(g)]
        run_oracle = oracle.group_gemm
    total_macs = sum(m * n * k for m, n, k in zip(M, N, K))
    threads = oracle.max_threads()

    def run(frac, nthreads):
        rows = [max(1, min(M[i], int(round(M[i] * frac)))) for i in range(g)]
        A = [inputs[i][0][:rows[i]] for i in range(g)]
        SA = [inputs[i][2][:rows[i]] for i in range(g)]
        t0 = time.perf_counter()
        run_oracle(rows, N, K, A, [x[1] for x in inputs], SA, [x[3] for x in inputs], nthreads=nthreads)
        t = time.perf_counter() - t0
        return rows, sum(r * n * k for r, n, k in zip(rows, N, K)), t

    one = target_s / 3
    frac = min(1.0, threads / max(1.0, sum(M)))
    rows, macs, t = run(frac, threads)
    while t < one / 4 and frac < 1.0:
        frac = min(1.0, frac * 2)
        rows, macs, t = run(frac, threads)
    if t < one * 0.7 and frac < 1.0:
        frac = min(1.0, frac * one / max(t, 1e-3))
    times = []
    for _ in range(3):
        rows, macs, t = run(frac, threads)
        times.append(t)
    t_med = float(np.median(times))
    rows1, macs1, t1 = run(frac / threads, 1)
    return {"value": round(t_med * 1e6 * total_macs / macs, 1), "unit": "µs/call", "cores": threads,
            "kind": "oracle",
            "sample": "first rows %s of the %d groups (all N, all K): %d of %d multiply-adds (%.2f%%), "
                      "median of 3 runs on %d threads (%s s), extrapolated to the whole workload by "
                      "multiply-add count" % (rows, g, macs, total_macs, 100.0 * macs / total_macs, threads,
                                              ", ".join("%.2f" % x for x in times)),
            "cpu_model": cpu_model(),
            "single_thread": {"value": round(t1 * 1e6 * total_macs / macs1, 1), "unit": "µs/call",
                              "sample": "first rows %s: %d multiply-adds in %.2f s on 1 thread, "
                                        "extrapolated by multiply-add count" % (rows1, macs1, t1)},
            "oracle_build": "gcc -O3 -fopenmp"}


def counters_from(paths, kernel: str):
    """Per-dispatch means of every counter in rocprofv3 counter_collection.csv
    files, for the dispatches of `kernel`."""
    out = {}
    for path in paths:
        acc = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"]:
                    acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for name, vals in acc.items():
            out[name] = {"dispatches": len(vals), "mean": sum(vals) / len(vals)}
    return out


def stats_from(path: str, kernel: str):
    """The row of `kernel` in a rocprofv3 kernel_stats.csv."""
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Name"]:
                return {k: r[k] for k in ("Name", "Calls", "AverageNs", "MinNs", "MaxNs", "StdDev") if k in r}
    raise SystemExit("%s: no row for %s" % (path, kernel))


def main():
    args = parse()
    if args.traffic_from:
        mb = args.calib_copy_mb or 512
        t = traffic_from(args.traffic_from[0], args.traffic_from[1], mb, kernel_name(args))
        total = int(round(t["FETCH_SIZE"]["bytes"] + t["WRITE_SIZE"]["bytes"]))
        print("source_sha256: %s" % source_digest())
        print("calib_copy_mib: %d" % mb)
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            v = t[c]
            print("%s: kernel mean %.1f KiB over %d dispatches; copy %.1f KiB; factor %.4f; %d bytes per launch"
                  % (c, v["gemm_kib"], v["gemm_dispatches"], v["copy_kib"], v["factor"], round(v["bytes"])))
        print("fetch_bytes_per_launch: %d" % round(t["FETCH_SIZE"]["bytes"]))
        print("write_bytes_per_launch: %d" % round(t["WRITE_SIZE"]["bytes"]))
        print("traffic_bytes_per_launch: %d" % total)
        return
    if args.counters_from:
        print("source_sha256: %s" % source_digest())
        for name, v in sorted(counters_from(args.counters_from, kernel_name(args)).items()):
            print("%s: %.1f (mean of %d dispatches)" % (name, v["mean"], v["dispatches"]))
        return
    if args.stats_from:
        print("source_sha256: %s" % source_digest())
        for k, v in stats_from(args.stats_from, kernel_name(args)).items():
            print("%s: %s" % (k, v))
        return
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
    mx = args.format == "mxfp4"
    if args.batch > 1 and (mx or args.sf_layout == "blocked"):
        print("bench.py: the batched entry point takes NVFP4 row-major scales only", file=sys.stderr)
        sys.exit(2)
    if args.launch_per_group and args.batch > 1:
        print("bench.py: --launch-per-group takes batch L = 1", file=sys.stderr)
        sys.exit(2)
    if mx and args.sf_layout == "blocked":
        print("bench.py: the MXFP4 entry point takes row-major scales only", file=sys.stderr)
        sys.exit(2)
    abytes = workloads.algorithmic_bytes(M, N, K, 32 if mx else 16) * args.batch
    flops = workloads.algorithmic_flops(M, N, K) * args.batch
    nsets = args.sets or min(64, max(1, -(-384 * 2 ** 20 // abytes)))
    blocked = args.sf_layout == "blocked"
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    if args.batch > 1:
        # Every group a batch of L slices (input variants v L .. v L + L - 1),
        # consecutive in one allocation per operand.
        sets = []
        for v in range(nsets):
            parts = [workloads.config_inputs(cfg, variant=v * args.batch + l) for l in range(args.batch)]
            cat = lambda j, i: torch.from_numpy(np.ascontiguousarray(
                np.concatenate([p[j][i].reshape(-1) for p in parts]))).cuda()
            sets.append(dict(A=[cat(0, i) for i in range(len(M))], B=[cat(1, i) for i in range(len(M))],
                             SA=[cat(2, i) for i in range(len(M))], SB=[cat(3, i) for i in range(len(M))],
                             C=[torch.empty(args.batch * m * n, dtype=torch.float16, device="cuda")
                                for m, n in zip(M, N)]))
        Ls = [args.batch] * len(M)
        calls = [(lambda s=s: nv.group_gemm_batched_ptrs(
            M, N, K, Ls, [t.data_ptr() for t in s["A"]], [t.data_ptr() for t in s["B"]],
            [t.data_ptr() for t in s["SA"]], [t.data_ptr() for t in s["SB"]], [t.data_ptr() for t in s["C"]], sh))
            for s in sets]
    else:
        sets = make_device_sets(cfg, nsets, torch, blocked, nv.blocked_scale_bytes, args.format)
        calls = [nv.GroupGemmCall(M, N, K, [t.data_ptr() for t in s["A"]], [t.data_ptr() for t in s["B"]],
                                  [t.data_ptr() for t in s["SA"]], [t.data_ptr() for t in s["SB"]],
                                  [t.data_ptr() for t in s["C"]], sh, blocked=blocked, fmt=args.format)
                 for s in sets]
        if args.launch_per_group:
            # The same products as g launches of one group each, back to
            # back on one stream: what a grouped launch saves.
            def per_group(s):
                one = [nv.GroupGemmCall(M[i:i + 1], N[i:i + 1], K[i:i + 1], [s["A"][i].data_ptr()],
                                        [s["B"][i].data_ptr()], [s["SA"][i].data_ptr()],
                                        [s["SB"][i].data_ptr()], [s["C"][i].data_ptr()], sh,
                                        blocked=blocked, fmt=args.format) for i in range(len(M))]

                def run():
                    for c in one:
                        rc = c()
                        if rc != nv.OK:
                            return rc
                    return nv.OK
                return run
            calls = [per_group(s) for s in sets]

    def step(i):
        rc = calls[i % nsets]()
        if rc != nv.OK:
            raise RuntimeError(nv.last_error())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Events on the stream the kernel is launched on, one between every two
    # calls: the mean gap is the kernel's average duration in the loop.
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
        n = args.calib_copy_mb * 2 ** 20 // 4     # fp32 elements: reads and writes calib_copy_mb MiB
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()

    gbps = abytes / us / 1e3
    tflops = flops / us / 1e6
    traffic = read_traffic(cfg["name"], kernel_name(args))
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
                   "sf_layout": args.sf_layout, "input_sets_rotated": nsets},
        "us_per_call": {"mean": round(us, 3), "std": round(float(per.std()), 3),
                        "min": round(float(per.min()), 3), "max": round(float(per.max()), 3),
                        "wall_mean": round(wall / args.steps * 1e6, 3)},
        "achieved_hbm_GBps": round(gbps, 1),
        "achieved_TFLOPs": round(tflops, 1),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "hbm": {"achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes": abytes}},
    }
    if args.batch > 1:
        out["config"]["batch_L"] = args.batch
        out["config"]["workload"] = cfg["name"] + "_l%d" % args.batch
        out["roofline"]["traffic"] = None
    if mx:
        # The FP4 MFMA floor (5.95 us at g8 K7168 N4096) lies far below the
        # HBM one: this form is bound by HBM.
        out["config"]["format"] = "mxfp4"
        out["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                           "algorithmic_bytes": abytes,
                           "mfma": {"achieved": round(tflops, 1), "peak": FP4_MFMA_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(tflops / FP4_MFMA_PEAK_TFLOPS, 4)}}
        out["dtype"] = "fp4"
        out["metric"] = METRIC.replace("NVFP4", "MXFP4")
    if args.launch_per_group:
        out["config"]["launches"] = "one per group"
        out["config"]["workload"] = cfg["name"] + "_per_group_launches"
        out["roofline"]["traffic"] = None
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, args.format)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
