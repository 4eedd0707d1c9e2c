"""Benchmark: int8 implicit-GEMM conv2d fprop on one MI355X.

One step = one conv2d_fprop_run of the headline workload (int8 3x3 conv, N32
C256 28x28 K256, stride 1, pad 1, NCxHWx<32> / CxRSKx<32>, fused alpha / rint /
saturate epilogue) on inputs already resident in HBM.  Prints ONE JSON line.

Secondary measurements (same line, key "extra"): microseconds per call of the
smallest shape (device events, host wall clock, graph replay), the strided
3x3 workload, the fp32 dilated workload and the layout transforms.  The CPU
oracle is timed on the host as a reported baseline ("cpu_baseline").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8 conv fprop TOPS (% of MFMA int8 peak); µs/call at smallest shape"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
# every source that shapes the int8 kernels' code or launch
# Every source the library is built from: a counter summary whose hash no
# longer matches was taken on other code and is not reported.
KERNEL_SOURCES = sorted(
    os.path.relpath(os.path.join(dp, fn), ROOT)
    for dp, _, fns in os.walk(os.path.join(ROOT, "convolution_forward_gemm_amd", "csrc"))
    for fn in fns if fn.endswith((".hip", ".hpp", ".inc", ".h"))
) + ["convolution_forward_gemm_amd/build.py", "include/convfprop.h"]


def traffic_file(key: str) -> str:
    return os.path.join(PROFILES, "conv_i8_%s_traffic.json" % key)


def committed_traffic(key: str, config: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of a workload, or None unless the kernel sources and
    the configuration still match what was profiled."""
    tf = traffic_file(key)
    if not os.path.exists(tf):
        return None
    with open(tf) as f:
        tr = json.load(f)
    if (tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("workload") == key
            and tr.get("kernel_config") == config):
        return tr.get("hbm_bytes_per_launch")
    return None


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def conv_ops(wk, P, Q) -> int:
    return 2 * wk.N * wk.K * P * Q * wk.C * wk.R * wk.S


def conv_bytes(wk, P, Q, esize) -> int:
    return esize * (wk.N * wk.C * wk.H * wk.W + wk.K * wk.C * wk.R * wk.S + wk.N * wk.K * P * Q)


def setup(wk, torch, b):
    """Descriptor plus device-resident inputs/outputs in the kernel layouts."""
    from convolution_forward_gemm_amd import workloads as wl
    x, w = wl.make_inputs(wk)
    conv = b.Conv2dFprop(wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S, pad=wk.pad,
                         stride=wk.stride, dil=wk.dil, dtype=wk.dtype)
    if wk.dtype == "int8":
        xd = b.nchw_to_nc32hw32(torch.from_numpy(x).cuda())
        wd = b.kcrs_to_c32rsk32(torch.from_numpy(w).cuda())
        yd = torch.empty(conv.y_shape, dtype=torch.int8, device="cuda")
    else:
        xd = torch.from_numpy(x).cuda()
        wd = torch.from_numpy(w).cuda()
        yd = torch.empty(conv.y_shape, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    return conv, xd, wd, yd, (x, w)


def time_device(torch, fn, steps, warmup):
    """Average device time per call (ms) with HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def clock_ramp(torch, fn, min_ms=60.0, batch=200):
    """Sustained untimed load before any warm-up count: the GPU reaches its
    steady clock only after tens of milliseconds under load, so a short
    warm-up alone would time a still-ramping clock.  Launches fn in batches
    until at least min_ms of wall time has passed; returns (ms, launches)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(batch):
            fn()
        n += batch
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) * 1e3
        if el >= min_ms:
            return el, n


def latency_suite(torch, conv, xd, wd, yd, alpha, calls=1000):
    """p5-style microseconds per call: device events, host wall, graph replay."""
    stream = torch.cuda.current_stream().cuda_stream
    xp, wp, yp = xd.data_ptr(), wd.data_ptr(), yd.data_ptr()

    def call():
        conv.run_ptr(xp, wp, yp, alpha, stream)

    dev_ms = time_device(torch, call, calls, 50)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    host_us = (time.perf_counter() - t0) / calls * 1e6

    graph_us = None
    try:
        # the library's own capture of 20 back-to-back calls
        # (conv2d_fprop_graph_create), replayed on the current stream
        from convolution_forward_gemm_amd import binding as b
        g = b.ConvGraph(conv, xp, wp, yp, alpha, 20)
        g.launch(stream)
        torch.cuda.synchronize()
        reps = 50
        ms = time_device(torch, lambda: g.launch(stream), reps, 5)
        graph_us = ms * 1e3 / 20
        del g
    except Exception as e:  # graph capture is a secondary measurement
        graph_us = "unavailable: %s" % (type(e).__name__,)
    return {"device_us_per_call": round(dev_ms * 1e3, 3),
            "host_wall_us_per_call": round(host_us, 3),
            "graph_replay_us_per_call": graph_us if isinstance(graph_us, str) else round(graph_us, 3)}


def cold_run(torch, conv, xd, wd, yd, wk, ops, cache_bytes=256 << 20):
    """Average per call over calls that each use a different copy of the
    operands, the copies together more than twice the Infinity Cache, so a
    call finds none of its operands in any cache."""
    def slot(t):  # bytes per copy, rounded to 256 B (keeps 16-byte alignment)
        return -(-t.numel() * t.element_size() // 256) * 256
    per_set = slot(xd) + slot(wd) + slot(yd)
    sets = max(2, -(-2 * cache_bytes // per_set) + 1)
    bufs = []
    for t in (xd, wd):
        n = slot(t)
        big = torch.empty((sets, n), dtype=torch.uint8, device="cuda")
        big[:, : t.numel() * t.element_size()].copy_(
            t.reshape(-1).view(torch.uint8).unsqueeze(0).expand(sets, -1))
        bufs.append(big)
    ybig = torch.empty((sets, slot(yd)), dtype=torch.uint8, device="cuda")
    xb, wb, yb = bufs[0].data_ptr(), bufs[1].data_ptr(), ybig.data_ptr()
    sx, sw, sy = bufs[0].stride(0), bufs[1].stride(0), ybig.stride(0)
    ptrs = [(xb + i * sx, wb + i * sw, yb + i * sy) for i in range(sets)]
    stream = torch.cuda.current_stream().cuda_stream
    for xp, wp, yp in ptrs:  # one pass over every copy (warms the code, not the data)
        conv.run_ptr(xp, wp, yp, wk.alpha, stream)
    torch.cuda.synchronize()
    reps = max(1, 200 // sets)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        for xp, wp, yp in ptrs:
            conv.run_ptr(xp, wp, yp, wk.alpha, stream)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (reps * sets)
    del bufs, ybig
    return {"us_per_call": round(ms * 1e3, 3), "TOPS": round(ops / (ms * 1e-3) / 1e12, 3),
            "copies": sets, "bytes_per_copy": per_set}


def cpu_baseline(wk, x, w):
    """The oracle as it stands, on the host cores (rank 0, N=1 only)."""
    import oracle
    threads = min(16, os.cpu_count() or 1)
    try:
        threads = min(threads, len(os.sched_getaffinity(0)))
    except AttributeError:
        pass
    # Bounded sample: whole passes over the workload (all images, channels and
    # output pixels), repeated until about 10 s of CPU work (at most 30 passes);
    # a pass over a few images when one full pass would take longer.
    t0 = time.perf_counter()
    acc, y = oracle.conv2d_i8(x[:1], w, wk.alpha, **wk.conv_kwargs, nthreads=threads)
    per_image = time.perf_counter() - t0
    n = wk.N if per_image * wk.N <= 10.0 else max(1, int(10.0 / per_image))
    passes, dt = 0, 0.0
    while passes < 30 and (passes == 0 or dt < 10.0):
        t0 = time.perf_counter()
        acc, y = oracle.conv2d_i8(x[:n], w, wk.alpha, **wk.conv_kwargs, nthreads=threads)
        dt += time.perf_counter() - t0
        passes += 1
    P, Q = acc.shape[2:]
    ops = passes * 2 * n * wk.K * P * Q * wk.C * wk.R * wk.S
    # the same oracle on one thread, over one image
    t0 = time.perf_counter()
    oracle.conv2d_i8(x[:1], w, wk.alpha, **wk.conv_kwargs, nthreads=1)
    dt1 = time.perf_counter() - t0
    ops1 = 2 * wk.K * P * Q * wk.C * wk.R * wk.S
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": threads,
            "kind": "oracle",
            "sample": "%d pass(es) over %d of %d images of the headline workload (all %d output "
                      "channels, %dx%d outputs), int64 accumulation + epilogue; %.1f s"
                      % (passes, n, wk.N, wk.K, P, Q, dt),
            "single_thread_value": round(ops1 / dt1 / 1e12, 6),
            "single_thread_sample": "1 image, %.2f s" % dt1,
            "nproc": os.cpu_count(), "affinity_cpus": affinity}


# ---------------------------------------------------------------------------
# Summaries of rocprofv3 output (run on the host after the profiled runs)
# ---------------------------------------------------------------------------
def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(dirname, suffix):
    for root, _, files in os.walk(dirname):
        for fn in sorted(files):
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError("no *%s under %s" % (suffix, dirname))


def _conv_kernel(names):
    """The conv kernel among profiled kernel names (most dispatches wins)."""
    conv = [n for n in names if "convfprop::conv_" in n]
    if not conv:
        raise ValueError("no conv kernel among %d profiled kernels" % len(names))
    return max(conv, key=lambda n: names[n])


def summarize_trace(key, trace_dir, command, tag=""):
    from convolution_forward_gemm_amd import workloads as wl
    rows = _csv_rows(_find(trace_dir, "kernel_stats.csv"))
    calls = {r["Name"]: int(r["Calls"]) for r in rows}
    kname = _conv_kernel(calls)
    lines = ["rocprofv3 kernel-trace summary: " + wl.WORKLOADS[key].name,
             "command: " + command,
             "kernel source hash (%s): %s" % (", ".join(os.path.basename(k) for k in KERNEL_SOURCES),
                                             kernel_source_hash()),
             "",
             "%-100s %6s %12s %12s %12s %11s" % ("kernel", "calls", "avg_ns", "min_ns", "max_ns", "stddev_ns")]
    for r in rows:
        lines.append("%-100s %6d %12.1f %12d %12d %11.1f" % (
            r["Name"][:100], int(r["Calls"]), float(r["AverageNs"]), int(float(r["MinNs"])),
            int(float(r["MaxNs"])), float(r["StdDev"])))
    avg = next(float(r["AverageNs"]) for r in rows if r["Name"] == kname)
    wk = wl.WORKLOADS[key]
    from convolution_forward_gemm_amd import binding as b
    conv = b.Conv2dFprop(wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S, pad=wk.pad,
                         stride=wk.stride, dil=wk.dil, dtype=wk.dtype)
    ops = conv_ops(wk, conv.P, conv.Q)
    if wk.dtype == "int8":
        lines += ["", "conv kernel average %.2f us -> %.1f TOPS = %.1f%% of the %.1f POP/s int8 MFMA peak"
                  % (avg / 1e3, ops / avg / 1e3, 100 * ops / avg / 1e3 / PEAK_INT8_TOPS,
                     PEAK_INT8_TOPS / 1e3)]
    else:
        lines += ["", "conv kernel average %.2f us -> %.1f TFLOPS = %.1f%% of the %.1f TFLOPS fp32 MFMA peak"
                  % (avg / 1e3, ops / avg / 1e3, 100 * ops / avg / 1e3 / PEAK_FP32_TFLOPS, PEAK_FP32_TFLOPS)]
    prefix = "conv_i8" if wk.dtype == "int8" else "conv_f32"
    out = os.path.join(PROFILES, "%s_%s%s_kernel_trace.txt" % (prefix, key, tag))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


def summarize_traffic(key, fetch_dir, write_dir, copy_mib, commands):
    """HBM bytes per launch of the conv kernel: rocprofv3 FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for a plain device copy of known size in the same process."""
    from convolution_forward_gemm_amd import workloads as wl
    from convolution_forward_gemm_amd import binding as b

    def per_kernel(d, counter):
        acc, cnt = {}, {}
        for r in _csv_rows(_find(d, "counter_collection.csv")):
            if r["Counter_Name"] != counter:
                continue
            acc[r["Kernel_Name"]] = acc.get(r["Kernel_Name"], 0.0) + float(r["Counter_Value"])
            cnt[r["Kernel_Name"]] = cnt.get(r["Kernel_Name"], 0) + 1
        return {k: acc[k] / cnt[k] for k in acc}, cnt

    copy_bytes = copy_mib << 20
    fetch, fcnt = per_kernel(fetch_dir, "FETCH_SIZE")
    write, _ = per_kernel(write_dir, "WRITE_SIZE")
    kname = _conv_kernel(fcnt)
    copy_k = [k for k in fetch if "copyBuffer" in k or "copy" in k.lower() and "conv" not in k]
    if not copy_k:
        raise ValueError("the calibration copy kernel was not profiled")
    ck = max(copy_k, key=lambda k: fetch[k])
    f_factor = copy_bytes / (fetch[ck] * 1024)
    w_factor = copy_bytes / (write[ck] * 1024)
    rd = fetch[kname] * 1024 * f_factor
    wr = write[kname] * 1024 * w_factor
    wk = wl.WORKLOADS[key]
    conv = b.Conv2dFprop(wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S, pad=wk.pad,
                         stride=wk.stride, dil=wk.dil, dtype=wk.dtype)
    res = {
        "workload": key, "workload_name": wk.name, "kernel": kname,
        "kernel_config": conv.config, "kernel_source_hash": kernel_source_hash(),
        "fetch_size_kib_per_dispatch_raw": round(fetch[kname], 1),
        "write_size_kib_per_dispatch_raw": round(write[kname], 1),
        "calibration": {"copy_bytes": copy_bytes, "copy_kernel": ck,
                        "fetch_size_kib": round(fetch[ck], 1), "write_size_kib": round(write[ck], 1),
                        "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4)},
        "hbm_read_bytes_per_launch": int(rd), "hbm_write_bytes_per_launch": int(wr),
        "hbm_bytes_per_launch": int(rd + wr),
        "algorithmic_bytes_per_launch": conv_bytes(wk, conv.P, conv.Q, 1),
        "commands": commands, "dispatches_averaged": fcnt[kname],
    }
    out = traffic_file(key)
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    return out


def summarize_counters(key, dirs, commands, tag=""):
    """Average per-dispatch value of every counter collected for the conv
    kernel, over rocprofv3 --pmc runs of this script."""
    from convolution_forward_gemm_amd import workloads as wl
    acc, cnt, kname = {}, {}, None
    for d in dirs:
        rows = _csv_rows(_find(d, "counter_collection.csv"))
        calls = {}
        for r in rows:
            calls[r["Kernel_Name"]] = calls.get(r["Kernel_Name"], 0) + 1
        k = _conv_kernel(calls)
        kname = kname or k
        for r in rows:
            if r["Kernel_Name"] == k:
                acc[r["Counter_Name"]] = acc.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                cnt[r["Counter_Name"]] = cnt.get(r["Counter_Name"], 0) + 1
    lines = ["# conv kernel counters: " + wl.WORKLOADS[key].name, "",
             "Kernel: `%s`" % kname,
             "Kernel source hash (%s): %s" % (", ".join(os.path.basename(k) for k in KERNEL_SOURCES),
                                              kernel_source_hash()),
             "", "Commands (one rocprofv3 run per pass):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "| counter | per dispatch | dispatches |", "|---|---|---|"]
    for c in sorted(acc):
        lines.append("| %s | %.1f | %d |" % (c, acc[c] / cnt[c], cnt[c]))
    prefix = "conv_i8" if wl.WORKLOADS[key].dtype == "int8" else "conv_f32"
    out = os.path.join(PROFILES, "%s_%s%s_counters.md" % (prefix, key, tag))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


def _tag(args):
    return "" if args.config is None else "_cfg%d" % args.config


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU clock ramps up over tens of milliseconds of sustained load;
    # every run first spends at least --clock-ramp-ms of untimed launches of
    # the timed step (reported as clock_ramp_ms), whatever --warmup is.
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--clock-ramp-ms", type=float, default=60.0)
    ap.add_argument("--no-extras", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--workload", default="c3", help="headline workload key (c3 default)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed region, run a plain device copy of this many MiB "
                         "(three times) to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write profiles/conv_i8_<workload>_kernel_trace.txt from a rocprofv3 "
                         "--kernel-trace --stats output directory of this script, then exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/conv_i8_<workload>_traffic.json from rocprofv3 --pmc "
                         "FETCH_SIZE and WRITE_SIZE runs of this script with --calib-copy-mib, then exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="write profiles/conv_i8_<workload>_counters.md from rocprofv3 --pmc "
                         "output directories of this script, then exit")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize-*: the profiling command(s) to record")
    ap.add_argument("--config", type=int, default=None,
                    help="run another compiled configuration of the workload (for profiling "
                         "alternatives; summaries then carry a _cfg<N> suffix)")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(args.workload, args.summarize_counters, args.command, _tag(args)))
        return
    if args.summarize_trace or args.summarize_traffic:
        if args.summarize_trace:
            print(summarize_trace(args.workload, args.summarize_trace, " && ".join(args.command),
                                  _tag(args)))
        if args.summarize_traffic:
            print(summarize_traffic(args.workload, *args.summarize_traffic,
                                    args.calib_copy_mib or 256, args.command))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from convolution_forward_gemm_amd import binding as b
    from convolution_forward_gemm_amd import workloads as wl

    wk = wl.WORKLOADS[args.workload]
    conv, xd, wd, yd, host_inputs = setup(wk, torch, b)
    if args.config is not None:  # profiling another configuration; not the reported choice
        conv.set_config(args.config)
    stream = torch.cuda.current_stream().cuda_stream
    xp, wp, yp = xd.data_ptr(), wd.data_ptr(), yd.data_ptr()

    def step():
        conv.run_ptr(xp, wp, yp, wk.alpha, stream)

    torch.cuda.synchronize()
    ramp_ms, ramp_n = clock_ramp(torch, step, args.clock_ramp_ms)
    ms = time_device(torch, step, args.steps, args.warmup)
    ops = conv_ops(wk, conv.P, conv.Q)
    tops = ops / (ms * 1e-3) / 1e12

    traffic = committed_traffic(wk.key, conv.config)

    out = {
        "metric": METRIC,
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_ms": round(ramp_ms, 1),
        "clock_ramp_launches": ramp_n,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded uniform int8, resident in HBM)",
        "config": {"workload": wk.name, "N": wk.N, "C": wk.C, "H": wk.H, "W": wk.W,
                   "K": wk.K, "R": wk.R, "S": wk.S, "pad": list(wk.pad),
                   "stride": list(wk.stride), "dilation": list(wk.dil),
                   "alpha": wk.alpha, "layout": "NCxHWx<32> / CxRSKx<32>",
                   "kernel_config": conv.config, "pct_of_int8_peak": round(100 * tops / PEAK_INT8_TOPS, 2)},
        # achieved: algorithmic int8 ops of one launch / average launch time
        # (HIP events on the launch stream over the timed region)
        "roofline": {"bound": "mfma", "achieved": round(tops, 3), "peak": PEAK_INT8_TOPS,
                     "unit": "TOPS", "frac": round(tops / PEAK_INT8_TOPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": conv_bytes(wk, conv.P, conv.Q, 1),
                     "ops_per_launch": ops},
    }

    if not args.no_extras:
        extra = {}
        # smallest shape: microseconds per call
        w1 = wl.WORKLOADS["c1"]
        c1, x1, w1d, y1, _ = setup(w1, torch, b)
        lat = latency_suite(torch, c1, x1, w1d, y1, w1.alpha)
        lat["config"] = c1.config
        lat["GBps_device"] = round(conv_bytes(w1, c1.P, c1.Q, 1) / (lat["device_us_per_call"] * 1e-6) / 1e9, 3)
        extra["c1_smallest_us_per_call"] = lat
        out["us_per_call_smallest"] = lat["device_us_per_call"]
        w2 = wl.WORKLOADS["c2"]
        c2, x2, w2d, y2, _ = setup(w2, torch, b)
        lat2 = latency_suite(torch, c2, x2, w2d, y2, w2.alpha)
        lat2["config"] = c2.config
        lat2["GBps_device"] = round(conv_bytes(w2, c2.P, c2.Q, 1) / (lat2["device_us_per_call"] * 1e-6) / 1e9, 3)
        extra["c2_1x1_us_per_call"] = lat2
        # strided 3x3
        w4 = wl.WORKLOADS["c4"]
        c4, x4, w4d, y4, _ = setup(w4, torch, b)
        s4 = torch.cuda.current_stream().cuda_stream
        ms4 = time_device(torch, lambda: c4.run_ptr(x4.data_ptr(), w4d.data_ptr(), y4.data_ptr(), w4.alpha, s4), 2000, 3000)
        t4 = conv_ops(w4, c4.P, c4.Q) / (ms4 * 1e-3) / 1e12
        extra["c4_strided"] = {"ms": round(ms4, 6), "TOPS": round(t4, 3),
                               "pct_of_int8_peak": round(100 * t4 / PEAK_INT8_TOPS, 2), "config": c4.config,
                               "algorithmic_GBps": round(conv_bytes(w4, c4.P, c4.Q, 1) / (ms4 * 1e-3) / 1e9, 1)}
        tr4 = committed_traffic("c4", c4.config)
        if tr4 is not None:  # measured HBM bytes of one launch over this run's time
            extra["c4_strided"]["hbm_traffic_bytes"] = tr4
            extra["c4_strided"]["hbm_GBps"] = round(tr4 / (ms4 * 1e-3) / 1e9, 1)
        # per-output-channel scale and bias (conv2d_fprop_run_scaled) on the
        # headline workload
        gen = np.random.default_rng((2026, 31, 3))
        al = torch.from_numpy((wk.alpha * gen.uniform(0.5, 2.0, wk.K)).astype(np.float32)).cuda()
        bi = torch.from_numpy(gen.uniform(-3.0, 3.0, wk.K).astype(np.float32)).cuda()
        mss = time_device(torch, lambda: conv.run_scaled_ptr(xp, wp, yp, al.data_ptr(), bi.data_ptr(),
                                                             stream), 2000, 500)
        extra["c3_per_channel_scale_bias"] = {"ms": round(mss, 6),
                                              "TOPS": round(ops / (mss * 1e-3) / 1e12, 3)}
        # cold operands: rotate through enough copies of x, w, y that the
        # 256 MB Infinity Cache (and every L2) holds none of a call's operands
        # when it starts (more than twice the cache in total)
        extra["c3_cold"] = cold_run(torch, conv, xd, wd, yd, wk, ops)
        c1c = cold_run(torch, c1, x1, w1d, y1, w1, conv_ops(w1, c1.P, c1.Q))
        extra["c1_cold_us_per_call"] = c1c["us_per_call"]
        # transforms (GB/s, bytes read + written)
        xs = torch.from_numpy(host_inputs[0]).cuda()
        ilb = torch.empty((wk.N, wk.C // 32, wk.H, wk.W, 32), dtype=torch.int8, device="cuda")
        lt = b.lib.conv_nchw_to_nc32hw32_i8
        mst = time_device(torch, lambda: lt(xs.data_ptr(), ilb.data_ptr(), wk.N, wk.C, wk.H, wk.W, s4), 200, 20)
        extra["transform_nchw_to_nc32hw32_c3x"] = {"ms": round(mst, 6),
                                                   "GBps": round(2 * xs.numel() / (mst * 1e-3) / 1e9, 1)}
        del xs, ilb
        # one GPU's share under the sharding plan (design only here): the
        # 3x3 C256 workload split 8 ways over the batch (N = 4 per GPU), and
        # the dilated fp32 one split 8 ways over output rows (64 rows per GPU
        # read 72 input rows, halo included); configurations from the
        # selection model, not the per-shape table
        shard = {}
        for key, swk in (
                ("c3_batch_shard_n4", wl.Workload("c3n4", "", "int8", 4, 256, 28, 28, 256, 3, 3, (1, 1),
                                                  (1, 1), (1, 1), -128, 127, 2.0 ** -14, 2)),
                ("c5_row_shard_72x512", wl.Workload("c5h", "", "fp32", 8, 32, 72, 512, 64, 5, 9, (0, 4),
                                                    (1, 1), (2, 3), 0, 0, 1.0, 4))):
            cs, xs_, ws_, ys_, _ = setup(swk, torch, b)
            n_it = 2000 if swk.dtype == "int8" else 50
            mss_ = time_device(torch, lambda: cs.run_ptr(xs_.data_ptr(), ws_.data_ptr(), ys_.data_ptr(),
                                                         swk.alpha, s4), n_it, n_it // 2)
            tt = conv_ops(swk, cs.P, cs.Q) / (mss_ * 1e-3) / 1e12
            shard[key] = {"us": round(mss_ * 1e3, 3), "T_ops_per_s": round(tt, 3), "config": cs.config}
            del cs, xs_, ws_, ys_
        extra["one_gpu_share_of_sharded_workloads"] = shard
        # fp32 dilated
        w5 = wl.WORKLOADS["c5"]
        c5, x5, w5d, y5, _ = setup(w5, torch, b)
        ms5 = time_device(torch, lambda: c5.run_ptr(x5.data_ptr(), w5d.data_ptr(), y5.data_ptr(), 1.0, s4), 20, 15)
        t5 = conv_ops(w5, c5.P, c5.Q) / (ms5 * 1e-3) / 1e12
        extra["c5_fp32_dilated"] = {"ms": round(ms5, 4), "TFLOPS": round(t5, 3),
                                    "pct_of_fp32_peak": round(100 * t5 / PEAK_FP32_TFLOPS, 2),
                                    "config": c5.config}
        out["extra"] = extra

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = n
        del src, dst

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wk, *host_inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
