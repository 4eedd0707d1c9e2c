"""Configuration sweep for one conv2d fprop shape.

Runs every compiled configuration that can run the shape, back to back on
one stream, and reports each one's device time; the configuration the
library picks by itself for the shape is marked.  This is the evidence
behind the per-shape table in api.hip (kShapeTable).

    python -m convolution_forward_gemm_amd.sweep --workload c3

Under `rocprofv3 --kernel-trace` the same run gives each configuration's
dispatch durations; `--summarize-trace DIR` turns that output into a table
under profiles/ (each configuration runs a kernel instantiation of its own,
and the sweep runs them in configuration order, so a kernel name maps to the
configuration that first dispatched it).  With `--graph` each configuration
is also timed per call in HIP-graph replay (20 captured back-to-back calls),
the criterion for the launch-latency-bound shapes; `--sweep-log FILE` adds
that table, from the sweep's own JSON line, to the summary.

Inputs are the seeded synthetic operands of the workload, already resident
in device memory; the GPU first runs the default configuration long enough
to reach its steady clock.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _ops(wk, P, Q):
    return 2 * wk.N * wk.K * P * Q * wk.C * wk.R * wk.S


def _new_conv(b, wk):
    return b.Conv2dFprop(wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S, pad=wk.pad,
                         stride=wk.stride, dil=wk.dil, dtype=wk.dtype)


def applicable(b, wk):
    """[(index, config string)] of the configurations that run the shape, and
    the index the library chooses by itself."""
    conv = _new_conv(b, wk)
    default = int(conv.config.split()[0].split("=")[1])
    out = []
    for i in range(b.num_configs(wk.dtype)):
        try:
            conv.set_config(i)
        except b.ConvError as e:
            if e.status != b.CONV_ERR_UNSUPPORTED:
                raise
            continue
        out.append((i, conv.config))
    return out, default


def _graph_us(torch, conv, xp, wp, yp, alpha, reps=30):
    """Median microseconds per call over replays of 20 captured calls."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            conv.run_ptr(xp, wp, yp, alpha, s.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(20):
            conv.run_ptr(xp, wp, yp, alpha, s.cuda_stream)
    t = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3 / 200)
    t.sort()
    return t[len(t) // 2]


def run_sweep(key, calls, warmup, rounds, graph=False):
    import torch
    from . import binding as b
    from . import workloads as wl

    wk = wl.WORKLOADS[key]
    cfgs, default = applicable(b, wk)
    x, w = wl.make_inputs(wk)
    if wk.dtype == "int8":
        xd = b.nchw_to_nc32hw32(torch.from_numpy(x).cuda())
        wd = b.kcrs_to_c32rsk32(torch.from_numpy(w).cuda())
        ydt = torch.int8
    else:
        xd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
        ydt = torch.float32
    convs = []
    for i, _ in cfgs:
        c = _new_conv(b, wk)
        c.set_config(i)
        convs.append(c)
    y = torch.empty(convs[0].y_shape, dtype=ydt, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    xp, wp, yp = xd.data_ptr(), wd.data_ptr(), y.data_ptr()
    # steady clock first (default configuration), then every configuration
    # once in index order (this fixes the kernel-name order in a trace)
    dflt = convs[[i for i, _ in cfgs].index(default)]
    for _ in range(warmup):
        dflt.run_ptr(xp, wp, yp, wk.alpha, s)
    for c in convs:
        c.run_ptr(xp, wp, yp, wk.alpha, s)
    torch.cuda.synchronize()
    times = {i: [] for i, _ in cfgs}
    for _ in range(rounds):
        for (i, _), c in zip(cfgs, convs):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(calls):
                c.run_ptr(xp, wp, yp, wk.alpha, s)
            e1.record()
            torch.cuda.synchronize()
            times[i].append(e0.elapsed_time(e1) * 1e3 / calls)
    gus = {}
    if graph:
        for (i, _), c in zip(cfgs, convs):
            gus[i] = _graph_us(torch, c, xp, wp, yp, wk.alpha)
    ops = _ops(wk, convs[0].P, convs[0].Q)
    rows = []
    for i, cfg in cfgs:
        t = sorted(times[i])
        med = t[len(t) // 2]
        rows.append({"config": i, "name": cfg.split()[1], "us": round(med, 3),
                     "tops": round(ops / med / 1e6, 1), "default": i == default})
        if graph:
            rows[-1]["graph_us"] = round(gus[i], 3)
    return {"workload": key, "name": wk.name, "calls": calls, "rounds": rounds,
            "warmup": warmup, "rows": rows}


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, d))
    return hits[0]


def summarize_trace(key, trace_dir, command, out_dir, sweep_log=None):
    """profiles/conv_config_sweep_<key>.txt from a rocprofv3 --kernel-trace
    run of this sweep (and, given its log, the graph-replay table)."""
    from . import binding as b
    from . import workloads as wl

    wk = wl.WORKLOADS[key]
    cfgs, default = applicable(b, wk)
    with open(_find(trace_dir, "kernel_trace.csv")) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    conv_rows = [r for r in rows if "conv_" in r["Kernel_Name"] and "_to_" not in r["Kernel_Name"]]
    durs, order = {}, []
    for r in conv_rows:
        k = r["Kernel_Name"]
        durs.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        if k not in order:
            order.append(k)
    # the warm-up runs the default configuration first; then every
    # configuration once in index order
    first = order[0]
    seq = [k for k in order if k != first]
    idx = [i for i, _ in cfgs]
    mapping = {}
    pos = idx.index(default)
    rest = idx[:pos] + idx[pos + 1:]
    if len(seq) != len(rest):
        raise ValueError("%d kernels for %d configurations: a kernel runs two of them"
                         % (len(seq) + 1, len(idx)))
    mapping[first] = default
    for k, i in zip(seq, rest):
        mapping[k] = i
    conv = _new_conv(b, wk)
    ops = _ops(wk, conv.P, conv.Q)
    cname = dict(cfgs)
    lines = ["rocprofv3 kernel-trace sweep of every configuration that runs: " + wk.name,
             "command: " + command,
             "(each configuration's dispatch durations; the warm-up dispatches of the "
             "default configuration are excluded)", "",
             "%-4s %-92s %6s %10s %10s %9s" % ("cfg", "configuration", "calls", "avg_us", "min_us", "TOPS")]
    res = []
    for k, i in mapping.items():
        d = durs[k]
        if i == default:
            d = d[-(len(durs[seq[0]]) if seq else len(d)):]  # drop the warm-up
        avg = sum(d) / len(d) / 1e3
        res.append((avg, i, len(d), min(d) / 1e3))
    for avg, i, n, mn in sorted(res):
        unit = ops / avg / 1e6
        lines.append("%-4d %-92s %6d %10.2f %10.2f %9.1f%s" % (
            i, cname[i].split()[1][:92], n, avg, mn, unit, "  <- chosen" if i == default else ""))
    best = min(res)
    tail = ["", "chosen configuration %d; fastest by trace average: %d (%.2f us)" % (default, best[1], best[0])]
    if sweep_log:
        with open(sweep_log) as f:
            js = [json.loads(l) for l in f if l.startswith("{")][-1]
        g = sorted((r["graph_us"], r["config"]) for r in js["rows"] if "graph_us" in r)
        if g:
            lines += ["", "graph replay (20 captured back-to-back calls, same run), us per call:",
                      "%-4s %-92s %10s" % ("cfg", "configuration", "us/call")]
            for us, i in g:
                lines.append("%-4d %-92s %10.3f%s" % (i, cname[i].split()[1][:92], us,
                                                       "  <- chosen" if i == default else ""))
            tail.append("fastest per call in graph replay: %d (%.3f us)" % (g[0][1], g[0][0]))
    lines += tail
    path = os.path.join(out_dir, "conv_config_sweep_%s.txt" % key)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


# ---------------------------------------------------------------------------
# Shape grids for the configuration-selection model (fit_select.py): every
# configuration that runs each shape, timed back to back on resident
# synthetic operands.  "train" fits the model, "validate" (held-out shapes,
# seeded random plus the per-GPU shares of the sharding plan) checks it.
# A shape is (dtype, N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw).
# ---------------------------------------------------------------------------
_FILTERS_I8 = ((1, 1, 0, 0, 1, 1, 1, 1), (3, 3, 1, 1, 1, 1, 1, 1), (3, 3, 1, 1, 2, 2, 1, 1),
               (5, 5, 2, 2, 1, 1, 1, 1), (3, 3, 2, 2, 1, 1, 2, 2), (7, 7, 3, 3, 2, 2, 1, 1))
_FILTERS_F32 = ((3, 3, 1, 1, 1, 1, 1, 1), (5, 9, 2, 4, 1, 1, 2, 3), (1, 1, 0, 0, 1, 1, 1, 1),
                (5, 5, 2, 2, 2, 2, 1, 1))


def _out_dim(x, pad, dil, k, st):
    return (x + 2 * pad - dil * (k - 1) - 1) // st + 1


def _shape_ok(sh, max_elems=1 << 26, max_ops=2.5e11):
    dt, N, C, H, W, K, R, S, ph, pw, sth, stw, dh, dw = sh
    P, Q = _out_dim(H, ph, dh, R, sth), _out_dim(W, pw, dw, S, stw)
    if P < 1 or Q < 1:
        return False
    ops = 2.0 * N * K * P * Q * C * R * S
    return N * C * H * W <= max_elems and N * K * P * Q <= max_elems and ops <= max_ops


def grid_shapes(kind):
    import numpy as np
    out = []
    if kind == "train":
        for N in (1, 4, 16, 64):
            for C, K in ((64, 64), (128, 128), (256, 256), (512, 512), (64, 256), (256, 64)):
                for H in (7, 14, 28, 56):
                    for R, S, ph, pw, sh, sw, dh, dw in _FILTERS_I8[:3]:
                        out.append(("int8", N, C, H, H, K, R, S, ph, pw, sh, sw, dh, dw))
        for N in (2, 32):
            for C, K in ((96, 160), (320, 192), (32, 448)):
                for H in (9, 20, 41):
                    for R, S, ph, pw, sh, sw, dh, dw in _FILTERS_I8[3:]:
                        out.append(("int8", N, C, H, H, K, R, S, ph, pw, sh, sw, dh, dw))
        for N in (1, 8):
            for C in (3, 32, 64):
                for K in (32, 64, 128):
                    for H, W in ((64, 64), (256, 256), (128, 200)):
                        for R, S, ph, pw, sh, sw, dh, dw in _FILTERS_F32:
                            out.append(("fp32", N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw))
        # short reductions (C/32 * R * S from 3 to 27 taps): the tiny
        # kernels' domain, one compiled configuration per tap count
        for N in (4, 16, 48):
            for K in (32, 160, 320):
                for H, W in ((10, 10), (16, 40), (28, 28)):
                    for C, f in ((32, 1), (32, 3), (96, 0), (96, 1), (192, 0), (288, 0), (384, 0)):
                        R, S, ph, pw, sh, sw, dh, dw = _FILTERS_I8[f]
                        out.append(("int8", N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw))
        # a network's first layer: 7x7 stride 2 on three channels
        for N in (1, 8, 32):
            for H in (112, 224):
                for K in (32, 64):
                    out.append(("fp32", N, 3, H, H, K, 7, 7, 3, 3, 2, 2, 1, 1))
    elif kind == "validate":
        out += [("int8", 4, 256, 28, 28, 256, 3, 3, 1, 1, 1, 1, 1, 1),    # 3x3 C256 share, N/8
                ("int8", 4, 128, 56, 56, 256, 3, 3, 1, 1, 2, 2, 1, 1),    # stride-2 share, N/8
                ("fp32", 8, 32, 72, 512, 64, 5, 9, 0, 4, 1, 1, 2, 3)]     # dilated 5x9 share, H/8
        rng = np.random.default_rng((2026, 77))
        while len(out) < 3 + 30:
            f = _FILTERS_I8[rng.integers(len(_FILTERS_I8))]
            H = int(rng.integers(5, 61))
            sh = ("int8", int(rng.integers(1, 49)), 32 * int(rng.integers(1, 17)), H,
                  int(rng.choice([H, rng.integers(5, 61)])), 32 * int(rng.integers(1, 17))) + f
            if _shape_ok(sh):
                out.append(sh)
        while len(out) < 3 + 30 + 10:
            f = _FILTERS_F32[rng.integers(len(_FILTERS_F32))]
            H = int(rng.integers(16, 300))
            sh = ("fp32", int(rng.integers(1, 9)), int(rng.integers(1, 65)), H,
                  int(rng.integers(16, 300)), 16 * int(rng.integers(1, 9))) + f
            if _shape_ok(sh):
                out.append(sh)
        # three-channel first layers (the tiny fp32 kernels' domain)
        out += [("fp32", 2, 3, 96, 150, 48, 3, 3, 1, 1, 1, 1, 1, 1),
                ("fp32", 4, 3, 160, 160, 64, 7, 7, 3, 3, 2, 2, 1, 1),
                ("fp32", 1, 3, 300, 200, 32, 5, 5, 2, 2, 1, 1, 1, 1)]
    else:
        raise ValueError(kind)
    return [sh for sh in out if _shape_ok(sh)]


def _parse_config(text):
    import re
    m = re.match(r"config=(\d+) (\S+) tile=(\d+)ch x (\d+)px grid=(\d+) lds=(\d+) threads=(\d+)", text)
    i, name, bm, bn, grid, lds, thr = m.groups()
    return {"config": int(i), "name": name, "bm": int(bm), "bn": int(bn), "grid": int(grid),
            "lds": int(lds), "threads": int(thr)}


def _median_us(torch, fn, target_us=300.0, reps=3):
    def run(calls):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(calls):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / calls
    t = run(2)
    calls = int(min(200, max(3, target_us / max(t, 1e-3))))
    ts = sorted(run(calls) for _ in range(reps))
    return ts[len(ts) // 2]


def run_shape_grid(kind, out_path, only=None, skip_known=None):
    """Time every configuration that runs each shape of the grid (or only the
    named ones); one JSON line per (shape, configuration) appended to
    out_path."""
    import torch
    from . import binding as b

    shapes = grid_shapes(kind)
    if skip_known:  # only the shapes a kept sweep does not hold yet
        from .fit_select import load
        known = {tuple(r["shape"]) for r in load(skip_known)}
        shapes = [sh for sh in shapes if tuple(sh) not in known]
    s = torch.cuda.current_stream().cuda_stream
    # steady clock first: ~0.1 s of back-to-back work
    wc = b.Conv2dFprop(32, 256, 28, 28, 256, 3, 3, pad=1)
    xw = torch.zeros(wc.x_shape, dtype=torch.int8, device="cuda")
    ww = torch.zeros(wc.w_shape, dtype=torch.int8, device="cuda")
    yw = torch.empty(wc.y_shape, dtype=torch.int8, device="cuda")
    for _ in range(6000):
        wc.run_ptr(xw.data_ptr(), ww.data_ptr(), yw.data_ptr(), 1.0, s)
    torch.cuda.synchronize()
    del xw, ww, yw
    gen = torch.Generator(device="cuda")
    with open(out_path, "a") as f:
        for si, sh in enumerate(shapes):
            dt, N, C, H, W, K, R, S, ph, pw, sth, stw, dh, dw = sh
            conv = b.Conv2dFprop(N, C, H, W, K, R, S, pad=(ph, pw), stride=(sth, stw), dil=(dh, dw),
                                 dtype=dt)
            default = _parse_config(conv.config)["config"]
            gen.manual_seed(si)
            if dt == "int8":
                x = torch.randint(-128, 128, conv.x_shape, dtype=torch.int8, device="cuda", generator=gen)
                w = torch.randint(-128, 128, conv.w_shape, dtype=torch.int8, device="cuda", generator=gen)
                y = torch.empty(conv.y_shape, dtype=torch.int8, device="cuda")
                alpha = 2.0 ** -14
            else:
                x = torch.randn(conv.x_shape, device="cuda", generator=gen)
                w = torch.randn(conv.w_shape, device="cuda", generator=gen) / (C * R * S) ** 0.5
                y = torch.empty(conv.y_shape, device="cuda")
                alpha = 1.0
            xp, wp, yp = x.data_ptr(), w.data_ptr(), y.data_ptr()
            n = 0
            for i in range(b.num_configs(dt)):
                try:
                    conv.set_config(i)
                except b.ConvError as e:
                    if e.status != b.CONV_ERR_UNSUPPORTED:
                        raise
                    continue
                if only and _parse_config(conv.config)["name"] not in only:
                    continue
                us = _median_us(torch, lambda: conv.run_ptr(xp, wp, yp, alpha, s))
                rec = {"kind": kind, "shape": list(sh)}
                rec.update(_parse_config(conv.config))
                rec["us"] = round(us, 3)
                rec["default"] = i == default
                f.write(json.dumps(rec) + "\n")
                n += 1
            f.flush()
            print("shape %d/%d %s: %d configurations" % (si + 1, len(shapes), sh, n), flush=True)
            del x, w, y, conv


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--calls", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--graph", action="store_true", help="also time each configuration in graph replay")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--sweep-log", metavar="FILE", help="with --summarize-trace: the sweep's output")
    ap.add_argument("--command", default="")
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--grid", choices=["train", "validate"], help="time a shape grid (model fit)")
    ap.add_argument("--out", help="with --grid: JSON-lines output file")
    ap.add_argument("--only", help="with --grid: comma-separated configuration names to time")
    ap.add_argument("--skip-known", metavar="CSV_GZ",
                    help="with --grid: skip the shapes this kept sweep already holds")
    a = ap.parse_args()
    if a.grid:
        run_shape_grid(a.grid, a.out, set(a.only.split(",")) if a.only else None, a.skip_known)
        return
    if a.summarize_trace:
        print(summarize_trace(a.workload, a.summarize_trace, a.command, a.out_dir, a.sweep_log))
        return
    res = run_sweep(a.workload, a.calls, a.warmup, a.rounds, a.graph)
    for r in sorted(res["rows"], key=lambda r: r["us"]):
        print("%3d %-90s %9.2f us %8.1f %s" % (r["config"], r["name"], r["us"], r["tops"],
                                               "<- chosen" if r["default"] else ""), flush=True)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    if __package__ in (None, ""):
        sys.path.insert(0, ROOT)
        __package__ = "convolution_forward_gemm_amd"
    main()
