"""Fit the configuration-selection model from shape-grid sweeps.

`sweep.py --grid train|validate --out FILE` times every configuration that
runs each shape of a grid (one JSON line per shape and configuration).  This
script fits, per configuration, a small cost model of its measured time

    t = a + R * (b + c * W + d * L + e * C / 100 + f * Rf * Sf / 10) + g * G * W / 1000

    R = ceil(G / (256 * occ))   rounds of workgroups over the 256 CUs
    occ = min(occ_c, 160 KiB // lds, 2048 // threads)   workgroups per CU
    W = bm * bn * C * Rf * Sf / 1e6   multiply-adds of one tile (millions)
    L = C * Rf * Sf / 1e3             reduction length of one tile

The R terms are the busiest CU's rounds of tiles (a tile's fixed cost, its
work, its reduction steps, its channel chunks and taps); the G * W term is
the whole grid's work at the configuration's throughput, which the rounds
alone quantise too coarsely.  a..g >= 0 (non-negative least squares on
relative error) and the per-configuration occupancy occ_c (1..8) that fits
best.  G, bm, bn, lds and threads are those the library plans for the
shape.  desc_create evaluates the same model for every configuration that
plans and takes the least predicted time (shapes in the per-shape table keep
their entry).

    python -m convolution_forward_gemm_amd.fit_select \
        tuning/select_train.csv.gz tuning/select_validate.csv.gz

writes csrc/select_model.inc (the table compiled into the library) and
profiles/conv_config_model_fit.txt (fit quality: for each shape, the
measured time of the predicted choice over the best measured time).
"""
from __future__ import annotations

import argparse
import collections
import json
import math
import os

import numpy as np
from scipy.optimize import nnls

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OCC_CHOICES = (1, 2, 3, 4, 6, 8)


_CSV_FIELDS = ("dtype", "N", "C", "H", "W", "K", "R", "S", "ph", "pw", "sh", "sw", "dh", "dw",
               "config", "name", "bm", "bn", "grid", "lds", "threads", "us", "default")


def load(path):
    """Sweep records from the sweep's JSON lines or a packed .csv.gz."""
    if path.endswith(".csv.gz"):
        import csv
        import gzip
        out = []
        with gzip.open(path, "rt", newline="") as f:
            for row in csv.DictReader(f):
                sh = [row["dtype"]] + [int(row[k]) for k in _CSV_FIELDS[1:14]]
                out.append({"shape": sh, "config": int(row["config"]), "name": row["name"],
                            "bm": int(row["bm"]), "bn": int(row["bn"]), "grid": int(row["grid"]),
                            "lds": int(row["lds"]), "threads": int(row["threads"]),
                            "us": float(row["us"]), "default": row["default"] == "1"})
        return out
    with open(path) as f:
        return [json.loads(l) for l in f if l.strip()]


def pack(rows, path):
    """Write sweep records as a .csv.gz (the form kept beside this script)."""
    import csv
    import gzip
    with gzip.open(path, "wt", newline="") as f:
        w = csv.writer(f)
        w.writerow(_CSV_FIELDS)
        for r in rows:
            w.writerow(list(r["shape"]) + [r["config"], r["name"], r["bm"], r["bn"], r["grid"],
                                           r["lds"], r["threads"], r["us"], int(r["default"])])


def occ_eff(occ, lds, threads):
    lim = min(occ, 163840 // lds if lds > 0 else occ, max(1, 2048 // threads))
    return max(1, lim)


def features(r, occ):
    _, N, C, H, W, K, Rf, Sf = r["shape"][:8]
    R = math.ceil(r["grid"] / (256 * occ_eff(occ, r["lds"], r["threads"])))
    Wt = r["bm"] * r["bn"] * C * Rf * Sf / 1e6
    L = C * Rf * Sf / 1e3
    return np.array([1.0, R, R * Wt, R * L, R * C / 100, R * Rf * Sf / 10, r["grid"] * Wt / 1e3])


# With fewer shapes than coefficients a configuration gets the three-term
# model t = a + b * R + g * G * W (the other coefficients zero).
FULL_ROWS = 8
REDUCED = (0, 1, 6)


def fit_config(rows):
    """(occ, coefficients, relative rms) minimising the relative error."""
    t = np.array([r["us"] for r in rows])
    cols = list(range(7)) if len(rows) >= FULL_ROWS else list(REDUCED)
    best = None
    for occ in OCC_CHOICES:
        A = np.stack([features(r, occ) for r in rows]) / t[:, None]
        sub, _ = nnls(A[:, cols], np.ones(len(rows)))
        coef = np.zeros(A.shape[1])
        coef[cols] = sub
        res = float(np.sqrt(np.mean((A @ coef - 1.0) ** 2)))
        if best is None or res < best[2] - 1e-9:
            best = (occ, coef, res)
    return best


def predict(model, r):
    occ, coef = model
    return float(features(r, occ) @ coef)


def evaluate(models, rows):
    """Per shape: (shape, measured us of the predicted choice, best us,
    default us, predicted configuration name, fastest configuration name)."""
    by = collections.defaultdict(list)
    for r in rows:
        by[tuple(r["shape"])].append(r)
    out = []
    for sh, rs in by.items():
        cand = [r for r in rs if (r["shape"][0], r["name"]) in models]
        pick = min(cand, key=lambda r: (predict(models[(r["shape"][0], r["name"])], r), r["config"]))
        best = min(rs, key=lambda r: r["us"])
        dflt = [r for r in rs if r["default"]][0]
        out.append((sh, pick["us"], best["us"], dflt["us"], pick["name"], best["name"]))
    return out


def summary_lines(title, ev):
    lines = [title]
    for dt in ("int8", "fp32"):
        e = [x for x in ev if x[0][0] == dt]
        if not e:
            continue
        m = np.array([x[1] / x[2] for x in e])
        o = np.array([x[3] / x[2] for x in e])
        lines.append("  %-4s %3d shapes | model: mean %.3f median %.3f max %.2f, within 5%% of best %3.0f%%"
                     " | sweep-time default: mean %.3f median %.3f max %.2f, within 5%% %3.0f%%"
                     % (dt, len(e), m.mean(), np.median(m), m.max(), 100 * (m <= 1.05).mean(),
                        o.mean(), np.median(o), o.max(), 100 * (o <= 1.05).mean()))
    return lines


def _c_float(v):
    t = "%.7g" % v
    return (t if ("." in t or "e" in t) else t + ".0") + "f"


def write_table(models, path):
    lines = ["// Generated by convolution_forward_gemm_amd/fit_select.py from shape-grid",
             "// sweeps: per configuration, its workgroups per CU and the coefficients",
             "// {a, b, c, d, e, f, g} of its predicted time (select_time in api.hip).",
             "// {dtype, configuration name, occupancy, {a, b, c, d, e, f, g}}"]
    for (dt, name), (occ, coef) in sorted(models.items()):
        lines.append('{CONV_DTYPE_%s, "%s", %d, {%s}},'
                     % ("INT8" if dt == "int8" else "FP32", name, occ,
                        ", ".join(_c_float(v) for v in coef)))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("train")
    ap.add_argument("validate")
    ap.add_argument("--table", default=os.path.join(HERE, "csrc", "select_model.inc"))
    ap.add_argument("--summary", default=os.path.join(ROOT, "profiles", "conv_config_model_fit.txt"))
    ap.add_argument("--command", default="")
    ap.add_argument("--pack", nargs=2, metavar=("TRAIN_OUT", "VALIDATE_OUT"),
                    help="also store the inputs as .csv.gz files")
    a = ap.parse_args()
    train, val = load(a.train), load(a.validate)
    if a.pack:
        pack(train, a.pack[0])
        pack(val, a.pack[1])
    per = collections.defaultdict(list)
    for r in train:
        per[(r["shape"][0], r["name"])].append(r)
    models, fits = {}, []
    for key, rows in sorted(per.items()):
        if len(rows) < len(REDUCED):  # too few shapes even for the reduced model
            continue
        occ, coef, res = fit_config(rows)
        models[key] = (occ, coef)
        fits.append((key, len(rows), occ, res))
    write_table(models, a.table)
    # a validation shape that is also in the training grid is not held out
    seen = {tuple(r["shape"]) for r in train}
    held = [r for r in val if tuple(r["shape"]) not in seen]
    ev_t, ev_v = evaluate(models, train), evaluate(models, held)
    lines = ["Configuration-selection model: fit on %d shapes, checked on %d held-out shapes"
             % (len(seen), len({tuple(r['shape']) for r in held})),
             "command: " + a.command,
             "(per shape: measured time of the configuration the model predicts fastest, over the",
             " fastest measured; 'sweep-time default' is the configuration the library chose when",
             " the sweep ran: the previous fit's pick, except the 189 short-reduction int8",
             " training shapes added later, where it is this fit's pick before they were added)", ""]
    lines += summary_lines("training shapes:", ev_t) + [""]
    lines += summary_lines("held-out shapes:", ev_v) + [""]
    lines.append("held-out shapes, one by one (us: model's pick / fastest / sweep-time default):")
    for sh, mu, bu, du, pc, bc in ev_v:
        lines.append("  %-60s %9.2f %9.2f %9.2f  %s%s" % (sh, mu, bu, du, pc,
                                                         "" if pc == bc else " (fastest: %s)" % bc))
    lines += ["", "per-configuration fit (shapes, occupancy, relative rms error):"]
    for (dt, name), n, occ, res in fits:
        lines.append("  %-4s %-80s %4d %2d %6.3f" % (dt, name[:80], n, occ, res))
    with open(a.summary, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:16]))


if __name__ == "__main__":
    main()
