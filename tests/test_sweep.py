"""CPU checks of the configuration sweep tool (no GPU: planning and the
trace summary only)."""
import csv
import os

import pytest

from convolution_forward_gemm_amd import binding as b
from convolution_forward_gemm_amd import sweep
from convolution_forward_gemm_amd import workloads as wl


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_applicable_lists_the_default(key):
    cfgs, default = sweep.applicable(b, wl.WORKLOADS[key])
    idx = [i for i, _ in cfgs]
    assert default in idx
    assert idx == sorted(set(idx))
    assert all(name.startswith("config=%d " % i) for i, name in cfgs)


def test_summarize_trace_maps_kernels_in_sweep_order(tmp_path):
    key = "c1"
    cfgs, default = sweep.applicable(b, wl.WORKLOADS[key])
    idx = [i for i, _ in cfgs]
    kname = {i: "convfprop::conv_fake_kernel_%d" % i for i in idx}
    # the sweep's dispatch order: warm-up (default), every configuration once
    # in index order, then rounds of each configuration
    seq = [default] * 5 + idx + [i for _ in range(2) for i in idx for _ in range(3)]
    dur = {i: 1000 + 10 * n for n, i in enumerate(idx)}
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        t = 0
        for i in seq:
            wr.writerow({"Kernel_Name": kname[i], "Start_Timestamp": t, "End_Timestamp": t + dur[i]})
            t += 5000
        # a layout transform is not a conv configuration
        wr.writerow({"Kernel_Name": "convfprop::nchw_to_nc32_kernel", "Start_Timestamp": t,
                     "End_Timestamp": t + 1})
    path = sweep.summarize_trace(key, str(tmp_path / "trace"), "cmd", str(tmp_path))
    lines = open(path).read().splitlines()
    rows = [l for l in lines if l[:1].isdigit()]
    assert len(rows) == len(idx)
    got = {int(r.split()[0]): float(r.split()[3]) for r in rows}
    assert got == {i: dur[i] / 1e3 for i in idx}
    chosen = [r for r in rows if r.endswith("<- chosen")]
    assert len(chosen) == 1 and int(chosen[0].split()[0]) == default


def test_shape_grids_are_fixed_and_disjoint():
    # the kept sweep data are keyed by these shapes: the grids must not drift,
    # and no held-out shape may appear in the training grid
    train, val = sweep.grid_shapes("train"), sweep.grid_shapes("validate")
    assert train == sweep.grid_shapes("train") and val == sweep.grid_shapes("validate")
    assert len(train) == 755 and len(val) == 46
    # the only shared shape: 3x3 C256 at N = 4, also one GPU's share of the
    # batch-sharded N = 32 workload (the fit summary leaves it out of the
    # held-out figures)
    assert set(train) & set(val) == {("int8", 4, 256, 28, 28, 256, 3, 3, 1, 1, 1, 1, 1, 1)}
    for sh in train + val:
        dt, N, C, H, W, K, R, S, ph, pw, sth, stw, dh, dw = sh
        conv = b.Conv2dFprop(N, C, H, W, K, R, S, pad=(ph, pw), stride=(sth, stw), dil=(dh, dw),
                             dtype=dt)
        assert conv.P >= 1 and conv.Q >= 1


def test_kept_sweeps_cover_the_grids():
    import os
    from convolution_forward_gemm_amd import fit_select as fs
    tuning = os.path.join(os.path.dirname(sweep.__file__), "tuning")
    for kind in ("train", "validate"):
        rows = fs.load(os.path.join(tuning, "select_%s.csv.gz" % kind))
        assert {tuple(r["shape"]) for r in rows} == set(sweep.grid_shapes(kind))
        # exactly one library default per shape
        per = {}
        for r in rows:
            per[tuple(r["shape"])] = per.get(tuple(r["shape"]), 0) + int(r["default"])
        assert set(per.values()) == {1}
