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
