"""CPU checks of the configuration-selection model (no GPU: descriptor
planning only).

* The compiled table (csrc/select_model.inc) is what fit_select.py writes
  from the sweep data kept in tuning/ (regenerated here byte for byte).
* For every swept shape, desc_create picks the configuration whose predicted
  time, evaluated in Python from the same table and the library's own plans,
  is least (shapes in the per-shape table keep their entry).
* On the held-out shapes the model's picks stay within a few percent of the
  fastest measured configuration (a bad refit fails here).
"""
import os
import re

import numpy as np
import pytest

from convolution_forward_gemm_amd import binding as b
from convolution_forward_gemm_amd import fit_select as fs
from convolution_forward_gemm_amd import sweep
from convolution_forward_gemm_amd import workloads as wl

PKG = os.path.dirname(os.path.abspath(fs.__file__))
TUNING = os.path.join(PKG, "tuning")
TABLE = os.path.join(PKG, "csrc", "select_model.inc")


def _table():
    models = {}
    for line in open(TABLE):
        m = re.match(r'\{CONV_DTYPE_(\w+), "(\S+)", (\d+), \{([^}]*)\}\},', line)
        if m:
            dt = "int8" if m.group(1) == "INT8" else "fp32"
            coef = np.array([float(v.rstrip("f")) for v in m.group(4).split(",")])
            models[(dt, m.group(2))] = (int(m.group(3)), coef)
    return models


def _graded(sh):
    for wk in wl.WORKLOADS.values():
        if (wk.dtype, wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S) + tuple(wk.pad) + tuple(wk.stride) \
                + tuple(wk.dil) == tuple(sh):
            return True
    return False


def test_table_is_the_fit_of_the_kept_sweeps(tmp_path):
    out = tmp_path / "select_model.inc"
    summ = tmp_path / "fit.txt"
    import sys
    from unittest import mock
    argv = ["fit_select", os.path.join(TUNING, "select_train.csv.gz"),
            os.path.join(TUNING, "select_validate.csv.gz"), "--table", str(out), "--summary", str(summ)]
    with mock.patch.object(sys, "argv", argv):
        fs.main()
    assert out.read_text() == open(TABLE).read()


@pytest.mark.parametrize("kind", ["validate", "train"])
def test_library_pick_is_the_model_minimum(kind):
    models = _table()
    assert models, "empty selection table"
    shapes = sweep.grid_shapes(kind)
    if kind == "train":
        shapes = shapes[::5]  # a fifth of the training grid keeps this quick
    checked = 0
    for sh in shapes:
        if _graded(sh):
            continue
        dt, N, C, H, W, K, R, S, ph, pw, sth, stw, dh, dw = sh
        conv = b.Conv2dFprop(N, C, H, W, K, R, S, pad=(ph, pw), stride=(sth, stw), dil=(dh, dw),
                             dtype=dt)
        chosen = sweep._parse_config(conv.config)["name"]
        preds = []
        for i in range(b.num_configs(dt)):
            try:
                conv.set_config(i)
            except b.ConvError:
                continue
            r = sweep._parse_config(conv.config)
            r["shape"] = list(sh)
            if (dt, r["name"]) in models:
                preds.append((fs.predict(models[(dt, r["name"])], r), i, r["name"]))
        preds.sort()
        # the float32 table and double evaluation may order near-ties either way
        tied = [n for t, _, n in preds if t <= preds[0][0] * (1 + 1e-6)]
        assert chosen in tied, (sh, chosen, preds[:3])
        checked += 1
    assert checked > 20


def test_held_out_picks_are_close_to_the_fastest():
    models = _table()
    seen = {tuple(r["shape"]) for r in fs.load(os.path.join(TUNING, "select_train.csv.gz"))}
    held = [r for r in fs.load(os.path.join(TUNING, "select_validate.csv.gz"))
            if tuple(r["shape"]) not in seen]
    ev = fs.evaluate(models, held)
    for dt in ("int8", "fp32"):
        reg = np.array([x[1] / x[2] for x in ev if x[0][0] == dt])
        assert len(reg) >= 10
        assert reg.mean() < 1.06 and reg.max() < 1.3, (dt, reg.mean(), reg.max())
