"""GPU checks of the graph-capture entry points (conv2d_fprop_graph_create /
_launch / _destroy): every replay of a captured graph writes the bytes of an
eager run (int8) or equal floats (fp32, the same kernel on the same inputs),
with the output poisoned and eager work and synchronisation between replays.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from convolution_forward_gemm_amd import workloads as wl
from test_gpu_parity import _announce, _b, _dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _operands(b, wk):
    x, w = wl.make_inputs(wk)
    if wk.dtype == "int8":
        return b.nchw_to_nc32hw32(_dev(x)), b.kcrs_to_c32rsk32(_dev(w))
    return _dev(x), _dev(w)


def _conv(b, wk):
    return b.Conv2dFprop(wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S, pad=wk.pad, stride=wk.stride,
                         dil=wk.dil, dtype=wk.dtype)


@pytest.mark.parametrize("key,calls", [("c1", 1), ("c1", 7), ("c3", 3), ("c4", 2)])
def test_graph_replays_match_eager(key, calls):
    b = _b()
    wk = wl.WORKLOADS[key]
    conv = _conv(b, wk)
    xd, wd = _operands(b, wk)
    ref = conv.run(xd, wd, alpha=wk.alpha)
    torch.cuda.synchronize()
    ref = ref.cpu()
    y = torch.empty(conv.y_shape, dtype=ref.dtype, device="cuda")
    poison = 77 if wk.dtype == "int8" else float("nan")
    _announce("graph", key, "calls", calls)
    g = b.ConvGraph(conv, xd.data_ptr(), wd.data_ptr(), y.data_ptr(), wk.alpha, calls)
    s = torch.cuda.current_stream().cuda_stream
    for rep in range(3):
        y.fill_(poison)
        other = conv.run(xd, wd, alpha=wk.alpha)  # eager work between replays
        torch.cuda.synchronize()
        g.launch(s)
        torch.cuda.synchronize()
        assert torch.equal(y.cpu(), ref), rep
        assert torch.equal(other.cpu(), ref), rep
    del g


def test_graph_small_fp32_matches_eager():
    b = _b()
    N, C, H, W, K, R, S = 2, 5, 13, 11, 40, 3, 3
    x, w = wl.make_custom("fp32", N, C, H, W, K, R, S, seed=11)
    conv = b.Conv2dFprop(N, C, H, W, K, R, S, pad=(1, 1), dtype="fp32")
    xd, wd = _dev(x), _dev(w)
    ref = conv.run(xd, wd, alpha=0.5).cpu()
    y = torch.full(conv.y_shape, float("nan"), device="cuda")
    _announce("graph fp32 small")
    g = b.ConvGraph(conv, xd.data_ptr(), wd.data_ptr(), y.data_ptr(), 0.5, 4)
    for rep in range(2):
        y.fill_(float("nan"))
        g.launch(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(y.cpu(), ref), rep


def test_graph_outlives_descriptor_and_inputs_are_read_at_replay():
    # the captured kernels hold copies of the problem constants, so the graph
    # runs after the descriptor is destroyed; operands are read at replay time
    b = _b()
    wk = wl.WORKLOADS["c1"]
    conv = _conv(b, wk)
    xd, wd = _operands(b, wk)
    y = torch.empty(conv.y_shape, dtype=torch.int8, device="cuda")
    _announce("graph outlives descriptor")
    g = b.ConvGraph(conv, xd.data_ptr(), wd.data_ptr(), y.data_ptr(), wk.alpha, 2)
    x2, _ = wl.make_custom("int8", wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S, seed=5)
    ref2 = conv.run(b.nchw_to_nc32hw32(_dev(x2)), wd, alpha=wk.alpha)
    torch.cuda.synchronize()
    ref2 = ref2.cpu()
    g._conv = None
    del conv
    xd.copy_(b.nchw_to_nc32hw32(_dev(x2)))
    torch.cuda.synchronize()
    g.launch(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), ref2)


FIRST_IN_CAPTURE = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from convolution_forward_gemm_amd import binding as b, workloads as wl
wk = wl.WORKLOADS["c3"]
conv = b.Conv2dFprop(wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S, pad=wk.pad)
x, w = wl.make_inputs(wk)
xd = b.nchw_to_nc32hw32(torch.from_numpy(x).cuda())
wd = b.kcrs_to_c32rsk32(torch.from_numpy(w).cuda())
y = torch.empty(conv.y_shape, dtype=torch.int8, device="cuda")
torch.cuda.synchronize()
g = b.ConvGraph(conv, xd.data_ptr(), wd.data_ptr(), y.data_ptr(), wk.alpha, 2)  # first launch
g.launch(torch.cuda.current_stream().cuda_stream)
ref = conv.run(xd, wd, alpha=wk.alpha)
torch.cuda.synchronize()
print("EQUAL", bool(torch.equal(y.cpu(), ref.cpu())), flush=True)
"""


def test_graph_captures_a_kernel_never_launched_before():
    # in a fresh process the kernel's first launch (and its one-time
    # attribute set-up) happens inside the capture
    _announce("graph first launch in capture (child process)")
    r = subprocess.run([sys.executable, "-c", FIRST_IN_CAPTURE, ROOT], capture_output=True,
                       text=True, timeout=100)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "EQUAL True" in r.stdout, r.stdout[-2000:]
