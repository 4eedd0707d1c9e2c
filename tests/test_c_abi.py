"""The C ABI from plain C: tests/c/abi_from_c.c is compiled with gcc against
include/convfprop.h and the built library (and, for its GPU run, linked with
the oracle's C source), with no Python or C++ in between.

CPU: the entry points that need no GPU (descriptor creation, queries,
argument errors).  GPU: an int8 and an fp32 convolution run through the HIP
runtime's C API, compared with the oracle inside the program.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_from_c.c")
LIBDIR = os.path.join(ROOT, "convolution_forward_gemm_amd")
ROCM = "/opt/rocm"


def _build(tmp):
    exe = os.path.join(str(tmp), "abi_from_c")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Werror", "-ffp-contract=off", "-fopenmp",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), SRC, os.path.join(ROOT, "oracle", "conv_oracle.c"),
           "-o", exe, "-L", LIBDIR, "-lconvfprop", "-Wl,-rpath," + LIBDIR,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def _run(exe, *args):
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "all ok" in r.stdout
    return r.stdout


def test_c_program_host_entry_points(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libconvfprop.so")):
        pytest.skip("library not built")
    out = _run(_build(tmp_path))
    assert "ok desc_create int8 3x3" in out and "ok status strings" in out


@pytest.mark.gpu
def test_c_program_runs_convolutions(tmp_path):
    print("CASE C ABI program, int8 and fp32 runs", flush=True)
    out = _run(_build(tmp_path), "run")
    assert "ok int8 output equals the oracle, byte for byte" in out
    assert "ok fp32 output equals the oracle exactly on integer-valued operands" in out
