"""Build libconvfprop.so (gfx950) in-tree with hipcc.

Run as ``python -m convolution_forward_gemm_amd.build``.  The library is
always rebuilt from source when ``build()`` is called.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libconvfprop.so")
PEAK_PROBE = os.path.join(PKG, "peak_probe")
SOURCES = ["api.hip", "conv_i8.hip", "conv_i8_halo.hip", "conv_i8_small.hip", "conv_f32.hip",
           "conv_f32_halo.hip", "transforms.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # No contraction of separate fp32 operations into FMAs: the int8
    # epilogue must be exactly one multiply followed by rint.
    "-ffp-contract=off",
    # Keep the compiler from forming packed fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build_peak_probe(verbose: bool = False) -> str:
    """The throughput-ceiling probe (an executable, not part of the library)."""
    tmp = PEAK_PROBE + ".tmp%d" % os.getpid()
    flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    _run([HIPCC, *flags, os.path.join(CSRC, "peak_probe.hip"), "-o", tmp], verbose)
    os.replace(tmp, PEAK_PROBE)
    return PEAK_PROBE


def device_asm(source: str, verbose: bool = False) -> str:
    """gfx950 assembly text of one source under the library's flags."""
    import tempfile
    flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "dev.s")
        _run([HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, source), "-o", out],
             verbose)
        with open(out) as f:
            return f.read()


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link the library."""
    import concurrent.futures
    import tempfile
    cflags = [f for f in FLAGS if f != "-shared"]
    tmp = LIB + ".tmp%d" % os.getpid()
    with tempfile.TemporaryDirectory() as d:
        def compile_one(src):
            obj = os.path.join(d, src + ".o")
            _run([HIPCC, *cflags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            return obj
        workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """The library with its host code built under AddressSanitizer and
    UndefinedBehaviorSanitizer (descriptor creation, planning, the selection
    model, argument checks, launchers); the gfx950 device code is built as
    usual, unsanitized.  The sanitizer runtime is the shared one of the ROCm
    clang, so a test program built by that clang with the same flags shares
    it.  Written to `out`; the in-tree library is not touched."""
    import concurrent.futures
    import tempfile
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-shared-libsan"]
    cflags = [f for f in FLAGS if f != "-shared"] + ["-O1", "-g"] + san
    with tempfile.TemporaryDirectory() as d:
        def compile_one(src):
            obj = os.path.join(d, src + ".o")
            _run([HIPCC, *cflags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            return obj
        workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, *objs, "-o", out],
             verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_peak_probe(verbose=True))
