"""CPU oracle for 2D convolution forward (fprop) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library
(``convolution_forward_gemm_amd``) never imports it and it imports nothing from
the GPU library: the two share no code.  The only module both sides use is the
seeded input generator ``convolution_forward_gemm_amd.workloads``, which holds
no convolution arithmetic.

The arithmetic lives in ``conv_oracle.c`` (plain nested loops, built with gcc);
this module marshals numpy arrays into it.  What each function computes, and
the pages it follows, is stated in that file:

* the output-size rule and the zero-padded, dilated, strided cross-correlation
  come from the first turn of the "Kimi-K2.6 l1_p80" POPCORNBENCH transcript;
* the int8 operands, int32 accumulator, fp32 alpha-only scaling and int8 clamp,
  and the NCxHWx<32> / CxRSKx<32> layouts, come from the "CUTLASS Kernel
  Configuration" section of CUTLASS issue 2996 ("How to optimize cutlass int8
  fprop2d kernel with NCxHWx interleaved layout").

Readings where the pages are silent (rounding mode, epilogue order, the memory
order behind the layout names) are listed in the design notes and stated in
``conv_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
             "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = False) -> str:
    """Compile ``conv_oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load(path=None):
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(path or build())
        i32, i64, p = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        conv_args = [i32] * 13 + [i32]  # N C H W K R S ph pw sh sw dh dw nthreads
        lib.oracle_output_dim.argtypes = [i32] * 5
        lib.oracle_output_dim.restype = i32
        lib.oracle_conv2d_i8_acc.argtypes = [p, p, p] + conv_args
        lib.oracle_conv2d_i8_acc.restype = i32
        lib.oracle_conv2d_i8_points.argtypes = [p, p, p, i64, p] + conv_args
        lib.oracle_conv2d_i8_points.restype = i32
        lib.oracle_epilogue_i8.argtypes = [p, p, i64, ctypes.c_float]
        lib.oracle_epilogue_i8.restype = i32
        lib.oracle_epilogue_i8_per_channel.argtypes = [p, p, i32, i32, i64, p, p]
        lib.oracle_epilogue_i8_per_channel.restype = i32
        lib.oracle_epilogue_f32_per_channel.argtypes = [p, p, i32, i32, i64, p, p]
        lib.oracle_epilogue_f32_per_channel.restype = None
        lib.oracle_conv2d_f32_acc.argtypes = [p, p, p] + conv_args
        lib.oracle_conv2d_f32_acc.restype = i32
        lib.oracle_conv2d_f32_points.argtypes = [p, p, p, i64, p] + conv_args
        lib.oracle_conv2d_f32_points.restype = i32
        lib.oracle_epilogue_f32.argtypes = [p, p, i64, ctypes.c_float]
        lib.oracle_epilogue_f32.restype = None
        for name in ("oracle_nchw_to_nc32hw32", "oracle_nc32hw32_to_nchw",
                     "oracle_kcrs_to_c32rsk32", "oracle_c32rsk32_to_kcrs"):
            getattr(lib, name).argtypes = [p, p, i32, i32, i32, i32]
            getattr(lib, name).restype = i32
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i32
        _lib = lib
    return _lib


def _swap_library(path):
    """Bind this module to another build of conv_oracle.c; returns the old
    handle for ``_restore_library``.  Used only by the mutation tests, which
    plant a mistake in a copy of the source and check that the pins fail."""
    global _lib
    prev = _lib
    _lib = None
    _load(path)
    return prev


def _restore_library(prev):
    global _lib
    _lib = prev


class OracleError(RuntimeError):
    pass


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _pair(v):
    return (int(v), int(v)) if np.isscalar(v) else (int(v[0]), int(v[1]))


def output_dim(in_size: int, pad: int, dil: int, k: int, stride: int) -> int:
    """floor((in + 2*pad - dil*(k-1) - 1) / stride) + 1, or 0 if none fits."""
    return _load().oracle_output_dim(in_size, pad, dil, k, stride)


def output_hw(H, W, R, S, pad=0, stride=1, dil=1):
    ph, pw = _pair(pad)
    sh, sw = _pair(stride)
    dh, dw = _pair(dil)
    return output_dim(H, ph, dh, R, sh), output_dim(W, pw, dw, S, sw)


def _conv_args(x, w, pad, stride, dil):
    N, C, H, W = x.shape
    K, Cw, R, S = w.shape
    if Cw != C:
        raise OracleError("channel mismatch")
    ph, pw = _pair(pad)
    sh, sw = _pair(stride)
    dh, dw = _pair(dil)
    P, Q = output_dim(H, ph, dh, R, sh), output_dim(W, pw, dw, S, sw)
    if P <= 0 or Q <= 0:
        raise OracleError("empty output (P=%d, Q=%d)" % (P, Q))
    return (N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw), (N, K, P, Q)


def conv2d_i8_acc(x, w, pad=0, stride=1, dil=1, nthreads=1) -> np.ndarray:
    """int64 accumulators (N, K, P, Q) of the int8 convolution of NCHW x, KCRS w."""
    x = np.ascontiguousarray(x, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.int8)
    args, oshape = _conv_args(x, w, pad, stride, dil)
    acc = np.empty(oshape, dtype=np.int64)
    rc = _load().oracle_conv2d_i8_acc(_ptr(x), _ptr(w), _ptr(acc), *args, int(nthreads))
    if rc:
        raise OracleError("oracle_conv2d_i8_acc failed: %d" % rc)
    return acc


def conv2d_i8_points(x, w, points, pad=0, stride=1, dil=1, nthreads=1) -> np.ndarray:
    """int64 accumulators at the given (n, k, p, q) rows of ``points``."""
    x = np.ascontiguousarray(x, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.int8)
    pts = np.ascontiguousarray(points, dtype=np.int32).reshape(-1, 4)
    args, _ = _conv_args(x, w, pad, stride, dil)
    acc = np.empty(len(pts), dtype=np.int64)
    rc = _load().oracle_conv2d_i8_points(_ptr(x), _ptr(w), _ptr(pts), len(pts),
                                         _ptr(acc), *args, int(nthreads))
    if rc:
        raise OracleError("oracle_conv2d_i8_points failed: %d" % rc)
    return acc


def epilogue_i8(acc, alpha: float) -> np.ndarray:
    """clamp(rint(fl32(fl32(acc) * alpha)), -128, 127) as int8, elementwise."""
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    y = np.empty(acc.shape, dtype=np.int8)
    rc = _load().oracle_epilogue_i8(_ptr(acc), _ptr(y), acc.size, float(alpha))
    if rc:
        raise OracleError("oracle_epilogue_i8 failed: %d" % rc)
    return y


def conv2d_i8(x, w, alpha, pad=0, stride=1, dil=1, nthreads=1):
    """(acc int64, y int8) of the int8 conv fprop, all in logical NCHW/KCRS/NKPQ."""
    acc = conv2d_i8_acc(x, w, pad, stride, dil, nthreads)
    return acc, epilogue_i8(acc, alpha)


def _per_channel(alpha_k, bias_k, K):
    a = np.ascontiguousarray(alpha_k, dtype=np.float32).reshape(-1)
    if a.size != K:
        raise ValueError("alpha_k needs %d values" % K)
    b = None
    if bias_k is not None:
        b = np.ascontiguousarray(bias_k, dtype=np.float32).reshape(-1)
        if b.size != K:
            raise ValueError("bias_k needs %d values" % K)
    return a, b


def epilogue_i8_per_channel(acc, alpha_k, bias_k=None) -> np.ndarray:
    """clamp(rint(fl32(fl32(fl32(acc) * alpha[k]) + bias[k])), -128, 127) as
    int8 over acc in logical NKPQ (the per-output-channel variant)."""
    acc = np.ascontiguousarray(acc, dtype=np.int64)
    N, K = acc.shape[:2]
    a, b = _per_channel(alpha_k, bias_k, K)
    y = np.empty(acc.shape, dtype=np.int8)
    plane = int(np.prod(acc.shape[2:]))
    rc = _load().oracle_epilogue_i8_per_channel(_ptr(acc), _ptr(y), N, K, plane, _ptr(a),
                                                _ptr(b) if b is not None else None)
    if rc:
        raise OracleError("oracle_epilogue_i8_per_channel failed: %d" % rc)
    return y


def conv2d_i8_scaled(x, w, alpha_k, bias_k=None, pad=0, stride=1, dil=1, nthreads=1):
    """(acc int64, y int8) with the per-output-channel scale and bias."""
    acc = conv2d_i8_acc(x, w, pad, stride, dil, nthreads)
    return acc, epilogue_i8_per_channel(acc, alpha_k, bias_k)


def epilogue_f32_per_channel(acc, alpha_k, bias_k=None) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    N, K = acc.shape[:2]
    a, b = _per_channel(alpha_k, bias_k, K)
    y = np.empty(acc.shape, dtype=np.float32)
    _load().oracle_epilogue_f32_per_channel(_ptr(acc), _ptr(y), N, K, int(np.prod(acc.shape[2:])),
                                            _ptr(a), _ptr(b) if b is not None else None)
    return y


def conv2d_f32_acc(x, w, pad=0, stride=1, dil=1, nthreads=1) -> np.ndarray:
    """float64 accumulators (N, K, P, Q) of the fp32 convolution."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    args, oshape = _conv_args(x, w, pad, stride, dil)
    acc = np.empty(oshape, dtype=np.float64)
    rc = _load().oracle_conv2d_f32_acc(_ptr(x), _ptr(w), _ptr(acc), *args, int(nthreads))
    if rc:
        raise OracleError("oracle_conv2d_f32_acc failed: %d" % rc)
    return acc


def conv2d_f32_points(x, w, points, pad=0, stride=1, dil=1, nthreads=1) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    pts = np.ascontiguousarray(points, dtype=np.int32).reshape(-1, 4)
    args, _ = _conv_args(x, w, pad, stride, dil)
    acc = np.empty(len(pts), dtype=np.float64)
    rc = _load().oracle_conv2d_f32_points(_ptr(x), _ptr(w), _ptr(pts), len(pts),
                                          _ptr(acc), *args, int(nthreads))
    if rc:
        raise OracleError("oracle_conv2d_f32_points failed: %d" % rc)
    return acc


def epilogue_f32(acc, alpha: float = 1.0) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    y = np.empty(acc.shape, dtype=np.float32)
    _load().oracle_epilogue_f32(_ptr(acc), _ptr(y), acc.size, float(alpha))
    return y


def conv2d_f32(x, w, alpha=1.0, pad=0, stride=1, dil=1, nthreads=1):
    """(acc float64, y float32) of the fp32 conv fprop in logical layouts."""
    acc = conv2d_f32_acc(x, w, pad, stride, dil, nthreads)
    return acc, epilogue_f32(acc, alpha)


def _layout(fn, src, shape_in, shape_out, dims):
    src = np.ascontiguousarray(src, dtype=np.int8)
    if src.size != int(np.prod(shape_in)):
        raise OracleError("size mismatch")
    dst = np.empty(shape_out, dtype=np.int8)
    rc = getattr(_load(), fn)(_ptr(src), _ptr(dst), *dims)
    if rc:
        raise OracleError("%s failed: %d" % (fn, rc))
    return dst


def nchw_to_nc32hw32(x):
    """Logical NCHW int8 -> NCxHWx<32> buffer shaped (N, C/32, H, W, 32)."""
    N, C, H, W = x.shape
    return _layout("oracle_nchw_to_nc32hw32", x, (N, C, H, W),
                   (N, C // 32, H, W, 32), (N, C, H, W))


def nc32hw32_to_nchw(x_il, N, C, H, W):
    return _layout("oracle_nc32hw32_to_nchw", x_il, (N, C, H, W),
                   (N, C, H, W), (N, C, H, W))


def kcrs_to_c32rsk32(w):
    """Logical KCRS int8 -> CxRSKx<32> buffer shaped (C/32, R, S, K, 32)."""
    K, C, R, S = w.shape
    return _layout("oracle_kcrs_to_c32rsk32", w, (K, C, R, S),
                   (C // 32, R, S, K, 32), (K, C, R, S))


def c32rsk32_to_kcrs(w_il, K, C, R, S):
    return _layout("oracle_c32rsk32_to_kcrs", w_il, (K, C, R, S),
                   (K, C, R, S), (K, C, R, S))


def max_threads() -> int:
    return _load().oracle_max_threads()
