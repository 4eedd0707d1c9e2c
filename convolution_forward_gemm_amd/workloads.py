"""Seeded synthetic workloads for conv2d fprop.

This module is the one piece shared by the GPU library's callers and the CPU
oracle's callers: it describes the graded problem shapes and draws their
inputs from counter-free numpy generators keyed by a fixed tuple.  It holds no
convolution arithmetic (no output-size rule, no index maps, no epilogue).

Inputs are always produced in the logical layouts: activations NCHW and
filters KCRS (``[C_out][C_in][kH][kW]``, the weight layout of the "Kimi-K2.6
l1_p80" POPCORNBENCH transcript).  Each side converts them to the interleaved
NCxHWx<32> / CxRSKx<32> forms with its own code.

Value distributions:
  * int8 workloads: independent uniform integers on the stated closed range;
  * the fp32 workload: x ~ N(0, 1); w ~ N(0, 1) * (C*R*S)**-0.5 (fan-in
    scaling, multiplied once in fp32), the synthetic stand-in for the
    transcript's dilated conv problem (batch 8, 32 -> 64 channels, 5x9
    kernel, 512x512, padding (2, 4), dilation (2, 3)).
"""
from __future__ import annotations

import dataclasses
from typing import Tuple

import numpy as np

SEED_ROOT = 2026


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    name: str
    dtype: str          # "int8" or "fp32"
    N: int
    C: int
    H: int
    W: int
    K: int
    R: int
    S: int
    pad: Tuple[int, int] = (0, 0)
    stride: Tuple[int, int] = (1, 1)
    dil: Tuple[int, int] = (1, 1)
    lo: int = -128      # int8 value range, inclusive
    hi: int = 127
    alpha: float = 1.0
    index: int = 0      # seed component

    @property
    def conv_kwargs(self):
        return dict(pad=self.pad, stride=self.stride, dil=self.dil)


WORKLOADS = {
    "c1": Workload("c1", "int8 conv2d fprop 3x3 N1 C32 H8 W8 K32 stride1 pad1",
                   "int8", 1, 32, 8, 8, 32, 3, 3, (1, 1), (1, 1), (1, 1),
                   -8, 7, 2.0 ** -6, 0),
    "c2": Workload("c2", "int8 conv2d fprop 1x1 N2 C128 H8 W8 K128",
                   "int8", 2, 128, 8, 8, 128, 1, 1, (0, 0), (1, 1), (1, 1),
                   -128, 127, 2.0 ** -12, 1),
    "c3": Workload("c3", "int8 conv2d fprop 3x3 N32 C256 H28 W28 K256 stride1 pad1",
                   "int8", 32, 256, 28, 28, 256, 3, 3, (1, 1), (1, 1), (1, 1),
                   -128, 127, 2.0 ** -14, 2),
    "c4": Workload("c4", "int8 conv2d fprop 3x3 N32 C128 H56 W56 K256 stride2 pad1",
                   "int8", 32, 128, 56, 56, 256, 3, 3, (1, 1), (2, 2), (1, 1),
                   -64, 63, 2.0 ** -12, 3),
    "c5": Workload("c5", "fp32 conv2d fprop 5x9 N8 C32 H512 W512 K64 pad(2,4) dil(2,3)",
                   "fp32", 8, 32, 512, 512, 64, 5, 9, (2, 4), (1, 1), (2, 3),
                   0, 0, 1.0, 4),
}


def rng(*key) -> np.random.Generator:
    return np.random.default_rng((SEED_ROOT,) + tuple(int(k) for k in key))


def int8_uniform(shape, lo, hi, *key) -> np.ndarray:
    return rng(*key).integers(lo, hi, size=shape, dtype=np.int8, endpoint=True)


def normal_f32(shape, scale, *key) -> np.ndarray:
    a = rng(*key).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def make_inputs(wl: Workload, trial: int = 0):
    """(x NCHW, w KCRS) for a workload; ``trial`` selects another draw."""
    xs = (wl.N, wl.C, wl.H, wl.W)
    ws = (wl.K, wl.C, wl.R, wl.S)
    if wl.dtype == "int8":
        x = int8_uniform(xs, wl.lo, wl.hi, wl.index, 0, trial)
        w = int8_uniform(ws, wl.lo, wl.hi, wl.index, 1, trial)
    else:
        x = normal_f32(xs, 1.0, wl.index, 0, trial)
        w = normal_f32(ws, 1.0 / np.sqrt(wl.C * wl.R * wl.S), wl.index, 1, trial)
    return x, w


def make_custom(dtype, N, C, H, W, K, R, S, seed, lo=-128, hi=127, wscale=None):
    """Inputs for an arbitrary shape (random parity cases)."""
    if dtype == "int8":
        return (int8_uniform((N, C, H, W), lo, hi, 99, seed, 0),
                int8_uniform((K, C, R, S), lo, hi, 99, seed, 1))
    if wscale is None:
        wscale = 1.0 / np.sqrt(C * R * S)
    return (normal_f32((N, C, H, W), 1.0, 98, seed, 0),
            normal_f32((K, C, R, S), wscale, 98, seed, 1))
