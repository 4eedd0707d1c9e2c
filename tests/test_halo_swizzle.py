"""CPU check of the swizzled LDS halo layout (csrc/halo_swizzle.hpp).

tests/c/halo_swizzle_check.cpp includes the same header the gfx950 kernel
compiles and checks, for every tile of a problem: each halo row's columns
occupy distinct slots of the row and the inverse map (used by the LDS-DMA
sources) undoes the forward one (used by the fragment reads); and every
32-lane fragment read at every filter tap touches 16 (8) distinct banks in
each aligned group of 16 (8) lanes.  The plain row-major layout conflicts in
43% of the 16-lane groups on the 3x3 stride-1 workload and in all of them
on the stride-2 one (the rate rocprofv3's SQ_LDS_BANK_CONFLICT showed for
those layouts).
"""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "halo_swizzle_check.cpp")
CSRC = os.path.join(ROOT, "convolution_forward_gemm_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("swz") / "halo_swizzle_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", CSRC, SRC, "-o", exe], check=True, capture_output=True, text=True)
    return exe


def _check(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
    _, frags, plain = r.stdout.split()
    return int(frags), int(plain)


def test_headline_3x3_stride1(checker):
    # N32 C256 28x28 3x3 pad 1: 256-pixel tiles, pitch 32
    frags, plain = _check(checker, 32, 28, 28, 3, 3, 1, 1, 1, 1, 1, 1, 256, 32)
    assert frags == 784 * 9 and plain == 6048  # the plain layout: 43% of the groups


def test_strided_3x3(checker):
    # N32 C128 56x56 3x3 stride 2 pad 1: pitch 64, columns split by parity
    frags, plain = _check(checker, 32, 56, 56, 3, 3, 1, 1, 2, 2, 1, 1, 256, 64)
    assert frags == 784 * 9 and plain == 2 * frags  # the plain layout: every group


def test_224_pixel_tiles(checker):
    # 128 x 224 tiles (7 fragments): tiles start mid-image on both workloads
    frags, _ = _check(checker, 32, 28, 28, 3, 3, 1, 1, 1, 1, 1, 1, 224, 32)
    assert frags == 784 * 9
    frags, _ = _check(checker, 32, 56, 56, 3, 3, 1, 1, 2, 2, 1, 1, 224, 64)
    assert frags == 784 * 9


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(checker, seed):
    r = np.random.default_rng(900 + seed)
    while True:
        N, H, W = int(r.integers(1, 4)), int(r.integers(1, 40)), int(r.integers(1, 30))
        R, S = int(r.integers(1, 6)), int(r.integers(1, 6))
        ph, pw = int(r.integers(0, 3)), int(r.integers(0, 3))
        sh, sw = int(r.integers(1, 3)), int(r.integers(1, 3))
        dh, dw = int(r.integers(1, 3)), int(r.integers(1, 3))
        P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
        Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
        if P < 1 or Q < 1 or H + 2 * ph - dh * (R - 1) - 1 < 0 or W + 2 * pw - dw * (S - 1) - 1 < 0:
            continue
        WV = (Q - 1) * sw + (S - 1) * dw + 1
        need = 2 * ((WV + 1) // 2) if sw == 2 else WV
        pitch = 32 if need <= 32 else 64
        if need <= 64:
            break
    _check(checker, N, H, W, R, S, ph, pw, sh, sw, dh, dw, int(r.choice([64, 128, 256])), pitch)
