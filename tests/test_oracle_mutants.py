"""Plant plausible mistakes in a copy of the oracle and check the pins catch them.

Each mutant is a one-line textual change to conv_oracle.c, compiled with gcc
into a temporary library on the CPU.  The pins in test_oracle_pins.py are then
run against it; at least one must fail.  Mutants only permute or drop work, so
every one of them stays inside its buffers.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "conv_oracle.c")

MUTANTS = {
    "flipped_filter": ("int64_t wv = w[(((size_t)k * C + c) * R + r) * S + s];",
                       "int64_t wv = w[(((size_t)k * C + c) * R + (R - 1 - r)) * S + (S - 1 - s)];"),
    "pad_sign": ("int h = p * sh - ph + r * dh;\n            if (h < 0 || h >= H) continue; /* zero padding */",
                 "int h = p * sh + ph + r * dh;\n            if (h < 0 || h >= H) continue; /* zero padding */"),
    "dropped_dilation_w": ("int ww = q * sw - pw + s * dw;\n                if (ww < 0 || ww >= W) continue; /* zero padding */",
                           "int ww = q * sw - pw + s;\n                if (ww < 0 || ww >= W) continue; /* zero padding */"),
    "stride_dilation_swapped": ("int ww = q * sw - pw + s * dw;\n                if (ww < 0 || ww >= W) continue;\n",
                                "int ww = q * dw - pw + s * sw;\n                if (ww < 0 || ww >= W) continue;\n"),
    "dropped_last_channel": ("for (int c = 0; c < C; ++c)\n        for (int r = 0; r < R; ++r) {\n            int h = p * sh - ph + r * dh;\n            if (h < 0 || h >= H) continue; /* zero padding */",
                             "for (int c = 0; c < C - 1; ++c)\n        for (int r = 0; r < R; ++r) {\n            int h = p * sh - ph + r * dh;\n            if (h < 0 || h >= H) continue; /* zero padding */"),
    "transposed_input_hw": ("int64_t xv = x[(((size_t)n * C + c) * H + h) * W + ww];",
                            "int64_t xv = x[(((size_t)n * C + c) * W + ww) * H + h];"),
    "round_half_away": ("float r = rintf(g);", "float r = roundf(g);"),
    "dropped_clamp": ("if (r > 127.0f) r = 127.0f;", ""),
    "divide_not_multiply": ("volatile float g = f * alpha;", "volatile float g = f / (1.0f / alpha);"),
    "output_dim_off_by_one": ("return (int)(num / stride + 1);", "return (int)(num / stride);"),
    "f32_float_accumulator": ("double acc = 0.0;\n    for (int c = 0; c < C; ++c)",
                              "float acc = 0.0f;\n    for (int c = 0; c < C; ++c)"),
    "per_channel_bias_after_rounding": ("volatile float h = g + (bias ? bias[k] : 0.0f);\n                float r = rintf(h);",
                                        "volatile float h = g;\n                float r = rintf(h) + (bias ? bias[k] : 0.0f);"),
    "per_channel_wrong_channel": ("volatile float g = f * alpha[k];", "volatile float g = f * alpha[(k + 1) % K];"),
    "per_channel_fused": ("volatile float g = f * alpha[k];\n                volatile float h = g + (bias ? bias[k] : 0.0f);",
                          "volatile float g = 0.0f;\n                volatile float h = fmaf(f, alpha[k], bias ? bias[k] : 0.0f) + g;"),
    "f32_dropped_alpha": ("y[i] = (float)((double)alpha * acc[i]);", "y[i] = (float)acc[i];"),
    "f32_acc_rounded_before_alpha": ("y[i] = (float)((double)alpha * acc[i]);",
                                     "y[i] = (float)((double)alpha * (double)(float)acc[i]);"),
    "f32_alpha_in_fp32": ("y[i] = (float)((double)alpha * acc[i]);",
                          "y[i] = (float)acc[i] * alpha;"),
    "layout_hw_swapped": ("dst[((((size_t)n * (C / 32) + c / 32) * H + h) * W + w) * 32 + c % 32] =",
                          "dst[((((size_t)n * (C / 32) + c / 32) * W + w) * H + h) * 32 + c % 32] ="),
    "filter_layout_rs_swapped": ("dst[((((size_t)(c / 32) * R + r) * S + s) * K + k) * 32 + c % 32] =",
                                 "dst[((((size_t)(c / 32) * S + s) * R + r) * K + k) * 32 + c % 32] ="),
}


def _battery():
    """Run the pins; return the names of those that failed."""
    checks = [
        ("worked_dims", pins.test_output_dim_worked_examples, ()),
        ("bruteforce_dims", pins.test_output_dim_bruteforce, ()),
        ("tap_counts", pins.test_tap_trace_origin_counts, ()),
        ("tap_positions", pins.test_tap_trace_origin_positions, ()),
        ("rounding_c1", pins.test_rounding_c1_all_ones, ()),
        ("epilogue_numpy", pins.test_epilogue_against_numpy_float32, ()),
        ("saturation", pins.test_saturation_extremes_c3_channels, ()),
        ("one_hot", pins.test_one_hot_activation, ((3, 2), (2, 3), (3, 1))),
        ("matmul_1x1", pins.test_1x1_is_matmul, ()),
        ("im2col", pins.test_implicit_equals_explicit_im2col, (3,)),
        ("torch_i8", pins.test_int8_matches_torch_f64, (4,)),
        ("torch_f32", pins.test_f32_matches_torch_f64, (1,)),
        ("layout_hand", pins.test_nc32hw32_hand_listed, ()),
        ("filter_layout_hand", pins.test_c32rsk32_hand_listed, ()),
        ("layout_numpy", pins.test_layout_maps_match_numpy_reshape, ()),
        ("per_channel_hand", pins.test_per_channel_hand_values, ()),
        ("per_channel_two_roundings", pins.test_per_channel_multiply_then_add_rounds_twice, ()),
        ("per_channel_c1", pins.test_per_channel_c1_all_ones_with_bias, ()),
        ("per_channel_scalar", pins.test_per_channel_with_one_scale_is_the_scalar_epilogue, ()),
        ("f32_per_channel_hand", pins.test_f32_per_channel_hand_values, ()),
        ("f32_alpha_hand", pins.test_f32_epilogue_alpha_hand_values, ()),
        ("f32_alpha_tap_trace", pins.test_f32_alpha_scales_the_tap_trace, ()),
    ]
    for acc, alpha, expect in [(2088960, 2.0 ** -14, 127), (-2105344, 2.0 ** -14, -128),
                               (40960, 2.0 ** -14, 2), (25, 0.1, 2)]:
        checks.append(("hand_%d" % acc, pins.test_epilogue_hand_values, (acc, alpha, expect)))
    failed = []
    for name, fn, args in checks:
        try:
            fn(*args)
        except (AssertionError, oracle.OracleError, ValueError, IndexError):
            failed.append(name)
    return failed


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmutated_copy_passes_every_pin(workdir):
    lib = os.path.join(workdir, "lib_plain.so")
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, SRC, "-o", lib, "-lm"])
    prev = oracle._swap_library(lib)
    try:
        assert _battery() == []
    finally:
        oracle._restore_library(prev)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = src.replace(old, new, 1)
    csrc = os.path.join(workdir, name + ".c")
    lib = os.path.join(workdir, name + ".so")
    with open(csrc, "w") as f:
        f.write(mutated)
    subprocess.check_call(["gcc", *oracle.GCC_FLAGS, csrc, "-o", lib, "-lm"])
    prev = oracle._swap_library(lib)
    try:
        failed = _battery()
    finally:
        oracle._restore_library(prev)
    assert failed, "mutant %s passed every pin" % name
