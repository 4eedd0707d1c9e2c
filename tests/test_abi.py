"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/convfprop.h declares,
and validate problems at descriptor creation.  run() rejects null and
misaligned pointers before anything is enqueued, so those paths are exercised
here with fake pointer values that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convfprop.h")


@pytest.fixture(scope="module")
def b():
    from convolution_forward_gemm_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_0-9]+)\s*\(", text)
    return sorted({n for n in names if n.startswith(("conv2d_", "conv_"))})


def test_header_functions_are_exported(b):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(b.lib, n), n
        assert n in b.SIGNATURES, "binding lacks a signature for " + n
    assert sorted(b.SIGNATURES) == names


def test_status_strings(b):
    for code in range(9):
        s = b.status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in b.status_string(99)


def _create(b, *args, dtype=None, layout=None):
    h = ctypes.c_void_p(1234)
    dt = b.CONV_DTYPE_INT8 if dtype is None else dtype
    lay = b.CONV_LAYOUT_NC32HW32_C32RSK32 if layout is None else layout
    st = b.lib.conv2d_fprop_desc_create(ctypes.byref(h), *args, dt, lay)
    return st, h


GOOD = (32, 256, 28, 28, 256, 3, 3, 1, 1, 1, 1, 1, 1)


def test_create_and_query(b):
    st, h = _create(b, *GOOD)
    assert st == b.CONV_OK and h.value
    P, Q = ctypes.c_int(), ctypes.c_int()
    assert b.lib.conv2d_fprop_desc_get_output_dims(h, ctypes.byref(P), ctypes.byref(Q)) == 0
    assert (P.value, Q.value) == (28, 28)
    buf = ctypes.create_string_buffer(8)
    assert b.lib.conv2d_fprop_desc_get_config(h, buf, 8) == 0
    assert len(buf.value) == 7  # truncated, NUL-terminated
    assert b.lib.conv2d_fprop_desc_destroy(h) == 0
    assert b.lib.conv2d_fprop_desc_destroy(None) == 0


@pytest.mark.parametrize("args,expect", [
    ((0, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1), "CONV_ERR_INVALID_SHAPE"),
    ((1, 32, 8, 8, 32, 3, 3, -1, 1, 1, 1, 1, 1), "CONV_ERR_INVALID_SHAPE"),
    ((1, 32, 8, 8, 32, 3, 3, 1, 1, 0, 1, 1, 1), "CONV_ERR_INVALID_SHAPE"),
    ((1, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 0), "CONV_ERR_INVALID_SHAPE"),
    ((1, 32, 2, 2, 32, 5, 5, 0, 0, 1, 1, 1, 1), "CONV_ERR_INVALID_SHAPE"),  # P <= 0
    ((1, 48, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1), "CONV_ERR_UNSUPPORTED"),    # C % 32
    ((1, 32, 8, 8, 40, 3, 3, 1, 1, 1, 1, 1, 1), "CONV_ERR_UNSUPPORTED"),    # K % 32
    ((1, 16384, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1), "CONV_ERR_OVERFLOW_RISK"),  # CRS = 147456
    ((1, 14560, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1), "CONV_OK"),             # CRS = 131040
    ((1, 32, 65536, 1024, 32, 1, 1, 0, 0, 1, 1, 1, 1), "CONV_ERR_UNSUPPORTED"),  # 2 GiB tensor
])
def test_create_validation(b, args, expect):
    st, h = _create(b, *args)
    assert st == getattr(b, expect), b.status_string(st)
    if st == b.CONV_OK:
        b.lib.conv2d_fprop_desc_destroy(h)
    else:
        assert not h.value  # out is cleared on error


def test_create_dtype_layout_pairs(b):
    st, _ = _create(b, *GOOD, dtype=b.CONV_DTYPE_FP32, layout=b.CONV_LAYOUT_NC32HW32_C32RSK32)
    assert st == b.CONV_ERR_UNSUPPORTED
    st, _ = _create(b, *GOOD, dtype=b.CONV_DTYPE_INT8, layout=b.CONV_LAYOUT_NCHW_KCRS)
    assert st == b.CONV_ERR_UNSUPPORTED
    st, h = _create(b, 1, 3, 9, 9, 5, 3, 3, 1, 1, 1, 1, 1, 1,
                    dtype=b.CONV_DTYPE_FP32, layout=b.CONV_LAYOUT_NCHW_KCRS)
    assert st == b.CONV_OK  # fp32 has no multiple-of-32 rule
    b.lib.conv2d_fprop_desc_destroy(h)
    assert b.lib.conv2d_fprop_desc_create(None, *GOOD, 0, 1) == b.CONV_ERR_NULL


def test_output_dims_match_python_objects(b):
    c = b.Conv2dFprop(8, 32, 512, 512, 64, 5, 9, pad=(2, 4), dil=(2, 3), dtype="fp32")
    assert (c.P, c.Q) == (508, 496)
    c = b.Conv2dFprop(32, 128, 56, 56, 256, 3, 3, pad=1, stride=2)
    assert (c.P, c.Q) == (28, 28)


def test_set_config(b):
    # every compiled int8 configuration runs at least one of these shapes
    # (a configuration may not fit a shape: its halo ring can exceed LDS);
    # a refusal is CONV_ERR_UNSUPPORTED and leaves the descriptor usable
    shapes = [b.Conv2dFprop(*GOOD[:7], pad=1),
              b.Conv2dFprop(32, 128, 56, 56, 256, 3, 3, pad=1, stride=2),
              b.Conv2dFprop(2, 256, 9, 7, 320, 3, 3, pad=1),
              b.Conv2dFprop(1, 32, 8, 8, 32, 3, 3, pad=1),
              b.Conv2dFprop(2, 128, 8, 8, 128, 1, 1)]
    # one shape per tap count of the tap-count-unrolled kernels (C/32 * R * S)
    for C, R, S in ((64, 1, 1), (96, 1, 1), (64, 1, 3), (256, 1, 1), (128, 1, 3), (512, 1, 1),
                    (64, 3, 3), (32, 5, 5), (96, 3, 3)):
        shapes.append(b.Conv2dFprop(1, C, 7, 7, 32, R, S))
    names = set()
    for i in range(b.num_configs("int8")):
        ok = 0
        for c in shapes:
            try:
                c.set_config(i)
            except b.ConvError as e:
                assert e.status == b.CONV_ERR_UNSUPPORTED
                continue
            assert c.config.startswith("config=%d " % i)
            names.add(c.config.split()[1])
            ok += 1
        assert ok >= 1, "configuration %d runs none of the shapes" % i
    assert len(names) == b.num_configs("int8"), "configuration names are not unique"
    with pytest.raises(b.ConvError):
        shapes[0].set_config(b.num_configs("int8"))
    assert b.num_configs("fp32") >= 1


def test_run_rejects_null_and_misaligned_before_launch(b):
    st, h = _create(b, 1, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1)
    assert st == 0
    run = b.lib.conv2d_fprop_run
    assert run(h, 0, 4096, 8192, 1.0, None) == b.CONV_ERR_NULL
    assert run(h, 4096, 0, 8192, 1.0, None) == b.CONV_ERR_NULL
    assert run(h, 4096, 8192, 0, 1.0, None) == b.CONV_ERR_NULL
    assert run(None, 4096, 8192, 1 << 20, 1.0, None) == b.CONV_ERR_NULL
    assert run(h, 4097, 1 << 16, 1 << 20, 1.0, None) == b.CONV_ERR_MISALIGNED
    assert run(h, 4096, (1 << 16) + 8, 1 << 20, 1.0, None) == b.CONV_ERR_MISALIGNED
    assert run(h, 4096, 1 << 16, (1 << 20) + 4, 1.0, None) == b.CONV_ERR_MISALIGNED
    # y overlapping x is rejected too (x: 2 KiB at 4096)
    assert run(h, 4096, 1 << 16, 4096 + 1024, 1.0, None) == b.CONV_ERR_UNSUPPORTED
    # int8: an alpha without an int8 value is refused before any launch
    for bad in (float("nan"), float("inf"), float("-inf")):
        assert run(h, 4096, 1 << 16, 1 << 20, bad, None) == b.CONV_ERR_INVALID_ALPHA
    b.lib.conv2d_fprop_desc_destroy(h)


def test_run_scaled_rejects_bad_arguments_before_launch(b):
    st, h = _create(b, 1, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1)
    assert st == 0
    run = b.lib.conv2d_fprop_run_scaled
    x, w, y, a, bias = 4096, 1 << 16, 1 << 20, 1 << 24, (1 << 24) + 4096
    assert run(h, x, w, y, 0, bias, None) == b.CONV_ERR_NULL          # alpha required
    assert run(h, 0, w, y, a, bias, None) == b.CONV_ERR_NULL
    assert run(None, x, w, y, a, bias, None) == b.CONV_ERR_NULL
    assert run(h, x, w, y, a + 4, bias, None) == b.CONV_ERR_MISALIGNED  # 16-byte alignment
    assert run(h, x, w, y, a, bias + 8, None) == b.CONV_ERR_MISALIGNED
    assert run(h, x + 1, w, y, a, bias, None) == b.CONV_ERR_MISALIGNED
    # the per-channel arrays (32 floats) must not overlap y (2 KiB at 1 MiB)
    assert run(h, x, w, y, y + 512, bias, None) == b.CONV_ERR_UNSUPPORTED
    assert run(h, x, w, y, a, y + 1024, None) == b.CONV_ERR_UNSUPPORTED
    b.lib.conv2d_fprop_desc_destroy(h)


def test_graph_create_rejects_bad_arguments_before_capture(b):
    st, h = _create(b, 1, 32, 8, 8, 32, 3, 3, 1, 1, 1, 1, 1, 1)
    assert st == 0
    g = ctypes.c_void_p()
    create = b.lib.conv2d_fprop_graph_create
    x, w, y = 4096, 1 << 16, 1 << 20
    assert create(None, h, x, w, y, 1.0, 4) == b.CONV_ERR_NULL
    assert create(ctypes.byref(g), None, x, w, y, 1.0, 4) == b.CONV_ERR_NULL
    assert create(ctypes.byref(g), h, x + 1, w, y, 1.0, 4) == b.CONV_ERR_MISALIGNED
    assert create(ctypes.byref(g), h, x, w, y, float("nan"), 4) == b.CONV_ERR_INVALID_ALPHA
    for calls in (0, -1, 4097):
        assert create(ctypes.byref(g), h, x, w, y, 1.0, calls) == b.CONV_ERR_INVALID_SHAPE
    assert not g.value
    assert b.lib.conv2d_fprop_graph_launch(None, None) == b.CONV_ERR_NULL
    assert b.lib.conv2d_fprop_graph_destroy(None) == b.CONV_OK
    b.lib.conv2d_fprop_desc_destroy(h)


def test_transforms_reject_bad_arguments(b):
    f = b.lib.conv_nchw_to_nc32hw32_i8
    assert f(0, 4096, 1, 32, 2, 2, None) == b.CONV_ERR_NULL
    assert f(4096, 8192, 1, 48, 2, 2, None) == b.CONV_ERR_UNSUPPORTED
    assert f(4096, 8192, 0, 32, 2, 2, None) == b.CONV_ERR_INVALID_SHAPE
    assert f(4097, 8192, 1, 32, 2, 2, None) == b.CONV_ERR_MISALIGNED
    assert f(4096, 4096 + 64, 1, 32, 2, 2, None) == b.CONV_ERR_UNSUPPORTED  # overlap
    g = b.lib.conv_kcrs_to_c32rsk32_i8
    assert g(4096, 8192, 32, 40, 3, 3, None) == b.CONV_ERR_UNSUPPORTED


def test_binding_has_no_cpu_fallback():
    import convolution_forward_gemm_amd.binding as mod
    src = open(mod.__file__).read()
    assert "import oracle" not in src and "from oracle" not in src
    for name in os.listdir(os.path.join(ROOT, "convolution_forward_gemm_amd")):
        if name.endswith(".py"):
            text = open(os.path.join(ROOT, "convolution_forward_gemm_amd", name)).read()
            assert "import oracle" not in text and "from oracle" not in text, name


def test_shape_table_choices(b):
    # the per-shape table names configurations; a name that no longer exists
    # would silently fall back to the selection model
    from convolution_forward_gemm_amd import workloads as wl
    expect = {
        "c1": "i8_tiny_unrolled_r3s3_cb1_mfma32x32x32_frag1x1",
        "c2": "i8_tiny_unrolled_r1s1_cb4_mfma32x32x32_frag1x1",
        "c3": "i8_halo_regfilter_mfma32x32x32_wg4x2_frag1x4_r3s3_ring4_hj2_pitch32_cps1_pt7_swz",
        "c4": "i8_halo_regfilter_mfma32x32x32_wg4x2_frag2x2_r3s3_ring3_hj4_pitch64_cps1",
        "c5": "f32_rowhalo_mfma32x32x2_8waves_frag2x2_r5s9_dil2x3_pitch520_wsingle_dma16",
    }
    for key, name in expect.items():
        w = wl.WORKLOADS[key]
        c = b.Conv2dFprop(w.N, w.C, w.H, w.W, w.K, w.R, w.S, pad=w.pad, stride=w.stride,
                          dil=w.dil, dtype=w.dtype)
        assert c.config.split()[1] == name, (key, c.config)


def test_fixed_filter_fp32_kernel_serves_other_sizes(b):
    # the fp32 row-halo kernel is compiled for the 5x9 filter with dilation
    # (2, 3); the selection model takes it for other wide problems with that
    # filter (the 72-row shard of the 512 x 512 workload), and never for
    # another filter
    c = b.Conv2dFprop(8, 32, 72, 512, 64, 5, 9, pad=(2, 4), dil=(2, 3), dtype="fp32")
    assert c.config.split()[1].startswith("f32_rowhalo_"), c.config
    c = b.Conv2dFprop(8, 32, 72, 512, 64, 5, 9, pad=(2, 4), dil=(1, 1), dtype="fp32")
    assert not c.config.split()[1].startswith("f32_rowhalo_"), c.config
