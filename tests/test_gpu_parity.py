"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

int8: bit-exact outputs (the accumulators are exact integers and both sides
apply the same single-multiply / rint / clamp epilogue).  Accumulators are also
compared directly by running with alpha = 1 on small-valued inputs, where the
clamp is rarely reached.  fp32: the tolerance rule of the design notes --
allclose(rtol=1e-4, atol=1e-4) and max|y - ref| / max|ref| <= 1e-4 -- and exact
equality on integer-valued inputs.

Inputs come from the seeded generators; the GPU converts them to the
interleaved layouts with its own transform kernels, the oracle with its own
index maps.  Each case prints its name before it touches the GPU.
"""
import numpy as np
import pytest

import oracle
from convolution_forward_gemm_amd import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NTHREADS = 16  # oracle threads on the GPU machine's host share


def _b():
    from convolution_forward_gemm_amd import binding
    return binding


class ConfigNotApplicable(Exception):
    pass


def each_config(dtype, run):
    """Call run(cfg) for every compiled configuration the problem accepts."""
    ran = 0
    for cfg in range(_b().num_configs(dtype)):
        try:
            run(cfg)
        except ConfigNotApplicable:
            continue
        ran += 1
    assert ran >= 1


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_conv_i8(x, w, alpha, pad, stride, dil, config=None):
    """x NCHW, w KCRS (numpy int8) -> y in NCxHWx<32> (numpy), via GPU
    transforms and the int8 conv kernel."""
    b = _b()
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    conv = b.Conv2dFprop(N, C, H, W, K, R, S, pad=pad, stride=stride, dil=dil, dtype="int8")
    if config is not None:
        try:
            conv.set_config(config)
        except b.ConvError as e:
            # e.g. an (r, s)-outer configuration needs C/32 divisible by its
            # taps per stage
            if e.status != b.CONV_ERR_UNSUPPORTED:
                raise
            raise ConfigNotApplicable(str(e))
    x_il = b.nchw_to_nc32hw32(_dev(x))
    w_il = b.kcrs_to_c32rsk32(_dev(w))
    y = torch.full(conv.y_shape, 77, dtype=torch.int8, device="cuda")  # poison
    conv.run(x_il, w_il, y, alpha)
    torch.cuda.synchronize()
    return y.cpu().numpy(), conv


def oracle_i8_il(x, w, alpha, pad, stride, dil):
    acc, y = oracle.conv2d_i8(x, w, alpha, pad=pad, stride=stride, dil=dil, nthreads=NTHREADS)
    return acc, oracle.nchw_to_nc32hw32(y)


def _announce(*what):
    print("CASE", *what, flush=True)


# --------------------------------------------------------------------------
# Layout transforms: byte-equal to the oracle's index maps
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(1, 32, 8, 8), (2, 64, 5, 7), (3, 96, 1, 1),
                                   (1, 256, 28, 28), (2, 32, 13, 9), (1, 32, 1, 100)])
def test_activation_transforms(shape):
    _announce("transform x", shape)
    b = _b()
    x = wl.int8_uniform(shape, -128, 127, 7, *shape)
    il = b.nchw_to_nc32hw32(_dev(x))
    assert np.array_equal(il.cpu().numpy(), oracle.nchw_to_nc32hw32(x))
    back = b.nc32hw32_to_nchw(il)
    assert np.array_equal(back.cpu().numpy(), x)


@pytest.mark.parametrize("shape", [(32, 32, 3, 3), (256, 256, 3, 3), (64, 32, 5, 9),
                                   (96, 64, 1, 1), (32, 96, 2, 7)])
def test_filter_transforms(shape):
    _announce("transform w", shape)
    b = _b()
    w = wl.int8_uniform(shape, -128, 127, 8, *shape)
    il = b.kcrs_to_c32rsk32(_dev(w))
    assert np.array_equal(il.cpu().numpy(), oracle.kcrs_to_c32rsk32(w))
    back = b.c32rsk32_to_kcrs(il)
    assert np.array_equal(back.cpu().numpy(), w)


# --------------------------------------------------------------------------
# int8: the graded workloads at full size, in the default configuration
# --------------------------------------------------------------------------
@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4"])
def test_int8_workloads_full(key):
    wk = wl.WORKLOADS[key]
    _announce("int8 workload", key, wk.name)
    x, w = wl.make_inputs(wk)
    y, conv = gpu_conv_i8(x, w, wk.alpha, wk.pad, wk.stride, wk.dil)
    print("config:", conv.config, flush=True)
    acc, ref = oracle_i8_il(x, w, wk.alpha, wk.pad, wk.stride, wk.dil)
    assert np.array_equal(y, ref)
    # ties under a power-of-two alpha exercise half-to-even rounding
    a = int(round(-np.log2(wk.alpha)))
    ties = int(np.count_nonzero((acc % (1 << a)) == (1 << (a - 1))))
    print("ties:", ties, flush=True)


# --------------------------------------------------------------------------
# int8: every compiled configuration on shapes with several tiles and ragged
# tails; accumulators exposed with alpha = 1 on small values
# --------------------------------------------------------------------------
RAGGED = [
    # N, C, H, W, K, R, S, pad, stride, dil
    (2, 64, 13, 11, 96, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 32, 9, 17, 160, 3, 5, (2, 0), (2, 1), (1, 2)),
    (3, 96, 7, 7, 32, 1, 1, (0, 0), (1, 1), (1, 1)),
    (1, 32, 20, 6, 64, 5, 3, (3, 3), (3, 2), (2, 3)),
    (2, 128, 6, 6, 256, 3, 3, (1, 1), (2, 2), (1, 1)),
    (1, 32, 1, 1, 32, 1, 1, (0, 0), (1, 1), (1, 1)),
    (1, 32, 3, 3, 32, 3, 3, (0, 0), (1, 1), (1, 1)),       # single output pixel
    (1, 64, 4, 4, 32, 3, 3, (3, 3), (1, 1), (1, 1)),       # padding wider than kernel reach
    (2, 256, 9, 7, 320, 3, 3, (1, 1), (1, 1), (1, 1)),     # C/32 = 8, ragged K tile
    (1, 128, 11, 10, 64, 3, 2, (1, 0), (2, 2), (2, 1)),    # C/32 = 4, stride and dilation
    (3, 256, 5, 6, 96, 1, 1, (0, 0), (1, 1), (1, 1)),      # 1x1, C/32 = 8
    (3, 64, 23, 21, 96, 3, 3, (1, 1), (2, 2), (1, 1)),     # stride 2, ragged M and K tiles
    (1, 64, 56, 56, 64, 3, 3, (1, 1), (2, 2), (1, 1)),     # stride 2, 57-column halo rows
    (3, 128, 5, 7, 96, 1, 1, (0, 0), (1, 1), (1, 1)),      # 1x1 over 128 channels, ragged M
    (2, 32, 11, 9, 64, 3, 3, (2, 1), (2, 1), (1, 2)),      # 3x3 over 32 channels, stride, dilation
    (1, 64, 9, 10, 96, 3, 3, (1, 0), (1, 2), (2, 1)),      # 18 taps
    (2, 32, 7, 8, 32, 5, 5, (2, 2), (1, 1), (1, 1)),       # 25 taps, padding wider than half
    (2, 64, 6, 5, 64, 1, 1, (0, 0), (1, 1), (1, 1)),       # 2 taps
    (1, 32, 8, 9, 32, 2, 3, (1, 1), (1, 1), (1, 1)),       # 6 taps, even filter height
    (1, 128, 6, 6, 64, 1, 3, (0, 1), (1, 1), (1, 1)),      # 12 taps
    (2, 512, 3, 4, 32, 1, 1, (0, 0), (1, 1), (1, 1)),      # 16 taps
    (1, 96, 5, 5, 32, 3, 3, (1, 1), (2, 2), (1, 1)),       # 27 taps, stride 2
]


@pytest.mark.parametrize("case", RAGGED)
def test_int8_configs_accumulators(case):
    N, C, H, W, K, R, S, pad, stride, dil = case
    x = wl.int8_uniform((N, C, H, W), -2, 2, 21, *case[:7])
    w = wl.int8_uniform((K, C, R, S), -2, 2, 22, *case[:7])
    acc, ref = oracle_i8_il(x, w, 1.0, pad, stride, dil)

    def run(cfg):
        _announce("int8 acc", case, "config", cfg)
        y, conv = gpu_conv_i8(x, w, 1.0, pad, stride, dil, config=cfg)
        assert np.array_equal(y, ref), conv.config
    each_config("int8", run)


@pytest.mark.parametrize("case", RAGGED)
def test_int8_configs_full_range(case):
    N, C, H, W, K, R, S, pad, stride, dil = case
    x = wl.int8_uniform((N, C, H, W), -128, 127, 23, *case[:7])
    w = wl.int8_uniform((K, C, R, S), -128, 127, 24, *case[:7])
    alpha = 2.0 ** -10
    _, ref = oracle_i8_il(x, w, alpha, pad, stride, dil)

    def run(cfg):
        _announce("int8 full", case, "config", cfg)
        y, conv = gpu_conv_i8(x, w, alpha, pad, stride, dil, config=cfg)
        assert np.array_equal(y, ref), conv.config
    each_config("int8", run)


@pytest.mark.parametrize("seed", range(6))
def test_int8_random_shapes(seed):
    r = np.random.default_rng(400 + seed)
    N, C, K = int(r.integers(1, 4)), 32 * int(r.integers(1, 4)), 32 * int(r.integers(1, 6))
    R, S = int(r.integers(1, 6)), int(r.integers(1, 6))
    pad = (int(r.integers(0, 4)), int(r.integers(0, 4)))
    stride = (int(r.integers(1, 4)), int(r.integers(1, 4)))
    dil = (int(r.integers(1, 4)), int(r.integers(1, 4)))
    H = int(r.integers(1, 24)) + max(0, dil[0] * (R - 1) + 1 - 2 * pad[0])
    W = int(r.integers(1, 24)) + max(0, dil[1] * (S - 1) + 1 - 2 * pad[1])
    alpha = float(np.float32(r.uniform(1e-4, 1e-2)))
    x = wl.int8_uniform((N, C, H, W), -128, 127, 25, seed)
    w = wl.int8_uniform((K, C, R, S), -128, 127, 26, seed)
    _announce("int8 random", seed, (N, C, H, W, K, R, S, pad, stride, dil, alpha))
    _, ref = oracle_i8_il(x, w, alpha, pad, stride, dil)
    y, _ = gpu_conv_i8(x, w, alpha, pad, stride, dil)
    assert np.array_equal(y, ref)


def test_int8_saturation_and_ties():
    # 256 channels 3x3 on a 3x3 image: the centre sees all 2304 taps.
    _announce("int8 saturation")
    x = np.full((1, 256, 3, 3), 127, np.int8)
    w = np.full((64, 256, 3, 3), 127, np.int8)
    w[32:] = -128
    _, ref = oracle_i8_il(x, w, 2.0 ** -14, (1, 1), (1, 1), (1, 1))
    y, _ = gpu_conv_i8(x, w, 2.0 ** -14, (1, 1), (1, 1), (1, 1))
    assert np.array_equal(y, ref)
    assert y.max() == 127 and y.min() == -128
    # c1 with all ones: 4.5 -> 4 (half to even) at interior outputs
    _announce("int8 ties c1 ones")
    x = np.ones((1, 32, 8, 8), np.int8)
    w = np.ones((32, 32, 3, 3), np.int8)
    _, ref = oracle_i8_il(x, w, 2.0 ** -6, (1, 1), (1, 1), (1, 1))
    y, _ = gpu_conv_i8(x, w, 2.0 ** -6, (1, 1), (1, 1), (1, 1))
    assert np.array_equal(y, ref)
    assert (y == 4).sum() == 32 * 36


def test_int8_deterministic_reruns():
    wk = wl.WORKLOADS["c4"]
    _announce("int8 determinism c4")
    b = _b()
    x, w = wl.make_inputs(wk)
    conv = b.Conv2dFprop(wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S, pad=wk.pad,
                         stride=wk.stride, dil=wk.dil)
    x_il = b.nchw_to_nc32hw32(_dev(x))
    w_il = b.kcrs_to_c32rsk32(_dev(w))
    first = conv.run(x_il, w_il, alpha=wk.alpha).clone()
    for _ in range(20):
        y = conv.run(x_il, w_il, alpha=wk.alpha)
        assert torch.equal(y, first)


def test_run_errors_leave_output_untouched():
    _announce("int8 error paths")
    b = _b()
    conv = b.Conv2dFprop(1, 32, 8, 8, 32, 3, 3, pad=1)
    x = torch.zeros(conv.x_shape, dtype=torch.int8, device="cuda")
    w = torch.zeros(conv.w_shape, dtype=torch.int8, device="cuda")
    y = torch.full(conv.y_shape, 5, dtype=torch.int8, device="cuda")
    lib = b.lib
    st = lib.conv2d_fprop_run(conv._h, x.data_ptr() + 1, w.data_ptr(), y.data_ptr(), 1.0, 0)
    assert st == b.CONV_ERR_MISALIGNED
    st = lib.conv2d_fprop_run(conv._h, 0, w.data_ptr(), y.data_ptr(), 1.0, 0)
    assert st == b.CONV_ERR_NULL
    st = lib.conv2d_fprop_run(conv._h, y.data_ptr(), w.data_ptr(), y.data_ptr(), 1.0, 0)
    assert st == b.CONV_ERR_UNSUPPORTED  # x overlaps y
    torch.cuda.synchronize()
    assert bool((y == 5).all())


def test_run_ignores_an_earlier_pending_hip_error():
    # A failed HIP call of the caller (here hipSetDevice on a device that does
    # not exist) leaves an error pending.  run reports the status of its own
    # launch: CONV_OK, with a correct output.
    import ctypes
    _announce("int8 run after a pending HIP error")
    b = _b()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    wk = wl.WORKLOADS["c1"]
    x, w = wl.make_inputs(wk)
    conv = b.Conv2dFprop(wk.N, wk.C, wk.H, wk.W, wk.K, wk.R, wk.S, pad=wk.pad,
                         stride=wk.stride, dil=wk.dil)
    x_il = b.nchw_to_nc32hw32(_dev(x))
    w_il = b.kcrs_to_c32rsk32(_dev(w))
    y = torch.full(conv.y_shape, 77, dtype=torch.int8, device="cuda")
    hip.hipGetLastError.restype = ctypes.c_int
    torch.cuda.synchronize()
    pending = hip.hipSetDevice(4096)  # hipErrorInvalidDevice, now pending
    try:
        assert pending != 0
        st = b.lib.conv2d_fprop_run(conv._h, x_il.data_ptr(), w_il.data_ptr(), y.data_ptr(),
                                    wk.alpha, torch.cuda.current_stream().cuda_stream)
    finally:
        # the caller's error is still pending after run (run neither reported
        # nor consumed it); consume it here so that later calls see none
        left = hip.hipGetLastError()
    assert st == b.CONV_OK
    assert left == pending
    torch.cuda.synchronize()
    _, ref = oracle_i8_il(x, w, wk.alpha, wk.pad, wk.stride, wk.dil)
    assert np.array_equal(y.cpu().numpy(), ref)


# --------------------------------------------------------------------------
# fp32
# --------------------------------------------------------------------------
def gpu_conv_f32(x, w, pad, stride, dil, alpha=1.0, config=None):
    b = _b()
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    conv = b.Conv2dFprop(N, C, H, W, K, R, S, pad=pad, stride=stride, dil=dil, dtype="fp32")
    if config is not None:
        try:
            conv.set_config(config)
        except b.ConvError as e:
            # e.g. the configuration's LDS filter chunk does not fit this R*S
            if e.status != b.CONV_ERR_UNSUPPORTED:
                raise
            raise ConfigNotApplicable(str(e))
    y = torch.full(conv.y_shape, float("nan"), dtype=torch.float32, device="cuda")
    conv.run(_dev(x), _dev(w), y, alpha)
    torch.cuda.synchronize()
    return y.cpu().numpy(), conv


def assert_f32_rule(y, ref):
    ref32 = ref.astype(np.float64)
    assert np.all(np.isfinite(y))
    assert np.allclose(y, ref32, rtol=1e-4, atol=1e-4)
    scale = np.max(np.abs(ref32))
    if scale > 0:
        assert np.max(np.abs(y - ref32)) / scale <= 1e-4


F32_CASES = [
    (2, 5, 13, 11, 40, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 32, 20, 24, 64, 5, 9, (2, 4), (1, 1), (2, 3)),
    (3, 3, 9, 30, 17, 2, 4, (0, 2), (2, 3), (3, 1)),
    (1, 8, 1, 1, 8, 1, 1, (0, 0), (1, 1), (1, 1)),
    (2, 16, 33, 7, 96, 3, 1, (1, 0), (1, 2), (1, 1)),
    # three input channels: the tiny kernels' step counts (2, 14, 38, 68, 74)
    (3, 3, 9, 8, 33, 1, 1, (0, 0), (1, 1), (1, 1)),
    (2, 3, 17, 19, 40, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 3, 23, 21, 64, 5, 5, (2, 2), (2, 2), (1, 1)),
    (2, 3, 25, 40, 20, 5, 9, (2, 4), (1, 1), (2, 3)),
    (1, 3, 30, 30, 48, 7, 7, (3, 3), (2, 2), (1, 1)),
    # the 5x9 dilated filter on shapes the 16-byte row DMA takes (pw and W
    # multiples of 4, C even): several channel pairs, a partial channel
    # tile, strides
    (2, 6, 15, 36, 40, 5, 9, (2, 4), (1, 1), (2, 3)),
    (3, 4, 21, 44, 64, 5, 9, (2, 4), (2, 2), (2, 3)),
]


@pytest.mark.parametrize("case", F32_CASES)
def test_f32_configs(case):
    N, C, H, W, K, R, S, pad, stride, dil = case
    x, w = wl.make_custom("fp32", N, C, H, W, K, R, S, seed=hash(case) % 1000)
    ref = oracle.conv2d_f32_acc(x, w, pad=pad, stride=stride, dil=dil, nthreads=NTHREADS)

    def run(cfg):
        _announce("fp32", case, "config", cfg)
        y, conv = gpu_conv_f32(x, w, pad, stride, dil, config=cfg)
        assert_f32_rule(y, ref)
    each_config("fp32", run)


@pytest.mark.parametrize("case", F32_CASES)
def test_f32_integer_valued_exact(case):
    N, C, H, W, K, R, S, pad, stride, dil = case
    r = np.random.default_rng(abs(hash(case)) % 1000)
    x = r.integers(-1, 2, size=(N, C, H, W)).astype(np.float32)
    w = r.integers(-1, 2, size=(K, C, R, S)).astype(np.float32)
    ref = oracle.conv2d_f32_acc(x, w, pad=pad, stride=stride, dil=dil, nthreads=NTHREADS)

    def run(cfg):
        _announce("fp32 exact", case, "config", cfg)
        y, _ = gpu_conv_f32(x, w, pad, stride, dil, config=cfg)
        assert np.array_equal(y.astype(np.float64), ref)
    each_config("fp32", run)


# alpha != 1: the oracle's epilogue rounds fl32(alpha * acc) once from its
# double accumulator; the kernel multiplies its fp32 accumulator by alpha.
# Gaussian inputs: the tolerance rule.  Integer-valued inputs: the fp32
# accumulator is exact, so both sides round the same exact product once and
# must agree bit for bit.
F32_ALPHAS = (0.37, -2.5)


@pytest.mark.parametrize("case", F32_CASES)
def test_f32_configs_alpha(case):
    N, C, H, W, K, R, S, pad, stride, dil = case
    x, w = wl.make_custom("fp32", N, C, H, W, K, R, S, seed=(hash(case) + 1) % 1000)
    acc = oracle.conv2d_f32_acc(x, w, pad=pad, stride=stride, dil=dil, nthreads=NTHREADS)
    refs = {a: oracle.epilogue_f32(acc, a) for a in F32_ALPHAS}

    def run(cfg):
        for a in F32_ALPHAS:
            _announce("fp32 alpha", a, case, "config", cfg)
            y, _ = gpu_conv_f32(x, w, pad, stride, dil, alpha=a, config=cfg)
            assert_f32_rule(y, refs[a])
    each_config("fp32", run)


@pytest.mark.parametrize("case", F32_CASES)
def test_f32_integer_valued_alpha_exact(case):
    N, C, H, W, K, R, S, pad, stride, dil = case
    r = np.random.default_rng((abs(hash(case)) + 5) % 1000)
    x = r.integers(-1, 2, size=(N, C, H, W)).astype(np.float32)
    w = r.integers(-1, 2, size=(K, C, R, S)).astype(np.float32)
    acc = oracle.conv2d_f32_acc(x, w, pad=pad, stride=stride, dil=dil, nthreads=NTHREADS)
    refs = {a: oracle.epilogue_f32(acc, a) for a in F32_ALPHAS}

    def run(cfg):
        for a in F32_ALPHAS:
            _announce("fp32 alpha exact", a, case, "config", cfg)
            y, _ = gpu_conv_f32(x, w, pad, stride, dil, alpha=a, config=cfg)
            assert np.array_equal(y, refs[a])
    each_config("fp32", run)


def test_f32_workload_c5_slabs():
    # Whole output slabs of the dilated 5x9 workload, element by element: all
    # 64 output channels over the first 16 and the last 16 output rows of the
    # first and the last image (2 x 64 x 32 x 496 = 2,031,616 outputs).  They
    # hold 64 whole workgroup tiles of the chosen row-halo configuration (one
    # output row of all 64 channels each, 496 of its 512 columns real), the
    # rows whose taps reach into the top and bottom padding, and the output's
    # last tile.
    wk = wl.WORKLOADS["c5"]
    _announce("fp32 workload c5 slabs", wk.name)
    x, w = wl.make_inputs(wk)
    y, conv = gpu_conv_f32(x, w, wk.pad, wk.stride, wk.dil, alpha=wk.alpha)
    print("config:", conv.config, flush=True)
    N, K, P, Q = y.shape
    rows = list(range(16)) + list(range(P - 16, P))
    n_i, k_i, p_i, q_i = np.meshgrid([0, N - 1], np.arange(K), rows, np.arange(Q), indexing="ij")
    pts = np.stack([a.ravel() for a in (n_i, k_i, p_i, q_i)], axis=1).astype(np.int32)
    acc = oracle.conv2d_f32_points(x, w, pts, **wk.conv_kwargs, nthreads=NTHREADS)
    ref = oracle.epilogue_f32(acc, wk.alpha)
    got = y[tuple(pts.T)]
    assert_f32_rule(got, ref)
    assert np.all(np.isfinite(y))


def test_f32_workload_c5_sampled():
    wk = wl.WORKLOADS["c5"]
    _announce("fp32 workload c5", wk.name)
    x, w = wl.make_inputs(wk)
    y, conv = gpu_conv_f32(x, w, wk.pad, wk.stride, wk.dil)
    print("config:", conv.config, flush=True)
    N, K, P, Q = y.shape
    assert (P, Q) == (508, 496)
    r = np.random.default_rng(55)
    pts = [np.stack([r.integers(0, s, 20000) for s in (N, K, P, Q)], axis=1)]
    # every border row and column of one (image, channel) pair, and corners of all
    n0, k0 = int(r.integers(0, N)), int(r.integers(0, K))
    for p in (0, 1, P - 2, P - 1):
        pts.append(np.array([[n0, k0, p, q] for q in range(Q)]))
    for q in (0, 1, 2, 3, Q - 4, Q - 3, Q - 2, Q - 1):
        pts.append(np.array([[n0, k0, p, q] for p in range(P)]))
    for n in range(N):
        for k in range(K):
            pts.append(np.array([[n, k, 0, 0], [n, k, 0, Q - 1], [n, k, P - 1, 0], [n, k, P - 1, Q - 1]]))
    pts = np.concatenate(pts).astype(np.int32)
    ref = oracle.conv2d_f32_points(x, w, pts, **wk.conv_kwargs, nthreads=NTHREADS)
    got = y[tuple(pts.T)]
    assert_f32_rule(got, ref)
    assert np.all(np.isfinite(y))
