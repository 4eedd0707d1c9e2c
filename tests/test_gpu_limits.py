"""GPU parity at the limits the descriptor accepts.

* The longest int8 reduction: C*R*S just under 131072 (= 2^31 / 2^14), where
  the largest possible accumulator (C*R*S * 127 * 127) still fits int32:
  every compiled configuration, bit-exact against the oracle, plus the
  all-127 case whose centre output needs the full int32 range.
* Tensors just under the 2 GiB byte limit (int8 and fp32 activations):
  sampled outputs against the oracle's per-point evaluation, including the
  last pixels of the last image, where a 32-bit offset overflow or a
  clipped buffer descriptor would show.
"""
import numpy as np
import pytest

import oracle
from convolution_forward_gemm_amd import workloads as wl
from test_gpu_parity import (NTHREADS, _announce, _b, _dev, assert_f32_rule, each_config,
                             gpu_conv_i8, oracle_i8_il)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

C_MAX = 14560  # 455 channel blocks: C*9 = 131040 < 131072


def test_int8_longest_reduction_every_config():
    N, C, H, W, K = 1, C_MAX, 5, 5, 64
    x = wl.int8_uniform((N, C, H, W), -128, 127, 41, C)
    w = wl.int8_uniform((K, C, 3, 3), -128, 127, 42, C)
    alpha = 2.0 ** -16
    acc, ref = oracle_i8_il(x, w, alpha, (1, 1), (1, 1), (1, 1))
    assert np.abs(acc).max() > 2 ** 20  # well past fp32's exact-integer range

    def run(cfg):
        _announce("int8 longest reduction", (N, C, H, W, K), "config", cfg)
        y, conv = gpu_conv_i8(x, w, alpha, (1, 1), (1, 1), (1, 1), config=cfg)
        assert np.array_equal(y, ref), conv.config
    each_config("int8", run)


def test_int8_longest_reduction_extreme_accumulators():
    # x = 127 everywhere; the first 32 filters are +127, the rest -128: the
    # centre pixel's accumulators are 131040 * 127 * 127 = 2113614240 and
    # 131040 * 127 * -128 = -2130186240 (both inside int32)
    N, C, H, W, K = 1, C_MAX, 3, 3, 64
    x = np.full((N, C, H, W), 127, np.int8)
    w = np.full((K, C, 3, 3), 127, np.int8)
    w[32:] = -128
    b = _b()
    for alpha in (2.0 ** -24, 2.0 ** -31):
        _announce("int8 extreme accumulators", alpha)
        acc, ref = oracle_i8_il(x, w, alpha, (1, 1), (1, 1), (1, 1))
        assert acc.max() == C * 9 * 127 * 127 and acc.min() == C * 9 * 127 * -128
        y, _ = gpu_conv_i8(x, w, alpha, (1, 1), (1, 1), (1, 1))
        assert np.array_equal(y, ref)
    with pytest.raises(b.ConvError) as e:
        b.Conv2dFprop(1, C_MAX + 32, 3, 3, 64, 3, 3, pad=1)
    assert e.value.status == b.CONV_ERR_OVERFLOW_RISK


def _points(shape, n, seed):
    N, K, P, Q = shape
    r = np.random.default_rng(seed)
    pts = [np.stack([r.integers(0, s, n) for s in shape], axis=1)]
    for k in range(K):  # the first and the last pixel of the tensor, every channel
        pts.append(np.array([[0, k, 0, 0], [N - 1, k, P - 1, Q - 1], [N - 1, k, P - 1, 0]]))
    return np.concatenate(pts).astype(np.int32)


def test_int8_activation_just_under_2gib():
    N, C, H, W, K = 127, 256, 256, 256, 32
    assert N * C * H * W < 2 ** 31 - 1 and N * C * H * W > 2 ** 31 - 2 ** 25
    b = _b()
    _announce("int8 2 GiB activation", (N, C, H, W, K))
    x = wl.int8_uniform((N, C, H, W), -128, 127, 43, 0)
    w = wl.int8_uniform((K, C, 1, 1), -128, 127, 43, 1)
    alpha = 2.0 ** -12
    conv = b.Conv2dFprop(N, C, H, W, K, 1, 1)
    print("config:", conv.config, flush=True)
    xd = _dev(x)
    x_il = b.nchw_to_nc32hw32(xd)
    del xd
    w_il = b.kcrs_to_c32rsk32(_dev(w))
    y_il = torch.full(conv.y_shape, 77, dtype=torch.int8, device="cuda")
    conv.run(x_il, w_il, y_il, alpha)
    y = b.nc32hw32_to_nchw(y_il).view(N, K, H, W).cpu().numpy()
    del x_il, y_il
    torch.cuda.synchronize()
    pts = _points((N, K, H, W), 4000, 44)
    acc = oracle.conv2d_i8_points(x, w, pts, nthreads=NTHREADS)
    ref = oracle.epilogue_i8(acc, alpha)
    assert np.array_equal(y[tuple(pts.T)], ref)


def test_fp32_activation_just_under_2gib():
    N, C, H, W, K = 8, 63, 1024, 1024, 16
    assert N * C * H * W * 4 < 2 ** 31 - 1 and N * C * H * W * 4 > 2 ** 31 - 2 ** 27
    b = _b()
    _announce("fp32 2 GiB activation", (N, C, H, W, K))
    x = wl.normal_f32((N, C, H, W), 1.0, 45, 0)
    w = wl.normal_f32((K, C, 1, 1), C ** -0.5, 45, 1)
    conv = b.Conv2dFprop(N, C, H, W, K, 1, 1, dtype="fp32")
    print("config:", conv.config, flush=True)
    xd, wd = _dev(x), _dev(w)
    yd = torch.full(conv.y_shape, float("nan"), device="cuda")
    conv.run(xd, wd, yd, 1.0)
    y = yd.cpu().numpy()
    del xd, yd
    torch.cuda.synchronize()
    pts = _points((N, K, H, W), 4000, 46)
    ref = oracle.conv2d_f32_points(x, w, pts, nthreads=NTHREADS)
    assert_f32_rule(y[tuple(pts.T)], ref)
