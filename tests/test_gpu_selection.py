"""GPU parity on the configuration-selection model's held-out shapes: for
every shape of the validation grid (seeded random int8 and fp32 problems with
1x1 to 7x7 filters, strides, dilations and paddings, plus the per-GPU shares
of the sharding plan), the configuration desc_create picks must match the
oracle -- on every output where the oracle finishes quickly, else on sampled
outputs that include the tensor's first and last pixels of every channel.
"""
import numpy as np
import pytest

import oracle
from convolution_forward_gemm_amd import sweep
from convolution_forward_gemm_amd import workloads as wl
from test_gpu_parity import NTHREADS, _announce, _b, _dev, assert_f32_rule

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

FULL_MACS = 4e9  # above this, sampled outputs


def _points(N, K, P, Q, n, seed):
    r = np.random.default_rng(seed)
    pts = [np.stack([r.integers(0, s, n) for s in (N, K, P, Q)], axis=1)]
    for k in range(K):
        pts.append(np.array([[0, k, 0, 0], [N - 1, k, P - 1, Q - 1]]))
    return np.concatenate(pts).astype(np.int32)


@pytest.mark.parametrize("idx", range(len(sweep.grid_shapes("validate"))))
def test_selected_configuration_matches_oracle(idx):
    sh = sweep.grid_shapes("validate")[idx]
    dt, N, C, H, W, K, R, S, ph, pw, sth, stw, dh, dw = sh
    b = _b()
    kw = dict(pad=(ph, pw), stride=(sth, stw), dil=(dh, dw))
    conv = b.Conv2dFprop(N, C, H, W, K, R, S, dtype=dt, **kw)
    P, Q = conv.P, conv.Q
    _announce("selection", idx, sh, conv.config)
    macs = float(N) * K * P * Q * C * R * S
    if dt == "int8":
        x = wl.int8_uniform((N, C, H, W), -128, 127, 60, idx, 0)
        w = wl.int8_uniform((K, C, R, S), -128, 127, 60, idx, 1)
        alpha = 2.0 ** -12
        y_il = torch.full(conv.y_shape, 77, dtype=torch.int8, device="cuda")
        conv.run(b.nchw_to_nc32hw32(_dev(x)), b.kcrs_to_c32rsk32(_dev(w)), y_il, alpha)
        y = b.nc32hw32_to_nchw(y_il).view(N, K, P, Q).cpu().numpy()
        if macs <= FULL_MACS:
            _, ref = oracle.conv2d_i8(x, w, alpha, nthreads=NTHREADS, **kw)
            assert np.array_equal(y, ref)
        else:
            pts = _points(N, K, P, Q, 3000, idx)
            ref = oracle.epilogue_i8(oracle.conv2d_i8_points(x, w, pts, nthreads=NTHREADS, **kw),
                                     alpha)
            assert np.array_equal(y[tuple(pts.T)], ref)
    else:
        x = wl.normal_f32((N, C, H, W), 1.0, 61, idx, 0)
        w = wl.normal_f32((K, C, R, S), (C * R * S) ** -0.5, 61, idx, 1)
        yd = torch.full(conv.y_shape, float("nan"), device="cuda")
        conv.run(_dev(x), _dev(w), yd, 1.0)
        y = yd.cpu().numpy()
        if macs <= FULL_MACS:
            _, ref = oracle.conv2d_f32(x, w, 1.0, nthreads=NTHREADS, **kw)
            assert_f32_rule(y, ref)
        else:
            pts = _points(N, K, P, Q, 3000, idx)
            ref = oracle.conv2d_f32_points(x, w, pts, nthreads=NTHREADS, **kw)
            assert_f32_rule(y[tuple(pts.T)], ref)


def _train_sample():
    out = []
    for sh in sweep.grid_shapes("train")[::11]:
        dt, N, C, H, W = sh[:5]
        if N * C * H * W <= 8 << 20:
            out.append(sh)
    return out


@pytest.mark.parametrize("sh", _train_sample(), ids=lambda s: "x".join(str(v) for v in s))
def test_every_configuration_on_training_shapes(sh):
    # the sweep timed every configuration on these shapes; here each one's
    # output is checked (sampled outputs, first and last pixels included)
    dt, N, C, H, W, K, R, S, ph, pw, sth, stw, dh, dw = sh
    b = _b()
    kw = dict(pad=(ph, pw), stride=(sth, stw), dil=(dh, dw))
    conv = b.Conv2dFprop(N, C, H, W, K, R, S, dtype=dt, **kw)
    P, Q = conv.P, conv.Q
    seed = sum(sh[1:]) % 1000
    pts = _points(N, K, P, Q, 1000, seed)
    if dt == "int8":
        x = wl.int8_uniform((N, C, H, W), -128, 127, 62, *sh[1:8])
        w = wl.int8_uniform((K, C, R, S), -128, 127, 63, *sh[1:8])
        alpha = 2.0 ** -12
        xd, wd = b.nchw_to_nc32hw32(_dev(x)), b.kcrs_to_c32rsk32(_dev(w))
        ref = oracle.epilogue_i8(oracle.conv2d_i8_points(x, w, pts, nthreads=NTHREADS, **kw), alpha)
    else:
        x = wl.normal_f32((N, C, H, W), 1.0, 64, *sh[1:8])
        w = wl.normal_f32((K, C, R, S), (C * R * S) ** -0.5, 65, *sh[1:8])
        xd, wd = _dev(x), _dev(w)
        ref = oracle.conv2d_f32_points(x, w, pts, nthreads=NTHREADS, **kw)
    ran = 0
    for cfg in range(b.num_configs(dt)):
        try:
            conv.set_config(cfg)
        except b.ConvError as e:
            if e.status != b.CONV_ERR_UNSUPPORTED:
                raise
            continue
        _announce("training shape", sh, "config", cfg)
        if dt == "int8":
            y_il = torch.full(conv.y_shape, 77, dtype=torch.int8, device="cuda")
            conv.run(xd, wd, y_il, alpha)
            y = b.nc32hw32_to_nchw(y_il).view(N, K, P, Q).cpu().numpy()
            assert np.array_equal(y[tuple(pts.T)], ref), conv.config
        else:
            yd = torch.full(conv.y_shape, float("nan"), device="cuda")
            conv.run(xd, wd, yd, 1.0)
            assert_f32_rule(yd.cpu().numpy()[tuple(pts.T)], ref)
        ran += 1
    assert ran >= 1
