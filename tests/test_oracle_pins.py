"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes the oracle to something independent: values the pages print for
a worked example (fixtures under tests/golden/, each citing its page), closed
forms computed by hand, special cases that reduce to a library routine (numpy
matmul, torch's CPU conv2d in float64), and brute force on tiny inputs.  The
set is chosen so that a dropped term, a wrong sign or index, a flipped filter
or a transposed operand in the oracle fails at least one of them (the mutation
tests in test_oracle_mutants.py check that claim).
"""
import json
import os

import numpy as np
import pytest

import oracle
from convolution_forward_gemm_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Output size
# --------------------------------------------------------------------------
def test_output_dim_worked_examples():
    g = _golden("output_dims.json")
    for c in g["cases"]:
        assert oracle.output_dim(c["in"], c["pad"], c["dil"], c["k"], c["stride"]) == c["out"]
    P, Q = oracle.output_hw(512, 512, 5, 9, pad=(2, 4), stride=1, dil=(2, 3))
    assert [8, 64, P, Q] == g["output_shape"]


def _count_positions(in_size, pad, dil, k, stride):
    # Brute force: slide the dilated window over the padded input and count
    # start positions (multiples of the stride) where the last tap still fits.
    padded = in_size + 2 * pad
    span = dil * (k - 1) + 1
    return sum(1 for start in range(0, padded, stride) if start + span <= padded)


def test_output_dim_bruteforce():
    r = np.random.default_rng(7)
    for _ in range(2000):
        in_size = int(r.integers(1, 40))
        pad = int(r.integers(0, 5))
        dil = int(r.integers(1, 5))
        k = int(r.integers(1, 8))
        stride = int(r.integers(1, 5))
        assert oracle.output_dim(in_size, pad, dil, k, stride) == \
            _count_positions(in_size, pad, dil, k, stride), (in_size, pad, dil, k, stride)


def test_output_dim_graded_shapes():
    # Hand-evaluated: 8x8, 3x3, pad 1 -> 8; 1x1 no pad -> 8; 28x28 3x3 pad 1 ->
    # 28; 56x56 3x3 stride 2 pad 1 -> floor(55/2)+1 = 28.
    assert oracle.output_hw(8, 8, 3, 3, pad=1) == (8, 8)
    assert oracle.output_hw(8, 8, 1, 1, pad=0) == (8, 8)
    assert oracle.output_hw(28, 28, 3, 3, pad=1) == (28, 28)
    assert oracle.output_hw(56, 56, 3, 3, pad=1, stride=2) == (28, 28)


# --------------------------------------------------------------------------
# Padding and dilation taps: the transcript's hand trace of output[0,0,0,0]
# --------------------------------------------------------------------------
def test_tap_trace_origin_counts():
    g = _golden("tap_trace_origin.json")
    pr = g["problem"]
    x = np.ones((1, pr["C"], pr["H"], pr["W"]), np.float32)
    w = np.ones((1, pr["C"], pr["R"], pr["S"]), np.float32)
    acc = oracle.conv2d_f32_points(x, w, [[0, 0, 0, 0]], pad=pr["pad"], dil=pr["dil"])
    assert acc[0] == pr["C"] * len(g["inside_rows"]) * len(g["inside_cols"]) == 896
    xi = np.ones((1, pr["C"], pr["H"], pr["W"]), np.int8)
    wi = np.ones((1, pr["C"], pr["R"], pr["S"]), np.int8)
    acci = oracle.conv2d_i8_points(xi, wi, [[0, 0, 0, 0]], pad=pr["pad"], dil=pr["dil"])
    assert acci[0] == 896


def test_tap_trace_origin_positions():
    # Each input pixel gets a distinct value; a one-hot filter at (kh, kw) then
    # returns the value at exactly the traced input position (or 0 if outside).
    g = _golden("tap_trace_origin.json")
    pr = g["problem"]
    H = W = 24  # enough to contain every traced tap of output (0, 0)
    x = np.zeros((1, 1, H, W), np.float32)
    for h in range(H):
        for w_ in range(W):
            x[0, 0, h, w_] = 1000 + 100 * h + w_
    for kh in range(pr["R"]):
        for kw in range(pr["S"]):
            wt = np.zeros((1, 1, pr["R"], pr["S"]), np.float32)
            wt[0, 0, kh, kw] = 1
            got = oracle.conv2d_f32_points(x, wt, [[0, 0, 0, 0]], pad=pr["pad"], dil=pr["dil"])[0]
            ih, iw = g["row_taps"][str(kh)], g["col_taps"][str(kw)]
            inside = kh in g["inside_rows"] and kw in g["inside_cols"]
            assert inside == (0 <= ih < H and 0 <= iw < W)
            assert got == (1000 + 100 * ih + iw if inside else 0), (kh, kw)


def test_interior_region():
    g = _golden("interior_region.json")
    pr = g["problem"]
    C = 32
    x = np.ones((1, C, pr["H"], pr["W"]), np.float32)
    w = np.ones((1, C, pr["R"], pr["S"]), np.float32)
    acc = oracle.conv2d_f32_acc(x, w, pad=pr["pad"], dil=pr["dil"])[0, 0]
    full = C * pr["R"] * pr["S"]
    assert acc.size == g["total"]
    interior = acc == full
    assert int(interior.sum()) == g["interior_count"]
    assert int((~interior).sum()) == g["border_count"]
    rows = np.nonzero(interior.any(axis=1))[0]
    cols = np.nonzero(interior.any(axis=0))[0]
    assert [rows.min(), rows.max()] == g["interior_rows"]
    assert [cols.min(), cols.max()] == g["interior_cols"]
    assert acc.max() == full and acc.min() > 0


# --------------------------------------------------------------------------
# Epilogue: rounding mode, order, saturation (hand-computed)
# --------------------------------------------------------------------------
def test_rounding_c1_all_ones():
    # c1 shape (N1 C32 8x8 K32 3x3 pad 1), x = w = 1, alpha = 1/64.
    # Interior outputs see 9 taps: acc = 32*9 = 288 -> 4.5 -> rint (half to
    # even) 4; edges 6 taps: 192 -> 3; corners 4 taps: 128 -> 2.
    x = np.ones((1, 32, 8, 8), np.int8)
    w = np.ones((32, 32, 3, 3), np.int8)
    acc, y = oracle.conv2d_i8(x, w, 2.0 ** -6, pad=1)
    for k in range(32):
        a = acc[0, k]
        assert (a == 288).sum() == 36 and (a == 192).sum() == 24 and (a == 128).sum() == 4
        assert a[0, 0] == 128 and a[0, 3] == 192 and a[3, 3] == 288
        yk = y[0, k]
        assert (yk == 4).sum() == 36 and (yk == 3).sum() == 24 and (yk == 2).sum() == 4


@pytest.mark.parametrize("acc,alpha,expect", [
    (2088960, 2.0 ** -14, 127),      # 127.5 -> rint 128 -> clamp 127
    (-2105344, 2.0 ** -14, -128),    # -128.5 -> rint -128 (tie to even)
    (2072576, 2.0 ** -14, 126),      # 126.5 -> 126 (tie to even)
    (2056192, 2.0 ** -14, 126),      # 125.5 -> 126 (tie to even)
    (8192, 2.0 ** -14, 0),           # 0.5 -> 0
    (24576, 2.0 ** -14, 2),          # 1.5 -> 2
    (40960, 2.0 ** -14, 2),          # 2.5 -> 2
    (-8192, 2.0 ** -14, 0),          # -0.5 -> -0 -> 0
    (-24576, 2.0 ** -14, -2),        # -1.5 -> -2
    (8193, 2.0 ** -14, 1),           # just above a tie rounds up
    (37161216, 2.0 ** -14, 127),     # 2304*127*127 saturates
    (-37453824, 2.0 ** -14, -128),   # 2304*127*(-128) saturates
    (2 ** 31 - 1, 1.0, 127),
    (-2 ** 31, 1.0, -128),
    (288, 2.0 ** -6, 4),             # 4.5 -> 4
    (96, 2.0 ** -6, 2),              # 1.5 -> 2
    (16777217, 2.0 ** -24, 1),       # (float)16777217 = 16777216 (RNE) -> 1.0 -> 1
    (50331651, 2.0 ** -24, 3),       # (float) rounds to 50331652 -> 3.0000002 -> 3
    (100, 0.1, 10),                  # fl32(100 * fl32(0.1)) = 10.0 -> 10
    # fl32(0.1) = 0.100000001490116; 25 * that = 2.50000003725, whose nearest
    # float is 2.5 exactly (ulp 2.4e-7 there), so the single fp32 multiply
    # lands on a tie and rint gives 2 (half to even).
    (25, 0.1, 2),
    # fl32(0.3) = 0.300000011920928955078125; -375 * that = -112.50000447...,
    # nearest float -112.50000763 (ulp 7.6e-6 there), rint -> -113.  Dividing
    # by fl32(1/fl32(0.3)) = 3.33333325386 instead gives -112.5000016 ->
    # -112.5 -> -112: this case separates "times alpha" from "over 1/alpha".
    (-375, 0.3, -113),
])
def test_epilogue_hand_values(acc, alpha, expect):
    y = oracle.epilogue_i8(np.array([acc], np.int64), alpha)
    assert int(y[0]) == expect


def test_epilogue_against_numpy_float32():
    # numpy's float32 arithmetic is an independent implementation of the same
    # definition (int32 -> float32 RNE, one float32 multiply, rint, clamp).
    r = np.random.default_rng(11)
    acc = r.integers(-2 ** 31, 2 ** 31 - 1, size=200000, dtype=np.int64)
    acc[:1000] = (r.integers(-300, 300, 1000) * 2 + 1) * 2 ** 13  # ties at 2^-14
    for alpha in (2.0 ** -14, 2.0 ** -6, 2.0 ** -24, 1.0 / 3.0, 1e-5, 3.0e-9, 0.3, 0.013):
        # half the samples inside the non-saturating range of this alpha
        lim = int(min(2 ** 31 - 1, 130.0 / alpha))
        acc[100000:] = r.integers(-lim, lim, size=100000)
        y = oracle.epilogue_i8(acc, alpha)
        f = acc.astype(np.int32).astype(np.float32) * np.float32(alpha)
        ref = np.clip(np.rint(f), -128, 127).astype(np.int8)
        assert np.array_equal(y, ref), alpha


def test_epilogue_rejects_int32_overflow():
    with pytest.raises(oracle.OracleError):
        oracle.epilogue_i8(np.array([2 ** 31], np.int64), 1.0)


def test_saturation_extremes_c3_channels():
    # 256 channels, 3x3, pad 1 on a 3x3 image: the center output sees all
    # 2304 taps. x = 127, w = 127 -> 2304*16129 = 37,161,216 -> 127.
    x = np.full((1, 256, 3, 3), 127, np.int8)
    w = np.full((2, 256, 3, 3), 127, np.int8)
    acc, y = oracle.conv2d_i8(x, w, 2.0 ** -14, pad=1)
    assert acc[0, 0, 1, 1] == 37161216 and y[0, 0, 1, 1] == 127
    w[:] = -128
    acc, y = oracle.conv2d_i8(x, w, 2.0 ** -14, pad=1)
    assert acc[0, 1, 1, 1] == -37453824 and y[0, 1, 1, 1] == -128


# --------------------------------------------------------------------------
# Orientation, stride, dilation: one-hot inputs (scatter form)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("stride,dil,pad", [((1, 1), (1, 1), (1, 1)),
                                            ((2, 1), (1, 2), (0, 2)),
                                            ((3, 2), (2, 3), (3, 1))])
def test_one_hot_activation(stride, dil, pad):
    N, C, H, W, K, R, S = 2, 3, 9, 11, 4, 3, 4
    r = np.random.default_rng(5)
    w = r.integers(-128, 128, size=(K, C, R, S)).astype(np.int8)
    n0, c0, h0, w0 = 1, 2, 5, 6
    x = np.zeros((N, C, H, W), np.int8)
    x[n0, c0, h0, w0] = 1
    acc = oracle.conv2d_i8_acc(x, w, pad=pad, stride=stride, dil=dil)
    P, Q = acc.shape[2:]
    # Scatter: the single nonzero input reaches output (p, q) through tap
    # (r, s) exactly when it sits at that tap's input position.
    expect = np.zeros_like(acc)
    for p in range(P):
        for rr in range(R):
            if h0 != p * stride[0] - pad[0] + rr * dil[0]:
                continue
            for q in range(Q):
                for ss in range(S):
                    if w0 == q * stride[1] - pad[1] + ss * dil[1]:
                        expect[n0, :, p, q] += w[:, c0, rr, ss]
    assert np.array_equal(acc, expect)
    assert np.count_nonzero(acc[0]) == 0  # batch independence


# --------------------------------------------------------------------------
# Special cases that reduce to library routines
# --------------------------------------------------------------------------
def test_1x1_is_matmul():
    wk = wl.WORKLOADS["c2"]
    x, w = wl.make_inputs(wk)
    acc = oracle.conv2d_i8_acc(x, w)
    X = x.astype(np.int64).transpose(0, 2, 3, 1).reshape(-1, wk.C)      # (NHW, C)
    Wm = w.astype(np.int64).reshape(wk.K, wk.C)                          # (K, C)
    Y = (X @ Wm.T).reshape(wk.N, wk.H, wk.W, wk.K).transpose(0, 3, 1, 2)
    assert np.array_equal(acc, Y)


def _im2col_numpy(x, R, S, pad, stride, dil):
    # Explicit im2col with np.pad and strided slicing (no bounds checks):
    # column j = (c, r, s), row m = (n, p, q).
    N, C, H, W = x.shape
    ph, pw = pad
    sh, sw = stride
    dh, dw = dil
    xp = np.pad(x.astype(np.int64), ((0, 0), (0, 0), (ph, ph), (pw, pw)))
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    cols = np.empty((N, P, Q, C, R, S), np.int64)
    for rr in range(R):
        for ss in range(S):
            patch = xp[:, :, rr * dh: rr * dh + sh * (P - 1) + 1: sh,
                       ss * dw: ss * dw + sw * (Q - 1) + 1: sw]            # (N, C, P, Q)
            cols[:, :, :, :, rr, ss] = patch.transpose(0, 2, 3, 1)
    return cols.reshape(N * P * Q, C * R * S), (N, P, Q)


@pytest.mark.parametrize("seed", range(12))
def test_implicit_equals_explicit_im2col(seed):
    r = np.random.default_rng(100 + seed)
    N, C, K = int(r.integers(1, 3)), int(r.integers(1, 5)), int(r.integers(1, 6))
    R, S = int(r.integers(1, 6)), int(r.integers(1, 6))
    pad = (int(r.integers(0, 4)), int(r.integers(0, 4)))
    stride = (int(r.integers(1, 4)), int(r.integers(1, 4)))
    dil = (int(r.integers(1, 4)), int(r.integers(1, 4)))
    H = int(r.integers(1, 8)) + max(0, dil[0] * (R - 1) + 1 - 2 * pad[0])
    W = int(r.integers(1, 8)) + max(0, dil[1] * (S - 1) + 1 - 2 * pad[1])
    x = r.integers(-128, 128, size=(N, C, H, W)).astype(np.int8)
    w = r.integers(-128, 128, size=(K, C, R, S)).astype(np.int8)
    acc = oracle.conv2d_i8_acc(x, w, pad=pad, stride=stride, dil=dil)
    A, (n_, P, Q) = _im2col_numpy(x, R, S, pad, stride, dil)
    B = w.astype(np.int64).reshape(K, C * R * S).T                          # (CRS, K)
    Y = (A @ B).reshape(n_, P, Q, K).transpose(0, 3, 1, 2)
    assert np.array_equal(acc, Y)


def _torch_conv_f64(x, w, pad, stride, dil):
    import torch
    out = torch.nn.functional.conv2d(torch.from_numpy(np.asarray(x, np.float64)),
                                     torch.from_numpy(np.asarray(w, np.float64)),
                                     stride=stride, padding=pad, dilation=dil)
    return out.numpy()


def _random_shape(r):
    R, S = int(r.integers(1, 6)), int(r.integers(1, 6))
    dil = (int(r.integers(1, 4)), int(r.integers(1, 4)))
    stride = (int(r.integers(1, 4)), int(r.integers(1, 4)))
    pad = (int(r.integers(0, 4)), int(r.integers(0, 4)))
    # smallest extent with at least one output, plus a random margin
    H = int(r.integers(0, 9)) + max(1, dil[0] * (R - 1) + 1 - 2 * pad[0])
    W = int(r.integers(0, 9)) + max(1, dil[1] * (S - 1) + 1 - 2 * pad[1])
    return H, W, R, S, pad, stride, dil


@pytest.mark.parametrize("seed", range(20))
def test_int8_matches_torch_f64(seed):
    # All partial sums are below 2^53, so the float64 library conv is exact.
    r = np.random.default_rng(200 + seed)
    N, C, K = int(r.integers(1, 3)), int(r.choice([32, 64])), int(r.integers(1, 5))
    H, W, R, S, pad, stride, dil = _random_shape(r)
    x = r.integers(-128, 128, size=(N, C, H, W)).astype(np.int8)
    w = r.integers(-128, 128, size=(K, C, R, S)).astype(np.int8)
    acc = oracle.conv2d_i8_acc(x, w, pad=pad, stride=stride, dil=dil)
    ref = _torch_conv_f64(x, w, pad, stride, dil)
    assert np.array_equal(acc, ref.astype(np.int64))


@pytest.mark.parametrize("seed", range(10))
def test_f32_matches_torch_f64(seed):
    r = np.random.default_rng(300 + seed)
    N, C, K = int(r.integers(1, 3)), int(r.integers(1, 6)), int(r.integers(1, 5))
    H, W, R, S, pad, stride, dil = _random_shape(r)
    x = r.standard_normal((N, C, H, W)).astype(np.float32)
    w = r.standard_normal((K, C, R, S)).astype(np.float32)
    acc = oracle.conv2d_f32_acc(x, w, pad=pad, stride=stride, dil=dil)
    ref = _torch_conv_f64(x, w, pad, stride, dil)
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-12)


def test_f32_integer_valued_exact_and_equal_to_int8_path():
    # Inputs in {-1, 0, 1}: every partial sum is an exact small integer, so the
    # fp32 oracle, the int8 oracle and the float64 library conv agree exactly.
    r = np.random.default_rng(17)
    N, C, H, W, K, R, S = 2, 32, 13, 17, 6, 5, 9
    pad, stride, dil = (2, 4), (1, 1), (2, 3)
    xi = r.integers(-1, 2, size=(N, C, H, W)).astype(np.int8)
    wi = r.integers(-1, 2, size=(K, C, R, S)).astype(np.int8)
    acc_f, y_f = oracle.conv2d_f32(xi.astype(np.float32), wi.astype(np.float32),
                                   1.0, pad=pad, stride=stride, dil=dil)
    acc_i = oracle.conv2d_i8_acc(xi, wi, pad=pad, stride=stride, dil=dil)
    assert np.array_equal(acc_f, acc_i.astype(np.float64))
    assert np.array_equal(y_f, acc_i.astype(np.float32))
    assert np.array_equal(acc_i, _torch_conv_f64(xi, wi, pad, stride, dil).astype(np.int64))


# --------------------------------------------------------------------------
# fp32 output scale alpha: y = fl32(alpha * acc), one rounding of the exact
# product of the fp32 alpha and the double accumulator
# --------------------------------------------------------------------------
def test_f32_epilogue_alpha_hand_values():
    # Exact products (no rounding at all): 3/8 * 896 = 336, 3/8 * -7 = -2.625,
    # 3/8 * 1e6 = 375000; -5/2 * 896 = -2240, -5/2 * -7 = 17.5.
    y = oracle.epilogue_f32(np.array([896.0, -7.0, 1e6]), 0.375)
    assert y.tolist() == [336.0, -2.625, 375000.0]
    y = oracle.epilogue_f32(np.array([896.0, -7.0]), -2.5)
    assert y.tolist() == [-2240.0, 17.5]
    # One rounding, in the right place.  acc = 1 + 2^-24 + 2^-40 (exact in
    # double, between the floats 1 and 1 + 2^-23), alpha = 3:
    #   alpha * acc = 3 + 0.75 * 2^-22 + 3 * 2^-40; the floats in [2, 4) are
    #   2^-22 apart, so the nearest is 3 + 2^-22.
    # Rounding acc to fp32 first would give (1 + 2^-23) * 3 = 3 + 1.5 * 2^-22,
    # a tie between 3 + 2^-22 (odd mantissa) and 3 + 2^-21 (even): 3 + 2^-21.
    acc = 1.0 + 2.0 ** -24 + 2.0 ** -40
    y = oracle.epilogue_f32(np.array([acc, -acc]), 3.0)
    assert y.tolist() == [3.0 + 2.0 ** -22, -(3.0 + 2.0 ** -22)]
    # The same with a non-dyadic alpha: fl32(0.1) = 13421773 * 2^-27.
    # acc = 10 exactly: 10 * 13421773 * 2^-27 = 134217730 * 2^-27
    # = 1.0000000149..., whose neighbours in [1, 2) are 1 and 1 + 2^-23 =
    # 1.000000119...; the nearest is 1.0.
    y = oracle.epilogue_f32(np.array([10.0]), 0.1)
    assert y.tolist() == [1.0]


def test_f32_alpha_scales_the_tap_trace():
    # The transcript's trace of output (0,0,0,0) on all-ones data gives
    # acc = C * 4 rows * 7 columns = 896 (pinned above); with alpha = -2.5 the
    # output is -2240 exactly, and with alpha = 0.375 it is 336.
    # A 24 x 24 input holds every traced tap of output (0, 0), so that output
    # is the same as on the transcript's 512 x 512 image.
    g = _golden("tap_trace_origin.json")
    pr = g["problem"]
    x = np.ones((1, pr["C"], 24, 24), np.float32)
    w = np.ones((2, pr["C"], pr["R"], pr["S"]), np.float32)
    for alpha, expect in ((-2.5, -2240.0), (0.375, 336.0)):
        _, y = oracle.conv2d_f32(x, w, alpha, pad=pr["pad"], dil=pr["dil"])
        assert y[0, 0, 0, 0] == expect and y[0, 1, 0, 0] == expect


# --------------------------------------------------------------------------
# Metamorphic properties
# --------------------------------------------------------------------------
def test_linearity_in_w_and_k_permutation():
    r = np.random.default_rng(23)
    x = r.integers(-128, 128, size=(2, 32, 7, 6)).astype(np.int8)
    w1 = r.integers(-64, 64, size=(5, 32, 3, 2)).astype(np.int8)
    w2 = r.integers(-64, 64, size=(5, 32, 3, 2)).astype(np.int8)
    kw = dict(pad=(1, 2), stride=(2, 1), dil=(1, 2))
    a1 = oracle.conv2d_i8_acc(x, w1, **kw)
    a2 = oracle.conv2d_i8_acc(x, w2, **kw)
    a12 = oracle.conv2d_i8_acc(x, (w1.astype(np.int16) + w2).astype(np.int8), **kw)
    assert np.array_equal(a12, a1 + a2)
    perm = r.permutation(5)
    assert np.array_equal(oracle.conv2d_i8_acc(x, w1[perm], **kw), a1[:, perm])
    # batch independence: image 1 alone gives the same rows
    assert np.array_equal(oracle.conv2d_i8_acc(x[1:], w1, **kw), a1[1:])


def test_points_equal_full_and_threads_equal_serial():
    wk = wl.WORKLOADS["c1"]
    x, w = wl.make_inputs(wk)
    acc1 = oracle.conv2d_i8_acc(x, w, **wk.conv_kwargs, nthreads=1)
    accn = oracle.conv2d_i8_acc(x, w, **wk.conv_kwargs, nthreads=4)
    assert np.array_equal(acc1, accn)
    r = np.random.default_rng(3)
    pts = np.stack([r.integers(0, s, 300) for s in acc1.shape], axis=1)
    got = oracle.conv2d_i8_points(x, w, pts, **wk.conv_kwargs, nthreads=3)
    assert np.array_equal(got, acc1[tuple(pts.T)])
    xf = r.standard_normal((1, 3, 9, 8)).astype(np.float32)
    wf = r.standard_normal((2, 3, 2, 3)).astype(np.float32)
    af = oracle.conv2d_f32_acc(xf, wf, pad=1, dil=(2, 1))
    assert np.array_equal(af, oracle.conv2d_f32_acc(xf, wf, pad=1, dil=(2, 1), nthreads=4))
    pts = np.stack([r.integers(0, s, 50) for s in af.shape], axis=1)
    assert np.array_equal(oracle.conv2d_f32_points(xf, wf, pts, pad=1, dil=(2, 1)),
                          af[tuple(pts.T)])


def test_oracle_rejects_empty_output():
    x = np.zeros((1, 32, 2, 2), np.int8)
    w = np.zeros((1, 32, 5, 5), np.int8)
    with pytest.raises(oracle.OracleError):
        oracle.conv2d_i8_acc(x, w)
    assert oracle.output_dim(2, 0, 1, 5, 1) == 0


# --------------------------------------------------------------------------
# Interleaved layout maps
# --------------------------------------------------------------------------
def test_nc32hw32_hand_listed():
    # N=1, C=64, H=1, W=2 with x[c][w] = 2*c + w (mod 128).  Reading of the
    # name NCxHWx<32>: the 32 channels of a pixel are innermost, then W, then
    # H, then the 32-channel group.  So the buffer is
    #   group 0: pixel w=0 channels 0..31, pixel w=1 channels 0..31,
    #   group 1: pixel w=0 channels 32..63, pixel w=1 channels 32..63.
    x = np.zeros((1, 64, 1, 2), np.int8)
    for c in range(64):
        for w_ in range(2):
            x[0, c, 0, w_] = (2 * c + w_) % 128
    expect = []
    for g in range(2):
        for w_ in range(2):
            for ci in range(32):
                expect.append((2 * (32 * g + ci) + w_) % 128)
    got = oracle.nchw_to_nc32hw32(x).ravel()
    assert got.tolist() == expect
    assert np.array_equal(oracle.nc32hw32_to_nchw(got, 1, 64, 1, 2), x)


def test_c32rsk32_hand_listed():
    # K=2, C=64, R=1, S=2 with w[k][c][0][s] = k*100 + c + 3*s (mod 128, as
    # int8).  CxRSKx<32>: 32 input channels innermost, then K, then S, then R,
    # then the 32-channel group.
    K, C, R, S = 2, 64, 1, 2
    w = np.zeros((K, C, R, S), np.int8)
    for k in range(K):
        for c in range(C):
            for s in range(S):
                w[k, c, 0, s] = np.int8((k * 100 + c + 3 * s) % 128)
    expect = []
    for g in range(2):
        for s in range(S):
            for k in range(K):
                for ci in range(32):
                    expect.append((k * 100 + 32 * g + ci + 3 * s) % 128)
    got = oracle.kcrs_to_c32rsk32(w).ravel()
    assert got.tolist() == expect
    assert np.array_equal(oracle.c32rsk32_to_kcrs(got, K, C, R, S), w)


def test_layout_maps_match_numpy_reshape():
    r = np.random.default_rng(9)
    x = r.integers(-128, 128, size=(3, 96, 5, 7)).astype(np.int8)
    il = oracle.nchw_to_nc32hw32(x)
    ref = x.reshape(3, 3, 32, 5, 7).transpose(0, 1, 3, 4, 2)
    assert np.array_equal(il, ref)
    assert np.array_equal(oracle.nc32hw32_to_nchw(il, 3, 96, 5, 7), x)
    w = r.integers(-128, 128, size=(40, 64, 3, 2)).astype(np.int8)
    wil = oracle.kcrs_to_c32rsk32(w)
    wref = w.reshape(40, 2, 32, 3, 2).transpose(1, 3, 4, 0, 2)
    assert np.array_equal(wil, wref)
    assert np.array_equal(oracle.c32rsk32_to_kcrs(wil, 40, 64, 3, 2), w)


def test_layout_rejects_non_multiple_of_32():
    with pytest.raises(oracle.OracleError):
        oracle.nchw_to_nc32hw32(np.zeros((1, 48, 2, 2), np.int8))


# --------------------------------------------------------------------------
# Per-output-channel scale and bias (the "rowwise scaled" epilogue variant):
# y = clamp(rint(fl32(fl32(fl32(acc) * alpha[k]) + bias[k])), -128, 127).
# Expected values are worked by hand below.
# --------------------------------------------------------------------------
def test_per_channel_hand_values():
    acc = np.array([64, 96], np.int64).reshape(1, 2, 1, 1)
    # channel 0: 64 * 0.5 = 32, + 0.25 = 32.25 -> 32
    # channel 1: 96 * 0.25 = 24, - 0.5 = 23.5 -> 24 (tie to even)
    assert oracle.epilogue_i8_per_channel(acc, [0.5, 0.25], [0.25, -0.5]).ravel().tolist() == [32, 24]
    # swapped per-channel values must move with their channel:
    # channel 0: 64 * 0.25 = 16, - 0.5 = 15.5 -> 16; channel 1: 96 * 0.5 + 0.25 = 48.25 -> 48
    assert oracle.epilogue_i8_per_channel(acc, [0.25, 0.5], [-0.5, 0.25]).ravel().tolist() == [16, 48]
    # no bias: the scale alone
    assert oracle.epilogue_i8_per_channel(acc, [0.5, 0.25]).ravel().tolist() == [32, 24]
    # saturation through the bias
    one = np.ones((1, 2, 1, 1), np.int64)
    assert oracle.epilogue_i8_per_channel(one, [1.0, 1.0], [200.0, -300.0]).ravel().tolist() == [127, -128]


def test_per_channel_multiply_then_add_rounds_twice():
    # fl32(1/7) = 0.14285714924335479736328125; 7 * that = 1 + 0.75 * 2**-24,
    # which rounds to 1.0 in fp32 (a quarter ulp below the midpoint); 1.0 - 0.5
    # = 0.5 -> rint 0.  A fused multiply-add would round 0.5 + 0.75 * 2**-24
    # once, to 0.5 + 2**-24, and give 1.
    acc = np.array([7], np.int64).reshape(1, 1, 1, 1)
    a = float(np.float32(1.0 / 7.0))
    assert a == 0.14285714924335479736328125
    assert oracle.epilogue_i8_per_channel(acc, [a], [-0.5]).ravel().tolist() == [0]


def test_per_channel_c1_all_ones_with_bias():
    # c1 with x = w = 1: acc 288 (interior, 36 per plane), 192 (edge, 24),
    # 128 (corner, 4); alpha = 1/64 gives 4.5, 3, 2.  Bias by channel k % 3:
    #   +0.25: 4.75 -> 5, 3.25 -> 3, 2.25 -> 2
    #   -0.5 : 4.0  -> 4, 2.5  -> 2, 1.5  -> 2
    #   +0.5 : 5.0  -> 5, 3.5  -> 4, 2.5  -> 2
    x = np.ones((1, 32, 8, 8), np.int8)
    w = np.ones((32, 32, 3, 3), np.int8)
    bias = np.array([(0.25, -0.5, 0.5)[k % 3] for k in range(32)], np.float32)
    acc, y = oracle.conv2d_i8_scaled(x, w, np.full(32, 2.0 ** -6, np.float32), bias, pad=1)
    expect = {0: (5, 3, 2), 1: (4, 2, 2), 2: (5, 4, 2)}
    for k in range(32):
        yi, ye, yc = expect[k % 3]
        yk = y[0, k]
        assert yk[3, 3] == yi and yk[0, 3] == ye and yk[0, 0] == yc
        vals, counts = np.unique(yk, return_counts=True)
        want = {}
        for v, c in ((yi, 36), (ye, 24), (yc, 4)):
            want[v] = want.get(v, 0) + c
        assert dict(zip(vals.tolist(), counts.tolist())) == want


def test_per_channel_with_one_scale_is_the_scalar_epilogue():
    # every channel with the same alpha and no bias reduces to the pinned
    # scalar epilogue
    r = np.random.default_rng(11)
    acc = r.integers(-2 ** 26, 2 ** 26, size=(2, 5, 3, 4), dtype=np.int64)
    for alpha in (2.0 ** -14, 0.1, 1.0 / 3.0):
        a = np.full(5, alpha, np.float32)
        assert np.array_equal(oracle.epilogue_i8_per_channel(acc, a), oracle.epilogue_i8(acc, alpha))


def test_f32_per_channel_hand_values():
    acc = np.array([3.0, -5.0, 7.0, 11.0], np.float64).reshape(1, 2, 1, 2)
    # channel 0: 0.5 * 3 + 0.25 = 1.75, 0.5 * -5 + 0.25 = -2.25
    # channel 1: -2 * 7 + 1 = -13, -2 * 11 + 1 = -21
    y = oracle.epilogue_f32_per_channel(acc, [0.5, -2.0], [0.25, 1.0])
    assert y.ravel().tolist() == [1.75, -2.25, -13.0, -21.0]
