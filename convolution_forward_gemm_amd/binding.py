"""Thin ctypes binding of libconvfprop.so (declared in include/convfprop.h).

Argument marshalling only: every step of the convolution runs in the HIP
kernels behind the C ABI.  PyTorch is used for device memory and streams; the
binding passes ``tensor.data_ptr()`` and the current stream's handle.

Importing this module loads the library and raises ``ImportError`` if it has
not been built (``python -m convolution_forward_gemm_amd.build``).  There is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libconvfprop.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError("libconvfprop.so is not built (%s); run "
                      "`python -m convolution_forward_gemm_amd.build`" % _LIB_PATH)

lib = ctypes.CDLL(_LIB_PATH)

# conv_status_t
CONV_OK = 0
CONV_ERR_NULL = 1
CONV_ERR_INVALID_SHAPE = 2
CONV_ERR_UNSUPPORTED = 3
CONV_ERR_MISALIGNED = 4
CONV_ERR_OVERFLOW_RISK = 5
CONV_ERR_HIP = 6
CONV_ERR_NO_MEMORY = 7
CONV_ERR_INVALID_ALPHA = 8

# conv_dtype_t / conv_layout_t
CONV_DTYPE_INT8 = 0
CONV_DTYPE_FP32 = 1
CONV_LAYOUT_NCHW_KCRS = 0
CONV_LAYOUT_NC32HW32_C32RSK32 = 1

_i, _p, _f, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t

# Every symbol the header declares, with its ctypes signature.
SIGNATURES = {
    "conv2d_fprop_desc_create": (_i, [ctypes.POINTER(_p)] + [_i] * 13 + [_i, _i]),
    "conv2d_fprop_desc_destroy": (_i, [_p]),
    "conv2d_fprop_desc_get_output_dims": (_i, [_p, ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "conv2d_fprop_desc_get_config": (_i, [_p, ctypes.c_char_p, _sz]),
    "conv2d_fprop_num_configs": (_i, [_i]),
    "conv2d_fprop_desc_set_config": (_i, [_p, _i]),
    "conv2d_fprop_run": (_i, [_p, _p, _p, _p, _f, _p]),
    "conv2d_fprop_run_scaled": (_i, [_p, _p, _p, _p, _p, _p, _p]),
    "conv2d_fprop_graph_create": (_i, [ctypes.POINTER(_p), _p, _p, _p, _p, _f, _i]),
    "conv2d_fprop_graph_launch": (_i, [_p, _p]),
    "conv2d_fprop_graph_destroy": (_i, [_p]),
    "conv_nchw_to_nc32hw32_i8": (_i, [_p, _p, _i, _i, _i, _i, _p]),
    "conv_nc32hw32_to_nchw_i8": (_i, [_p, _p, _i, _i, _i, _i, _p]),
    "conv_kcrs_to_c32rsk32_i8": (_i, [_p, _p, _i, _i, _i, _i, _p]),
    "conv_c32rsk32_to_kcrs_i8": (_i, [_p, _p, _i, _i, _i, _i, _p]),
    "conv_status_string": (ctypes.c_char_p, [_i]),
}
for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class ConvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s" % (what, status_string(status)))


def status_string(status: int) -> str:
    return lib.conv_status_string(status).decode()


def _check(status: int, what: str):
    if status != CONV_OK:
        raise ConvError(status, what)


def _pair(v):
    if isinstance(v, int):
        return v, v
    return int(v[0]), int(v[1])


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Conv2dFprop:
    """A convolution problem bound to its compiled kernel configuration.

    ``dtype`` is "int8" (interleaved NCxHWx<32> / CxRSKx<32>) or "fp32"
    (NCHW / KCRS).  Creating the object validates the problem once; ``run``
    then checks tensors and launches, and ``run_ptr`` launches on raw device
    pointers with no Python-side checks.
    """

    def __init__(self, N, C, H, W, K, R, S, pad=0, stride=1, dil=1, dtype="int8"):
        self.N, self.C, self.H, self.W, self.K, self.R, self.S = N, C, H, W, K, R, S
        self.pad, self.stride, self.dil = _pair(pad), _pair(stride), _pair(dil)
        if dtype == "int8":
            dt, lay = CONV_DTYPE_INT8, CONV_LAYOUT_NC32HW32_C32RSK32
        elif dtype == "fp32":
            dt, lay = CONV_DTYPE_FP32, CONV_LAYOUT_NCHW_KCRS
        else:
            raise ValueError("dtype must be 'int8' or 'fp32'")
        self.dtype = dtype
        h = ctypes.c_void_p()
        _check(lib.conv2d_fprop_desc_create(
            ctypes.byref(h), N, C, H, W, K, R, S, self.pad[0], self.pad[1],
            self.stride[0], self.stride[1], self.dil[0], self.dil[1], dt, lay),
            "conv2d_fprop_desc_create")
        self._h = h
        P, Q = ctypes.c_int(), ctypes.c_int()
        _check(lib.conv2d_fprop_desc_get_output_dims(h, ctypes.byref(P), ctypes.byref(Q)),
               "get_output_dims")
        self.P, self.Q = P.value, Q.value

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and lib is not None:  # lib is None at interpreter exit
            lib.conv2d_fprop_desc_destroy(h)
            self._h = None

    @property
    def config(self) -> str:
        buf = ctypes.create_string_buffer(256)
        _check(lib.conv2d_fprop_desc_get_config(self._h, buf, 256), "get_config")
        return buf.value.decode()

    def set_config(self, index: int):
        _check(lib.conv2d_fprop_desc_set_config(self._h, index), "set_config")

    @property
    def x_shape(self):
        if self.dtype == "int8":
            return (self.N, self.C // 32, self.H, self.W, 32)
        return (self.N, self.C, self.H, self.W)

    @property
    def w_shape(self):
        if self.dtype == "int8":
            return (self.C // 32, self.R, self.S, self.K, 32)
        return (self.K, self.C, self.R, self.S)

    @property
    def y_shape(self):
        if self.dtype == "int8":
            return (self.N, self.K // 32, self.P, self.Q, 32)
        return (self.N, self.K, self.P, self.Q)

    def run_ptr(self, x_ptr: int, w_ptr: int, y_ptr: int, alpha: float, stream_handle: int = 0):
        """Launch on raw device pointers (no Python-side checks)."""
        _check(lib.conv2d_fprop_run(self._h, x_ptr, w_ptr, y_ptr, alpha, stream_handle),
               "conv2d_fprop_run")

    def run_scaled_ptr(self, x_ptr: int, w_ptr: int, y_ptr: int, alpha_ptr: int, bias_ptr,
                       stream_handle: int = 0):
        """Per-output-channel scale (and bias, or None) on raw device pointers."""
        _check(lib.conv2d_fprop_run_scaled(self._h, x_ptr, w_ptr, y_ptr, alpha_ptr, bias_ptr,
                                           stream_handle), "conv2d_fprop_run_scaled")

    def run_scaled(self, x, w, alpha, bias=None, y=None, stream=None):
        """y <- conv(x, w) with alpha[k] and bias[k] per output channel:
        contiguous float32 CUDA tensors of K values (bias may be None)."""
        import torch
        for name, t in (("alpha", alpha), ("bias", bias)):
            if t is None and name == "bias":
                continue
            if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or t.numel() != self.K:
                raise ValueError("%s must be a contiguous float32 CUDA tensor of %d values" % (name, self.K))
        tdt = torch.int8 if self.dtype == "int8" else torch.float32
        for name, t, shape in (("x", x, self.x_shape), ("w", w, self.w_shape)):
            if t.dtype != tdt or not t.is_cuda or not t.is_contiguous() or t.numel() != _prod(shape):
                raise ValueError("%s must be a contiguous %s CUDA tensor with %d elements"
                                 % (name, tdt, _prod(shape)))
        if y is None:
            y = torch.empty(self.y_shape, dtype=tdt, device=x.device)
        elif y.dtype != tdt or not y.is_cuda or not y.is_contiguous() or y.numel() != _prod(self.y_shape):
            raise ValueError("y must be a contiguous %s CUDA tensor of shape %s" % (tdt, self.y_shape))
        self.run_scaled_ptr(x.data_ptr(), w.data_ptr(), y.data_ptr(), alpha.data_ptr(),
                            bias.data_ptr() if bias is not None else None, _stream_handle(stream))
        return y

    def run(self, x, w, y=None, alpha: float = 1.0, stream=None):
        """y <- conv(x, w) on the GPU.  Tensors are torch CUDA tensors in the
        descriptor's layouts; y is allocated if not given.  Returns y."""
        import torch
        tdt = torch.int8 if self.dtype == "int8" else torch.float32
        for name, t, shape in (("x", x, self.x_shape), ("w", w, self.w_shape)):
            if t.dtype != tdt or not t.is_cuda or not t.is_contiguous() or t.numel() != _prod(shape):
                raise ValueError("%s must be a contiguous %s CUDA tensor with %d elements"
                                 % (name, tdt, _prod(shape)))
        if y is None:
            y = torch.empty(self.y_shape, dtype=tdt, device=x.device)
        elif y.dtype != tdt or not y.is_cuda or not y.is_contiguous() or y.numel() != _prod(self.y_shape):
            raise ValueError("y must be a contiguous %s CUDA tensor of shape %s" % (tdt, self.y_shape))
        self.run_ptr(x.data_ptr(), w.data_ptr(), y.data_ptr(), float(alpha),
                     _stream_handle(stream))
        return y


class ConvGraph:
    """`calls` back-to-back runs of a descriptor on fixed device buffers,
    captured once into a HIP graph by the library; launch() replays them."""

    def __init__(self, conv: "Conv2dFprop", x_ptr: int, w_ptr: int, y_ptr: int, alpha: float,
                 calls: int):
        self._h = None
        h = _p()
        _check(lib.conv2d_fprop_graph_create(ctypes.byref(h), conv._h, x_ptr, w_ptr, y_ptr,
                                             alpha, calls), "conv2d_fprop_graph_create")
        self._h = h
        self._conv = conv  # the descriptor outlives the graph
        self.calls = calls

    def launch(self, stream_handle: int = 0):
        _check(lib.conv2d_fprop_graph_launch(self._h, stream_handle), "conv2d_fprop_graph_launch")

    def __del__(self):
        if getattr(self, "_h", None) is not None and lib is not None:
            lib.conv2d_fprop_graph_destroy(self._h)
            self._h = None


def _prod(shape):
    r = 1
    for s in shape:
        r *= int(s)
    return r


def num_configs(dtype: str) -> int:
    return lib.conv2d_fprop_num_configs(CONV_DTYPE_INT8 if dtype == "int8" else CONV_DTYPE_FP32)


def _transform(fn, src, dst_shape, dims, stream):
    import torch
    if src.dtype != torch.int8 or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous int8 CUDA tensor")
    dst = torch.empty(dst_shape, dtype=torch.int8, device=src.device)
    _check(fn(src.data_ptr(), dst.data_ptr(), *dims, _stream_handle(stream)), fn.__name__)
    return dst


def nchw_to_nc32hw32(x, stream=None):
    """int8 NCHW (N, C, H, W) -> NCxHWx<32> (N, C/32, H, W, 32) on the GPU."""
    N, C, H, W = x.shape
    return _transform(lib.conv_nchw_to_nc32hw32_i8, x, (N, C // 32, H, W, 32), (N, C, H, W), stream)


def nc32hw32_to_nchw(x_il, stream=None):
    """int8 NCxHWx<32> (N, C/32, H, W, 32) -> NCHW (N, C, H, W) on the GPU."""
    N, CB, H, W, _ = x_il.shape
    return _transform(lib.conv_nc32hw32_to_nchw_i8, x_il, (N, CB * 32, H, W), (N, CB * 32, H, W), stream)


def kcrs_to_c32rsk32(w, stream=None):
    """int8 KCRS (K, C, R, S) -> CxRSKx<32> (C/32, R, S, K, 32) on the GPU."""
    K, C, R, S = w.shape
    return _transform(lib.conv_kcrs_to_c32rsk32_i8, w, (C // 32, R, S, K, 32), (K, C, R, S), stream)


def c32rsk32_to_kcrs(w_il, stream=None):
    """int8 CxRSKx<32> (C/32, R, S, K, 32) -> KCRS (K, C, R, S) on the GPU."""
    CB, R, S, K, _ = w_il.shape
    return _transform(lib.conv_c32rsk32_to_kcrs_i8, w_il, (K, CB * 32, R, S), (K, CB * 32, R, S), stream)
