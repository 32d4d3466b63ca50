"""MI355X (gfx950) 2-D convolution forward: thin Python binding of libconvfwd.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/conv.h.  The names mirror the C
calls (conv_output_extent, conv_resolve_auto_pad, conv_scratch_size,
conv_describe_variant, conv_forward, conv_transpose_forward).  Loading fails
loudly when the native library has not been built; there is no fallback.

Operands are device pointers (ints) or objects with a ``data_ptr()`` method
(torch tensors on the GPU).  PyTorch is only used by callers for device memory
and streams.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libconvfwd.so")

# enums of include/conv.h
CONV_OK, CONV_ERR_ARG, CONV_ERR_SHAPE, CONV_ERR_OVERLAP, CONV_ERR_SCRATCH, CONV_ERR_DEVICE = range(6)
CONV_F32, CONV_F16, CONV_BF16 = 0, 1, 2
DTYPES = {"f32": CONV_F32, "f16": CONV_F16, "bf16": CONV_BF16}
ACTIVATIONS = {
    "identity": 0, "relu": 1, "tanh": 2, "sigmoid": 3, "silu": 4,
    "hard_sigmoid": 5, "hard_swish": 6, "clip": 7, "leaky_relu": 8,
}
AUTO_PAD = {"NOTSET": 0, "SAME_UPPER": 1, "SAME_LOWER": 2, "VALID": 3}
VARIANTS = {
    "auto": 0, "implicit_gemm": 1, "pointwise_gemm": 2, "depthwise_direct": 3,
    "transpose_gemm_col2im": 4, "implicit_gemm_halo": 5, "implicit_gemm_rowband": 6,
    "implicit_gemm_grouped": 7, "winograd": 8,
}
# default activation parameters (ONNX): hard_sigmoid alpha/beta, leaky alpha
ACT_DEFAULTS = {"hard_sigmoid": (0.2, 0.5), "leaky_relu": (0.01, 0.0)}

EXPORTS = (
    "conv_output_extent", "conv_resolve_auto_pad", "conv_scratch_size",
    "conv_describe_variant", "conv_forward", "conv_transpose_forward",
    "conv_check", "conv_status_string", "conv_forward_noalloc",
    "pool_output_extent", "pool_resolve_auto_pad", "pool_describe_variant", "pool_check",
    "pool_forward", "conv_integer_describe_variant", "conv_integer_check", "conv_integer_forward",
)


class ConvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class conv_problem(ctypes.Structure):
    """Mirror of struct conv_problem in include/conv.h (same field order)."""

    _fields_ = [(n, ctypes.c_int64) for n in (
        "n", "c_in", "h", "w", "c_out", "kh", "kw", "groups",
        "stride_h", "stride_w", "dil_h", "dil_w",
        "pad_top", "pad_left", "pad_bottom", "pad_right",
        "out_pad_h", "out_pad_w",
        "x_off", "w_off", "b_off", "r_off", "y_off")] + [
        ("transpose", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("act_alpha", ctypes.c_float), ("act_beta", ctypes.c_float),
        ("has_bias", ctypes.c_int32), ("has_residual", ctypes.c_int32),
        ("variant_override", ctypes.c_int32), ("split_override", ctypes.c_int32)]


class pool_problem(ctypes.Structure):
    """Mirror of struct pool_problem in include/pool.h (same field order)."""

    _fields_ = [(n, ctypes.c_int64) for n in (
        "n", "c", "h", "w", "kh", "kw", "stride_h", "stride_w", "dil_h", "dil_w",
        "pad_top", "pad_left", "pad_bottom", "pad_right", "x_off", "y_off")] + [
        ("kind", ctypes.c_int32), ("ceil_mode", ctypes.c_int32),
        ("count_include_pad", ctypes.c_int32), ("reserved", ctypes.c_int32)]


POOL_KINDS = {"max": 0, "average": 1, "global_max": 2, "global_average": 3}

_lib = None


def lib():
    """The loaded native library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with convolution_forward_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(conv_problem)
        i64p = ctypes.POINTER(ctypes.c_int64)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        vp = ctypes.c_void_p
        L.conv_output_extent.argtypes = [P, i64p, i64p]
        L.conv_resolve_auto_pad.argtypes = [P, ctypes.c_int, i64p]
        L.conv_scratch_size.argtypes = [P, ctypes.c_int, u64p, u64p]
        L.conv_describe_variant.argtypes = [P, ctypes.c_int, ctypes.c_char_p, ctypes.c_uint64]
        fwd = [P, ctypes.c_int, vp, vp, vp, vp, vp, vp, ctypes.c_uint64, vp]
        L.conv_forward.argtypes = fwd
        L.conv_transpose_forward.argtypes = fwd
        L.conv_check.argtypes = [P, ctypes.c_int, vp, vp, vp, vp, vp, vp, ctypes.c_uint64]
        L.conv_forward_noalloc.argtypes = [P, ctypes.c_int, vp, vp, vp, vp, vp, vp]
        PP = ctypes.POINTER(pool_problem)
        L.pool_output_extent.argtypes = [PP, i64p, i64p]
        L.pool_resolve_auto_pad.argtypes = [PP, ctypes.c_int]
        L.pool_describe_variant.argtypes = [PP, ctypes.c_int, ctypes.c_char_p, ctypes.c_uint64]
        L.pool_check.argtypes = [PP, ctypes.c_int, vp, vp]
        L.pool_forward.argtypes = [PP, ctypes.c_int, vp, vp, vp]
        L.conv_integer_describe_variant.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_char_p,
                                                    ctypes.c_uint64]
        L.conv_integer_check.argtypes = [P, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp,
                                         ctypes.c_int, vp]
        L.conv_integer_forward.argtypes = [P, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp,
                                           ctypes.c_int, vp, vp]
        L.conv_status_string.argtypes = [ctypes.c_int]
        L.conv_status_string.restype = ctypes.c_char_p
        for name in EXPORTS:
            getattr(L, name).restype = L.conv_status_string.restype if name == "conv_status_string" else ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().conv_status_string(int(status)).decode()


def make_problem(n, c_in, h, w, c_out, kh, kw, *, groups=1, stride=(1, 1), dilation=(1, 1),
                 pads=(0, 0, 0, 0), out_pad=(0, 0), transpose=False, act="identity",
                 alpha=None, beta=None, bias=False, residual=False, offsets=(0, 0, 0, 0, 0),
                 variant="auto", splits=0) -> conv_problem:
    """Fill a conv_problem; pads are (top, left, bottom, right)."""
    da, db = ACT_DEFAULTS.get(act, (0.0, 0.0))
    p = conv_problem()
    p.n, p.c_in, p.h, p.w, p.c_out, p.kh, p.kw = n, c_in, h, w, c_out, kh, kw
    p.groups = groups
    p.stride_h, p.stride_w = stride
    p.dil_h, p.dil_w = dilation
    p.pad_top, p.pad_left, p.pad_bottom, p.pad_right = pads
    p.out_pad_h, p.out_pad_w = out_pad
    p.x_off, p.w_off, p.b_off, p.r_off, p.y_off = offsets
    p.transpose = int(bool(transpose))
    p.activation = ACTIVATIONS[act]
    p.act_alpha = da if alpha is None else alpha
    p.act_beta = db if beta is None else beta
    p.has_bias = int(bool(bias))
    p.has_residual = int(bool(residual))
    p.variant_override = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    p.split_override = splits
    return p


def _dt(dtype):
    return DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def conv_output_extent(p: conv_problem):
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    st = lib().conv_output_extent(ctypes.byref(p), ctypes.byref(ho), ctypes.byref(wo))
    if st:
        raise ConvError(st, "conv_output_extent")
    return ho.value, wo.value


def conv_resolve_auto_pad(p: conv_problem, auto_pad, output_shape_hw=None) -> conv_problem:
    mode = AUTO_PAD[auto_pad] if isinstance(auto_pad, str) else int(auto_pad)
    arr = None
    if output_shape_hw is not None:
        arr = (ctypes.c_int64 * 2)(*output_shape_hw)
    st = lib().conv_resolve_auto_pad(ctypes.byref(p), mode, arr)
    if st:
        raise ConvError(st, "conv_resolve_auto_pad")
    return p


def conv_scratch_size(p: conv_problem, dtype):
    whole, per = ctypes.c_uint64(), ctypes.c_uint64()
    st = lib().conv_scratch_size(ctypes.byref(p), _dt(dtype), ctypes.byref(whole), ctypes.byref(per))
    if st:
        raise ConvError(st, "conv_scratch_size")
    return whole.value, per.value


def conv_describe_variant(p: conv_problem, dtype) -> str:
    buf = ctypes.create_string_buffer(256)
    st = lib().conv_describe_variant(ctypes.byref(p), _dt(dtype), buf, len(buf))
    if st:
        raise ConvError(st, "conv_describe_variant")
    return buf.value.decode()


def _call(fn, name, p, dtype, x, w, bias, residual, y, scratch, scratch_bytes, stream, check):
    st = fn(ctypes.byref(p), _dt(dtype), _ptr(x), _ptr(w), _ptr(bias), _ptr(residual), _ptr(y),
            _ptr(scratch), int(scratch_bytes), stream or None)
    if check and st:
        raise ConvError(st, name)
    return st


def conv_forward(p, dtype, x, w, bias, residual, y, scratch=None, scratch_bytes=0, stream=None,
                 check=True) -> int:
    """Enqueue the Conv forward on `stream` (a hipStream_t as int; None = default)."""
    return _call(lib().conv_forward, "conv_forward", p, dtype, x, w, bias, residual, y, scratch,
                 scratch_bytes, stream, check)


def conv_check(p, dtype, x, w, bias, residual, y, scratch=None, scratch_bytes=0) -> int:
    """Status conv_forward / conv_transpose_forward would return (host only)."""
    return lib().conv_check(ctypes.byref(p), _dt(dtype), _ptr(x), _ptr(w), _ptr(bias),
                            _ptr(residual), _ptr(y), _ptr(scratch), int(scratch_bytes))


def conv_transpose_forward(p, dtype, x, w, bias, residual, y, scratch=None, scratch_bytes=0,
                           stream=None, check=True) -> int:
    """Enqueue the ConvTranspose forward on `stream`."""
    return _call(lib().conv_transpose_forward, "conv_transpose_forward", p, dtype, x, w, bias,
                 residual, y, scratch, scratch_bytes, stream, check)


def conv_forward_noalloc(p, dtype, x, w, bias, residual, y, stream=None, check=True) -> int:
    """Enqueue Conv (p.transpose == 0) or ConvTranspose (p.transpose == 1) with the
    library's own static scratch: no allocation, no scratch argument."""
    st = lib().conv_forward_noalloc(ctypes.byref(p), _dt(dtype), _ptr(x), _ptr(w), _ptr(bias),
                                    _ptr(residual), _ptr(y), stream or None)
    if check and st:
        raise ConvError(st, "conv_forward_noalloc")
    return st


# ------------------------------------------------------------------ pooling

def make_pool_problem(n, c, h, w, kind="max", kernel=(1, 1), stride=(1, 1), dilation=(1, 1),
                      pads=(0, 0, 0, 0), ceil_mode=False, count_include_pad=False,
                      offsets=(0, 0)) -> pool_problem:
    """A pool_problem; pads are (top, left, bottom, right)."""
    return pool_problem(n, c, h, w, kernel[0], kernel[1], stride[0], stride[1], dilation[0],
                        dilation[1], pads[0], pads[1], pads[2], pads[3], offsets[0], offsets[1],
                        POOL_KINDS[kind] if isinstance(kind, str) else int(kind), int(ceil_mode),
                        int(count_include_pad), 0)


def pool_output_extent(p: pool_problem):
    ho, wo = ctypes.c_int64(), ctypes.c_int64()
    st = lib().pool_output_extent(ctypes.byref(p), ctypes.byref(ho), ctypes.byref(wo))
    if st:
        raise ConvError(st, "pool_output_extent")
    return ho.value, wo.value


def pool_resolve_auto_pad(p: pool_problem, auto_pad) -> pool_problem:
    mode = AUTO_PAD[auto_pad] if isinstance(auto_pad, str) else int(auto_pad)
    st = lib().pool_resolve_auto_pad(ctypes.byref(p), mode)
    if st:
        raise ConvError(st, "pool_resolve_auto_pad")
    return p


def pool_describe_variant(p: pool_problem, dtype) -> str:
    buf = ctypes.create_string_buffer(128)
    st = lib().pool_describe_variant(ctypes.byref(p), _dt(dtype), buf, len(buf))
    if st:
        raise ConvError(st, "pool_describe_variant")
    return buf.value.decode()


def pool_check(p: pool_problem, dtype, x, y) -> int:
    return lib().pool_check(ctypes.byref(p), _dt(dtype), _ptr(x), _ptr(y))


def pool_forward(p: pool_problem, dtype, x, y, stream=None, check=True) -> int:
    """Enqueue the pooling forward on `stream`."""
    st = lib().pool_forward(ctypes.byref(p), _dt(dtype), _ptr(x), _ptr(y), stream or None)
    if check and st:
        raise ConvError(st, "pool_forward")
    return st


# -------------------------------------------------------------- ConvInteger

CONVI_TYPES = {"u8": 0, "i8": 1}


def _it(t):
    return CONVI_TYPES[t] if isinstance(t, str) else int(t)


def conv_integer_describe_variant(p: conv_problem, x_type, w_type) -> str:
    buf = ctypes.create_string_buffer(128)
    st = lib().conv_integer_describe_variant(ctypes.byref(p), _it(x_type), _it(w_type), buf,
                                             len(buf))
    if st:
        raise ConvError(st, "conv_integer_describe_variant")
    return buf.value.decode()


def conv_integer_check(p, x_type, w_type, x, w, x_zero, w_zero, w_zero_per_channel, y) -> int:
    return lib().conv_integer_check(ctypes.byref(p), _it(x_type), _it(w_type), _ptr(x), _ptr(w),
                                    _ptr(x_zero), _ptr(w_zero), int(w_zero_per_channel), _ptr(y))


def conv_integer_forward(p, x_type, w_type, x, w, x_zero, w_zero, w_zero_per_channel, y,
                         stream=None, check=True) -> int:
    """Enqueue ConvInteger (int32 output with wrap-around) on `stream`."""
    st = lib().conv_integer_forward(ctypes.byref(p), _it(x_type), _it(w_type), _ptr(x), _ptr(w),
                                    _ptr(x_zero), _ptr(w_zero), int(w_zero_per_channel), _ptr(y),
                                    stream or None)
    if check and st:
        raise ConvError(st, "conv_integer_forward")
    return st
