"""Plain fp64 CPU oracle for the convolution forward (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its binding) never does, and this package imports nothing
from the product.

Each function states the passage of the pages it follows; the C file carries
the definitions.  All arrays are converted to float64 before the call, so the
oracle sees exactly the values the GPU sees (inputs already rounded once to the
layer's element type by the caller).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# Activation codes, in the order the OneGpu page ("Layout and operands") lists
# the fused activations.
ACT = {
    "identity": 0,
    "relu": 1,
    "tanh": 2,
    "sigmoid": 3,
    "silu": 4,
    "hard_sigmoid": 5,
    "hard_swish": 6,
    "clip": 7,
    "leaky_relu": 8,
}

# auto_pad modes (ONNX names)
AUTO_PAD = {"NOTSET": 0, "SAME_UPPER": 1, "SAME_LOWER": 2, "VALID": 3}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc -O2 -fopenmp (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
             "-Wall", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Geom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n", "c_in", "h", "w", "c_out", "kh", "kw", "groups",
        "sh", "sw", "dh", "dw", "pt", "pl", "pb", "pr", "oph", "opw")] + [
        ("act", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("alpha", ctypes.c_double), ("beta", ctypes.c_double)]


class _PoolGeom(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n", "c", "h", "w", "kh", "kw", "sh", "sw", "dh", "dw", "pt", "pl", "pb", "pr")] + [
        ("kind", ctypes.c_int32), ("ceil_mode", ctypes.c_int32),
        ("count_include_pad", ctypes.c_int32), ("pad_", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        i64, i64p, dp = ctypes.c_int64, ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p
        lib.oracle_conv_extent.argtypes = [i64, i64, i64, i64, i64, i64, i64p]
        lib.oracle_convt_extent.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64p]
        lib.oracle_auto_pad.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, i64,
                                        i64, i64, i64p, i64p]
        lib.oracle_conv_macs.argtypes = [ctypes.POINTER(_Geom), i64, i64]
        lib.oracle_conv_macs.restype = i64
        lib.oracle_activation.argtypes = [ctypes.c_int, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_double]
        lib.oracle_activation.restype = ctypes.c_double
        g = ctypes.POINTER(_Geom)
        lib.oracle_conv2d.argtypes = [g, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_conv2d_points.argtypes = [g, dp, dp, dp, dp, dp, i64, dp, dp, ctypes.c_int]
        lib.oracle_conv2d_im2col.argtypes = [g, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_conv_transpose2d.argtypes = [g, dp, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_conv_transpose2d_gather.argtypes = [g, dp, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_pool_extent.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int, i64p]
        lib.oracle_pool2d.argtypes = [ctypes.POINTER(_PoolGeom), dp, ctypes.c_double, dp, dp]
        lib.oracle_global_pool.argtypes = [ctypes.c_int, i64, i64, dp, dp, dp]
        lib.oracle_conv_integer.argtypes = [ctypes.POINTER(_Geom), dp, dp, ctypes.c_int32, dp, dp,
                                            ctypes.c_int]
        lib.oracle_conv2d_winograd.argtypes = [g, dp, dp, dp, dp, dp, ctypes.c_int]
        _lib = lib
    return _lib


@dataclass
class Geom:
    """One problem's geometry with explicit pads (top, left, bottom, right)."""

    n: int
    c_in: int
    h: int
    w: int
    c_out: int
    kh: int
    kw: int
    groups: int = 1
    sh: int = 1
    sw: int = 1
    dh: int = 1
    dw: int = 1
    pt: int = 0
    pl: int = 0
    pb: int = 0
    pr: int = 0
    oph: int = 0
    opw: int = 0
    act: str = "identity"
    alpha: float = 0.0
    beta: float = 0.0

    def _c(self) -> _Geom:
        return _Geom(self.n, self.c_in, self.h, self.w, self.c_out, self.kh, self.kw,
                     self.groups, self.sh, self.sw, self.dh, self.dw, self.pt, self.pl,
                     self.pb, self.pr, self.oph, self.opw, ACT[self.act], 0,
                     float(self.alpha), float(self.beta))


def conv_extent(n_in, k, s, d, pad_begin, pad_end):
    """Boxed output-size equation ("Convolutions", section 2.1); None if no window fits."""
    out = ctypes.c_int64(0)
    rc = _load().oracle_conv_extent(n_in, k, s, d, pad_begin, pad_end, ctypes.byref(out))
    return None if rc else out.value


def convt_extent(n_in, k, s, d, pad_begin, pad_end, out_pad):
    """Transposed output size (section 2.1's inversion + output_padding)."""
    out = ctypes.c_int64(0)
    rc = _load().oracle_convt_extent(n_in, k, s, d, pad_begin, pad_end, out_pad,
                                     ctypes.byref(out))
    return None if rc else out.value


def auto_pad(transpose, mode, n_in, k, s, d, out_pad=0, out_req=-1, pads=(0, 0)):
    """ONNX auto_pad resolution (reading stated in the C file); None on error."""
    pb, pe = ctypes.c_int64(pads[0]), ctypes.c_int64(pads[1])
    rc = _load().oracle_auto_pad(int(transpose), AUTO_PAD[mode] if isinstance(mode, str)
                                 else int(mode), n_in, k, s, d, out_pad, out_req,
                                 ctypes.byref(pb), ctypes.byref(pe))
    return None if rc else (pb.value, pe.value)


def activation(name, v, alpha=0.0, beta=0.0):
    return _load().oracle_activation(ACT[name], float(v), float(alpha), float(beta))


def out_shape(g: Geom, transpose=False):
    if transpose:
        ho = convt_extent(g.h, g.kh, g.sh, g.dh, g.pt, g.pb, g.oph)
        wo = convt_extent(g.w, g.kw, g.sw, g.dw, g.pl, g.pr, g.opw)
    else:
        ho = conv_extent(g.h, g.kh, g.sh, g.dh, g.pt, g.pb)
        wo = conv_extent(g.w, g.kw, g.sw, g.dw, g.pl, g.pr)
    if ho is None or wo is None:
        raise ValueError("no output window fits")
    return (g.n, g.c_out, ho, wo)


def conv_macs(g: Geom, transpose=False):
    """MACs ("Convolutions", section 2.3); for ConvT the count of x*w products."""
    if transpose:
        return g.n * g.c_in * g.h * g.w * (g.c_out // g.groups) * g.kh * g.kw
    _, _, ho, wo = out_shape(g)
    return _load().oracle_conv_macs(ctypes.byref(g._c()), ho, wo)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data


def _check_shapes(g: Geom, x, w, b, r, yshape, transpose):
    assert x.shape == (g.n, g.c_in, g.h, g.w), x.shape
    if transpose:
        assert w.shape == (g.c_in, g.c_out // g.groups, g.kh, g.kw), w.shape
    else:
        assert w.shape == (g.c_out, g.c_in // g.groups, g.kh, g.kw), w.shape
    if b is not None:
        assert b.shape == (g.c_out,), b.shape
    if r is not None:
        assert r.shape == yshape, r.shape


def conv2d(g: Geom, x, w, b=None, r=None, threads=0, with_scale=True):
    """Direct definition of Conv (cross-correlation with zero padding, stride,
    dilation, groups) then bias, residual, activation in fp64.
    Returns (y, S) with S = sum |x*w| over each output's taps."""
    x, w, b, r = _f64(x), _f64(w), _f64(b), _f64(r)
    shp = out_shape(g)
    _check_shapes(g, x, w, b, r, shp, False)
    y = np.empty(shp, np.float64)
    s = np.empty(shp, np.float64) if with_scale else None
    rc = _load().oracle_conv2d(ctypes.byref(g._c()), _p(x), _p(w), _p(b), _p(r), _p(y),
                               _p(s), threads)
    if rc:
        raise ValueError("oracle_conv2d rejected the problem")
    return y, s


def conv2d_points(g: Geom, x, w, b, r, flat_idx, threads=0):
    """conv2d evaluated at the given flat NCHW output indices only."""
    x, w, b, r = _f64(x), _f64(w), _f64(b), _f64(r)
    shp = out_shape(g)
    _check_shapes(g, x, w, b, r, shp, False)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    y = np.empty(idx.shape, np.float64)
    s = np.empty(idx.shape, np.float64)
    rc = _load().oracle_conv2d_points(ctypes.byref(g._c()), _p(x), _p(w), _p(b), _p(r),
                                      _p(idx), idx.size, _p(y), _p(s), threads)
    if rc:
        raise ValueError("oracle_conv2d_points rejected the problem")
    return y, s


def conv2d_im2col(g: Geom, x, w, b=None, r=None, threads=0):
    """Unfold + matrix product formulation ("Convolutions", sections 1 and 2.4)."""
    x, w, b, r = _f64(x), _f64(w), _f64(b), _f64(r)
    shp = out_shape(g)
    _check_shapes(g, x, w, b, r, shp, False)
    y = np.empty(shp, np.float64)
    rc = _load().oracle_conv2d_im2col(ctypes.byref(g._c()), _p(x), _p(w), _p(b), _p(r),
                                      _p(y), threads)
    if rc:
        raise ValueError("oracle_conv2d_im2col rejected the problem")
    return y


def conv_transpose2d(g: Geom, x, w, b=None, r=None, threads=0, with_scale=True):
    """ConvTranspose by its scatter definition ("Convolutions", section 2.5);
    weight [Cin, Cout/g, KH, KW] (OneGpu "Layout and operands").  Returns (y, S)."""
    x, w, b, r = _f64(x), _f64(w), _f64(b), _f64(r)
    shp = out_shape(g, transpose=True)
    _check_shapes(g, x, w, b, r, shp, True)
    y = np.empty(shp, np.float64)
    s = np.empty(shp, np.float64) if with_scale else None
    rc = _load().oracle_conv_transpose2d(ctypes.byref(g._c()), _p(x), _p(w), _p(b), _p(r),
                                         _p(y), _p(s), threads)
    if rc:
        raise ValueError("oracle_conv_transpose2d rejected the problem")
    return y, s


def conv_transpose2d_gather(g: Geom, x, w, b=None, r=None, threads=0):
    """ConvTranspose by its gather form (independent cross-check of the scatter)."""
    x, w, b, r = _f64(x), _f64(w), _f64(b), _f64(r)
    shp = out_shape(g, transpose=True)
    _check_shapes(g, x, w, b, r, shp, True)
    y = np.empty(shp, np.float64)
    rc = _load().oracle_conv_transpose2d_gather(ctypes.byref(g._c()), _p(x), _p(w), _p(b),
                                                _p(r), _p(y), threads)
    if rc:
        raise ValueError("oracle_conv_transpose2d_gather rejected the problem")
    return y


def max_threads() -> int:
    return _load().oracle_max_threads()


# ------------------------------------------------------------------ pooling

# Lowest finite value of each element type (an empty max window's result,
# "Convolution, pooling and resize", "Pooling and resize").
LOWEST = {"f32": -3.4028234663852886e38, "f16": -65504.0, "bf16": -3.3895313892515355e38}


@dataclass
class PoolGeom:
    """A pooling problem: window, stride, dilation, explicit pads, ceil mode,
    count_include_pad; kind "max" or "average"."""

    n: int
    c: int
    h: int
    w: int
    kh: int = 1
    kw: int = 1
    sh: int = 1
    sw: int = 1
    dh: int = 1
    dw: int = 1
    pt: int = 0
    pl: int = 0
    pb: int = 0
    pr: int = 0
    kind: str = "max"
    ceil_mode: bool = False
    count_include_pad: bool = False

    def _c(self) -> _PoolGeom:
        return _PoolGeom(self.n, self.c, self.h, self.w, self.kh, self.kw, self.sh, self.sw,
                         self.dh, self.dw, self.pt, self.pl, self.pb, self.pr,
                         {"max": 0, "average": 1}[self.kind], int(self.ceil_mode),
                         int(self.count_include_pad), 0)


def pool_extent(n_in, k, s, d, pad_begin, pad_end, ceil_mode):
    """Pooling output size along one axis (floor or ceil mode); None if no window fits."""
    out = ctypes.c_int64(0)
    rc = _load().oracle_pool_extent(n_in, k, s, d, pad_begin, pad_end, int(ceil_mode),
                                    ctypes.byref(out))
    return None if rc else out.value


def pool_out_shape(g: PoolGeom):
    ho = pool_extent(g.h, g.kh, g.sh, g.dh, g.pt, g.pb, g.ceil_mode)
    wo = pool_extent(g.w, g.kw, g.sw, g.dw, g.pl, g.pr, g.ceil_mode)
    if ho is None or wo is None:
        raise ValueError("no pooling window fits")
    return (g.n, g.c, ho, wo)


def pool2d(g: PoolGeom, x, dtype="f32"):
    """MaxPool / AveragePool by their definitions in fp64 ("Pooling and resize":
    NaN, empty-window, ceil_mode and count_include_pad rules).  Returns
    (y, scale) with scale = sum|x| / divisor for the average (zeros for max)."""
    x = _f64(x)
    assert x.shape == (g.n, g.c, g.h, g.w), x.shape
    shp = pool_out_shape(g)
    y = np.empty(shp, np.float64)
    s = np.empty(shp, np.float64)
    rc = _load().oracle_pool2d(ctypes.byref(g._c()), _p(x), LOWEST[dtype], _p(y), _p(s))
    if rc:
        raise ValueError("oracle_pool2d rejected the problem")
    return y, s


def global_pool(kind, x):
    """GlobalMaxPool / GlobalAveragePool over each (n, c) plane of x [n, c, h, w].
    Returns (y [n, c, 1, 1], scale) with scale the mean |x| (zeros for max)."""
    x = _f64(x)
    n, c, h, w = x.shape
    y = np.empty((n, c, 1, 1), np.float64)
    s = np.empty((n, c, 1, 1), np.float64)
    rc = _load().oracle_global_pool({"max": 0, "average": 1}[kind], n * c, h * w, _p(x),
                                    _p(y), _p(s))
    if rc:
        raise ValueError("oracle_global_pool rejected the problem")
    return y, s


# -------------------------------------------------------------- ConvInteger

def conv_integer(g: Geom, x, w, x_zero=0, w_zero=0, threads=0):
    """ONNX ConvInteger ("Convolution, pooling and resize", "ConvInteger"):
    sum of (x - x_zero) * (w - w_zero[co]) over the real taps, exact, then
    wrapped to int32.  x and w are integer arrays of uint8 or int8 values;
    w_zero is a scalar or one value per output channel."""
    x = np.ascontiguousarray(np.asarray(x, np.int32))
    w = np.ascontiguousarray(np.asarray(w, np.int32))
    assert x.shape == (g.n, g.c_in, g.h, g.w), x.shape
    assert w.shape == (g.c_out, g.c_in // g.groups, g.kh, g.kw), w.shape
    wz = np.ascontiguousarray(np.broadcast_to(np.asarray(w_zero, np.int32), (g.c_out,)))
    y = np.empty(out_shape(g), np.int32)
    rc = _load().oracle_conv_integer(ctypes.byref(g._c()), _p(x), _p(w), int(x_zero), _p(wz),
                                     _p(y), threads)
    if rc:
        raise ValueError("oracle_conv_integer rejected the problem")
    return y


# ------------------------------------------------------------ Winograd F(2x2,3x3)

def conv2d_winograd(g: Geom, x, w, b=None, r=None, threads=0):
    """Winograd F(2x2, 3x3) in fp64 by the minimal filtering algorithm's steps
    ("Convolutions", section 2.6; Lavin and Gray 2016): weight and input-tile
    transforms, the sixteen products summed over input channels, the output
    transform, then the epilogue.  3x3, stride 1, dilation 1 only."""
    x, w, b, r = _f64(x), _f64(w), _f64(b), _f64(r)
    shp = out_shape(g)
    _check_shapes(g, x, w, b, r, shp, False)
    y = np.empty(shp, np.float64)
    rc = _load().oracle_conv2d_winograd(ctypes.byref(g._c()), _p(x), _p(w), _p(b), _p(r), _p(y),
                                        threads)
    if rc:
        raise ValueError("oracle_conv2d_winograd rejected the problem")
    return y
