"""Helpers shared by the GPU parity tests: run a layer through the C ABI on the
GPU (torch only allocates device memory and provides the stream) and compare it
with the fp64 oracle.

Parity bound, per output (the stated tolerances, "Convolution, pooling and
resize", "Tolerances"): |y_gpu - y_oracle| <= tol * S' + u(y_oracle), where
tol = 1e-5 for float32 and 2e-3 for float16 operands with float32 accumulation,
S' = sum |w*x| over the output's taps plus |bias| and |residual| (the bias and
residual are terms of the same sum), and u(v) is half a unit in the last place
of the output type at |v| (the final rounding of the stored value), plus, for
the transcendental activations (tanh, sigmoid, silu) that the epilogue evaluates
in float32, 4 float32 ulps at |v| (the evaluation error of expf/tanhf and the
division, which does not scale with the sum).
"""
from __future__ import annotations

import numpy as np
import torch

import convolution_forward_amd as cf
import oracle
import workloads

# bfloat16 (no page fixes its tolerance): fp16's 2e-3 is 4 units of fp16
# roundoff (2^-11); the same 4 units of bfloat16 roundoff (2^-8) give 1.6e-2.
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1.6e-2}
NP = {"f32": np.float32, "f16": np.float16, "bf16": np.int16}  # device storage
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_storage(a, dtype):
    """Host array of operand values -> the array whose bytes the device gets
    (bfloat16: the 16-bit patterns of bfloat16-exact values)."""
    if dtype == "bf16":
        return workloads.bf16_bits(a).view(np.int16)
    return np.asarray(a).astype(NP[dtype])


def from_storage(a, dtype):
    """Device bytes back to operand values (bfloat16 -> exact float32)."""
    if dtype == "bf16":
        return workloads.bf16_from_bits(np.asarray(a).view(np.uint16))
    return a


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def stream():
    return torch.cuda.current_stream().cuda_stream


def problem_from(geom: oracle.Geom, transpose=False, bias=False, residual=False, **kw):
    return cf.make_problem(geom.n, geom.c_in, geom.h, geom.w, geom.c_out, geom.kh, geom.kw,
                           groups=geom.groups, stride=(geom.sh, geom.sw),
                           dilation=(geom.dh, geom.dw),
                           pads=(geom.pt, geom.pl, geom.pb, geom.pr),
                           out_pad=(geom.oph, geom.opw), transpose=transpose, act=geom.act,
                           alpha=geom.alpha, beta=geom.beta, bias=bias, residual=residual, **kw)


def geom_from_layer(layer, n=None):
    t, l, b, r = layer.pads
    return oracle.Geom(n or layer.n, layer.c_in, layer.h, layer.w, layer.c_out, layer.kh,
                       layer.kw, groups=layer.groups, sh=layer.stride[0], sw=layer.stride[1],
                       dh=layer.dilation[0], dw=layer.dilation[1], pt=t, pl=l, pb=b, pr=r,
                       oph=layer.out_pad[0], opw=layer.out_pad[1], act=layer.act,
                       alpha=layer.alpha or cf.ACT_DEFAULTS.get(layer.act, (0.0, 0.0))[0],
                       beta=layer.beta or cf.ACT_DEFAULTS.get(layer.act, (0.0, 0.0))[1])


def run_gpu(geom, dtype, x, w, b=None, r=None, transpose=False, variant="auto", splits=0,
            scratch_images=None, offsets=None, alias_residual=False, y_init=None):
    """Run one problem through conv_forward / conv_transpose_forward.

    scratch_images: None = whole-batch scratch; k = scratch for k images (chunked).
    offsets: element offsets (x, w, b, r, y); each operand is placed at that
    offset inside a larger device buffer.
    Returns y as a numpy array of the operand dtype."""
    npdt = NP[dtype]
    offs = offsets or (0, 0, 0, 0, 0)
    p = problem_from(geom, transpose=transpose, bias=b is not None, residual=r is not None,
                     offsets=offs, variant=variant, splits=splits)
    ho, wo = cf.conv_output_extent(p)
    yshape = (geom.n, geom.c_out, ho, wo)

    def place(a, off, raw=False):
        if a is None:
            return None
        flat = np.zeros(off + a.size, npdt)
        flat[off:] = (a if raw else to_storage(a, dtype)).ravel()
        return dev(flat)

    xd, wd, bd = place(x, offs[0]), place(w, offs[1]), place(b, offs[2])
    ysize = int(np.prod(yshape))
    if alias_residual:
        assert r is not None and offs[3] == offs[4]
        yd = place(r, offs[4])
        rd = yd
    else:
        rd = place(r, offs[3])
        if y_init is not None:
            init = to_storage(y_init, dtype).ravel()
        elif dtype == "bf16":
            init = np.full(ysize, 0x7FC0, np.int16)  # quiet NaN
        else:
            init = np.full(ysize, np.nan, npdt)
        yd = place(init, offs[4], raw=True)
    whole, per = cf.conv_scratch_size(p, dtype)
    sbytes = whole if scratch_images is None else per * scratch_images
    scratch = torch.empty(max(sbytes, 16) // 4 + 4, dtype=torch.float32, device="cuda") \
        if sbytes else None
    fn = cf.conv_transpose_forward if transpose else cf.conv_forward
    fn(p, dtype, xd, wd, bd, rd, yd, scratch, sbytes if scratch is not None else 0, stream())
    torch.cuda.synchronize()
    out = yd.cpu().numpy()[offs[4]:].reshape(yshape)
    return from_storage(out, dtype)


def oracle_ref(geom, x, w, b=None, r=None, transpose=False):
    f = oracle.conv_transpose2d if transpose else oracle.conv2d
    return f(geom, x, w, b, r)


TRANSCENDENTAL = ("tanh", "sigmoid", "silu")


def bound(dtype, y_ref, s_ref, b=None, r=None, c_axis=1, act="identity"):
    """Per-output allowed error (see module docstring)."""
    sp = np.array(s_ref, dtype=np.float64)
    if b is not None:
        shp = [1] * sp.ndim
        shp[c_axis] = -1
        sp = sp + np.abs(np.asarray(b, np.float64)).reshape(shp)
    if r is not None:
        sp = sp + np.abs(np.asarray(r, np.float64))
    if dtype == "bf16":  # half an ulp of bfloat16 (8 significant bits) at |y|
        _, e = np.frexp(np.abs(np.asarray(y_ref, np.float64)))
        half_ulp = np.ldexp(1.0, e - 9)
    else:
        mag = np.abs(y_ref).astype(NP[dtype])
        half_ulp = np.spacing(mag).astype(np.float64) / 2
    if act in TRANSCENDENTAL:
        half_ulp = half_ulp + 4 * np.spacing(np.abs(y_ref).astype(np.float32)).astype(np.float64)
    return TOL[dtype] * sp + half_ulp


def assert_parity(dtype, y_gpu, y_ref, s_ref, b=None, r=None, what="", act="identity"):
    y_gpu = np.asarray(y_gpu, np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    err = np.abs(y_gpu - y_ref)
    lim = bound(dtype, y_ref, s_ref, b, r, act=act)
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outputs out of tolerance; first at "
            f"{tuple(i)}: gpu={y_gpu[tuple(i)]!r} oracle={y_ref[tuple(i)]!r} "
            f"err={err[tuple(i)]:.3g} bound={lim[tuple(i)]:.3g}")
    return float((err / np.maximum(lim, 1e-300)).max())
