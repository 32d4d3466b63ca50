"""Seeded synthetic workloads: the layer shapes and the input generators.

This module holds data only (shapes, distributions, seeds) and no arithmetic
of the method: output shapes are written out as given in the workload
statements, and both the HIP path and the oracle receive the arrays made here.

Workloads (one entry per layer; block workloads are their layers in order,
each layer with its own seeded input of the shape its chain implies):

1. single Conv fp32: N=1, 3->16, 32x32, 3x3, s1 p1, fused ReLU
2. ResNet-style bottleneck 3x3 fp16: N=32, 256->256, 14x14, s1 p1, bias,
   residual of the output's shape, then ReLU
3. stem 7x7 s2 p3 fp16 3->64 on 224x224 (-> 112x112), and a 1x1 pointwise
   64->256 on 56x56, bias + ReLU
4. depthwise-separable fp32: N=64, C=240, 28x28: depthwise 5x5 s1 p2 with
   hard-swish, depthwise 3x3 s2 p1, pointwise 1x1 240->80, bias
5. dilated grouped fp16: N=8, 256->256, 40x40, 3x3, dilation 2, pad 2,
   groups 32, sigmoid; then ConvTranspose W=[256,64,2,2] stride 2 ->
   64x80x80 with bias

Distributions: x ~ U[-1,1]; w ~ N(0, 2/fan_in) (He-normal, fan_in = weight
dim 1 * KH * KW); bias ~ U[-0.1,0.1]; residual ~ U[-1,1].  Values are drawn in
float64 and rounded once (round-to-nearest-even) to the layer's element type.
Seeds: 20261202 + 1000*workload + 10*layer + t, t = 0 x, 1 w, 2 bias, 3 residual.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

SEED_BASE = 20261202


@dataclass(frozen=True)
class Layer:
    name: str
    workload: int
    index: int
    dtype: str  # "f32", "f16" or "bf16"
    n: int
    c_in: int
    h: int
    w: int
    c_out: int
    kh: int
    kw: int
    out_shape: tuple  # as stated by the workload (N, C, H, W)
    groups: int = 1
    stride: tuple = (1, 1)
    dilation: tuple = (1, 1)
    pads: tuple = (0, 0, 0, 0)  # top, left, bottom, right
    out_pad: tuple = (0, 0)
    transpose: bool = False
    act: str = "identity"
    alpha: float = 0.0
    beta: float = 0.0
    bias: bool = True
    residual: bool = False
    variant: str = "auto"  # a variant the caller asks for (the plan's own choice by default)
    note: str = ""

    @property
    def np_dtype(self):
        """numpy type holding the operand values (bfloat16 values are held
        exactly in float32; numpy has no bfloat16 type)."""
        return np.float16 if self.dtype == "f16" else np.float32

    @property
    def w_shape(self):
        if self.transpose:
            return (self.c_in, self.c_out // self.groups, self.kh, self.kw)
        return (self.c_out, self.c_in // self.groups, self.kh, self.kw)

    @property
    def x_shape(self):
        return (self.n, self.c_in, self.h, self.w)

    def with_batch(self, n: int) -> "Layer":
        """Same layer at another batch size (output shape follows the batch)."""
        return replace(self, n=n, out_shape=(n,) + tuple(self.out_shape[1:]))


LAYERS = [
    Layer("w1_conv3x3_f32", 1, 0, "f32", 1, 3, 32, 32, 16, 3, 3, (1, 16, 32, 32),
          pads=(1, 1, 1, 1), act="relu"),
    Layer("w2_bottleneck3x3_f16", 2, 0, "f16", 32, 256, 14, 14, 256, 3, 3,
          (32, 256, 14, 14), pads=(1, 1, 1, 1), act="relu", residual=True),
    Layer("w3a_stem7x7s2_f16", 3, 0, "f16", 32, 3, 224, 224, 64, 7, 7, (32, 64, 112, 112),
          stride=(2, 2), pads=(3, 3, 3, 3), act="relu"),
    Layer("w3b_pointwise_f16", 3, 1, "f16", 32, 64, 56, 56, 256, 1, 1, (32, 256, 56, 56),
          act="relu"),
    Layer("w4a_depthwise5x5_f32", 4, 0, "f32", 64, 240, 28, 28, 240, 5, 5, (64, 240, 28, 28),
          groups=240, pads=(2, 2, 2, 2), act="hard_swish"),
    Layer("w4b_depthwise3x3s2_f32", 4, 1, "f32", 64, 240, 28, 28, 240, 3, 3,
          (64, 240, 14, 14), groups=240, stride=(2, 2), pads=(1, 1, 1, 1)),
    Layer("w4c_pointwise_f32", 4, 2, "f32", 64, 240, 14, 14, 80, 1, 1, (64, 80, 14, 14)),
    Layer("w5a_dilated_grouped_f16", 5, 0, "f16", 8, 256, 40, 40, 256, 3, 3, (8, 256, 40, 40),
          groups=32, dilation=(2, 2), pads=(2, 2, 2, 2), act="sigmoid"),
    Layer("w5b_convtranspose2x2s2_f16", 5, 1, "f16", 8, 256, 40, 40, 64, 2, 2, (8, 64, 80, 80),
          stride=(2, 2), transpose=True),
]

# Measured beside the five workloads: the late 3x3 layer of the RTX 4070
# single-layer split-k table (512 -> 512 channels at 7x7, batch 1), here in
# fp16 with bias and ReLU.  Its grid is small and its k long, so the planner
# cuts k into ranges.
EXTRA_LAYERS = [
    Layer("x1_late3x3_512_7x7_f16", 6, 0, "f16", 1, 512, 7, 7, 512, 3, 3, (1, 512, 7, 7),
          pads=(1, 1, 1, 1), act="relu"),
    # the bottleneck layer of workload 2 with bfloat16 operands
    Layer("x2_bottleneck3x3_bf16", 7, 0, "bf16", 32, 256, 14, 14, 256, 3, 3,
          (32, 256, 14, 14), pads=(1, 1, 1, 1), act="relu", residual=True),
    # the same layer (same seeded inputs as workload 2) through Winograd
    # F(2x2, 3x3), which the caller must ask for
    Layer("x3_bottleneck3x3_f16_winograd", 2, 0, "f16", 32, 256, 14, 14, 256, 3, 3,
          (32, 256, 14, 14), pads=(1, 1, 1, 1), act="relu", residual=True, variant="winograd"),
]

BY_NAME = {l.name: l for l in LAYERS + EXTRA_LAYERS}


def workload_layers(wl: int):
    return [l for l in LAYERS if l.workload == wl]


def seed(layer: Layer, t: int) -> int:
    return SEED_BASE + 1000 * layer.workload + 10 * layer.index + t


def fan_in(layer: Layer) -> int:
    ws = layer.w_shape
    return ws[1] * ws[2] * ws[3]


@dataclass
class Inputs:
    x: np.ndarray
    w: np.ndarray
    b: np.ndarray | None
    r: np.ndarray | None
    extra: dict = field(default_factory=dict)


def bf16_round(a) -> np.ndarray:
    """Round float64 values once, to nearest with ties to even, to bfloat16
    (8 significant bits), returned exactly as float32.  Done from float64
    directly (frexp / rint / ldexp are exact), not through float32, so there is
    no double rounding.  Finite values in the normal range only."""
    m, e = np.frexp(np.asarray(a, np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8).astype(np.float32)


def bf16_bits(a) -> np.ndarray:
    """The 16-bit patterns of bfloat16-exact float32 values (the upper halves)."""
    f = np.ascontiguousarray(a, np.float32)
    bits = f.view(np.uint32)
    assert not np.any(bits & 0xFFFF), "value not exact in bfloat16"
    return (bits >> 16).astype(np.uint16)


def bf16_from_bits(bits) -> np.ndarray:
    """float32 values of bfloat16 bit patterns."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize(a, dtype: str) -> np.ndarray:
    """Round float64 values once to the operand type ("f32", "f16", "bf16")."""
    if dtype == "bf16":
        return bf16_round(a)
    return np.asarray(a, np.float64).astype(np.float16 if dtype == "f16" else np.float32)


def make_inputs(layer: Layer, seeds: tuple | None = None) -> Inputs:
    """The layer's seeded inputs, drawn in float64 and rounded once to its dtype.

    Draws fill arrays in C order, so a smaller batch is a prefix of the full
    batch's x and residual."""
    q = lambda a: quantize(a, layer.dtype)
    s = seeds or tuple(seed(layer, t) for t in range(4))
    x = q(np.random.default_rng(s[0]).uniform(-1.0, 1.0, layer.x_shape))
    std = math.sqrt(2.0 / fan_in(layer))
    w = q(np.random.default_rng(s[1]).standard_normal(layer.w_shape) * std)
    b = (q(np.random.default_rng(s[2]).uniform(-0.1, 0.1, (layer.c_out,)))
         if layer.bias else None)
    r = (q(np.random.default_rng(s[3]).uniform(-1.0, 1.0, layer.out_shape))
         if layer.residual else None)
    return Inputs(x, w, b, r)


def random_tensor(rng: np.random.Generator, shape, dtype, lo=-1.0, hi=1.0):
    return rng.uniform(lo, hi, shape).astype(dtype)


def integer_tensor(rng: np.random.Generator, shape, dtype, lo=-2, hi=2):
    """Small integers: exact in fp16 and fp32, so sums are exact in any order."""
    return rng.integers(lo, hi + 1, shape).astype(dtype)


# ------------------------------------------------------------------ pooling

@dataclass(frozen=True)
class PoolLayer:
    """A pooling step of the same models ("Convolution, pooling and resize",
    "Pooling and resize"); x ~ U[-1,1] rounded once to the dtype."""

    name: str
    workload: int
    index: int
    dtype: str
    n: int
    c: int
    h: int
    w: int
    kind: str  # "max", "average", "global_max", "global_average"
    kernel: tuple = (1, 1)
    stride: tuple = (1, 1)
    dilation: tuple = (1, 1)
    pads: tuple = (0, 0, 0, 0)
    ceil_mode: bool = False
    count_include_pad: bool = False

    @property
    def x_shape(self):
        return (self.n, self.c, self.h, self.w)


POOL_LAYERS = [
    # the ResNet stem's max pool, on the stem convolution's output shape
    PoolLayer("p1_maxpool3x3s2_f16", 8, 0, "f16", 32, 64, 112, 112, "max", (3, 3), (2, 2),
              pads=(1, 1, 1, 1)),
    # an average pool in ceil mode without padding counted, on the depthwise
    # block's shape
    PoolLayer("p2_avgpool3x3s2_ceil_f32", 8, 1, "f32", 64, 240, 28, 28, "average", (3, 3),
              (2, 2), ceil_mode=True),
    # the classifier head: global average over 2048 planes of 7x7
    PoolLayer("p3_globalavg_f16", 8, 2, "f16", 32, 2048, 7, 7, "global_average"),
    # global max over the pointwise layer's output
    PoolLayer("p4_globalmax_f32", 8, 3, "f32", 64, 80, 14, 14, "global_max"),
]

POOL_BY_NAME = {l.name: l for l in POOL_LAYERS}


def make_pool_input(layer: PoolLayer) -> np.ndarray:
    rng = np.random.default_rng(SEED_BASE + 1000 * layer.workload + 10 * layer.index)
    return quantize(rng.uniform(-1.0, 1.0, layer.x_shape), layer.dtype)


# -------------------------------------------------------------- ConvInteger

@dataclass(frozen=True)
class IntLayer:
    """A quantized convolution ("Convolution, pooling and resize", "ConvInteger"):
    x and w uniform over their type's range, one x zero point, per-channel w
    zero points."""

    name: str
    workload: int
    index: int
    x_type: str  # "u8" or "i8"
    w_type: str
    n: int
    c_in: int
    h: int
    w: int
    c_out: int
    kh: int
    kw: int
    out_shape: tuple
    groups: int = 1
    stride: tuple = (1, 1)
    dilation: tuple = (1, 1)
    pads: tuple = (0, 0, 0, 0)


INT_LAYERS = [
    # the bottleneck 3x3 layer of workload 2, quantized: uint8 activations with a
    # zero point, int8 weights with one zero point per output channel
    IntLayer("q1_bottleneck3x3_u8i8", 9, 0, "u8", "i8", 32, 256, 14, 14, 256, 3, 3,
             (32, 256, 14, 14), pads=(1, 1, 1, 1)),
]

INT_BY_NAME = {l.name: l for l in INT_LAYERS}


def make_int_inputs(layer: IntLayer):
    """(x, w, x_zero, w_zero) as int64 arrays / ints of the operands' values."""
    lo = {"u8": 0, "i8": -128}
    s = [SEED_BASE + 1000 * layer.workload + 10 * layer.index + t for t in range(4)]
    x = np.random.default_rng(s[0]).integers(lo[layer.x_type], lo[layer.x_type] + 256,
                                             (layer.n, layer.c_in, layer.h, layer.w))
    w = np.random.default_rng(s[1]).integers(
        lo[layer.w_type], lo[layer.w_type] + 256,
        (layer.c_out, layer.c_in // layer.groups, layer.kh, layer.kw))
    xz = int(np.random.default_rng(s[2]).integers(lo[layer.x_type], lo[layer.x_type] + 256))
    wz = np.random.default_rng(s[3]).integers(lo[layer.w_type], lo[layer.w_type] + 256,
                                              layer.c_out)
    return x, w, xz, wz
