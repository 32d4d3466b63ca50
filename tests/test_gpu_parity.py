"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Covers the workload layers (reduced batch, full comparison; full size, sampled
outputs), a seeded sweep of small shapes over every variant, activation and
option, bit-exact index-mapping probes, integer exactness, determinism,
chunking, forced split-k and forced variants, element offsets and residual
aliasing.
"""
import dataclasses
import itertools
import re
import sys

import numpy as np
import pytest

import convolution_forward_amd as cf
import oracle
import workloads
from gpu_harness import TOL, assert_parity, geom_from_layer, oracle_ref, run_gpu

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cf.lib()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


REDUCED_N = {
    "w1_conv3x3_f32": 1, "w2_bottleneck3x3_f16": 4, "w3a_stem7x7s2_f16": 1,
    "w3b_pointwise_f16": 1, "w4a_depthwise5x5_f32": 2, "w4b_depthwise3x3s2_f32": 2,
    "w4c_pointwise_f32": 3, "w5a_dilated_grouped_f16": 1, "w5b_convtranspose2x2s2_f16": 1,
}


@pytest.mark.parametrize("name", [l.name for l in workloads.LAYERS])
def test_workload_layer_reduced_batch(name):
    layer = workloads.BY_NAME[name]
    lr = layer.with_batch(REDUCED_N[name])
    _say(f"[parity] {name} n={lr.n}")
    inp = workloads.make_inputs(lr)
    g = geom_from_layer(lr)
    y = run_gpu(g, lr.dtype, inp.x, inp.w, inp.b, inp.r, transpose=lr.transpose)
    assert y.shape == lr.out_shape
    yr, sr = oracle_ref(g, inp.x, inp.w, inp.b, inp.r, transpose=lr.transpose)
    q = assert_parity(lr.dtype, y, yr, sr, inp.b, inp.r, what=name, act=lr.act)
    _say(f"  max err / bound = {q:.3g}")


FULL_SIZE = [l.name for l in workloads.LAYERS] + [l.name for l in workloads.EXTRA_LAYERS]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_workload_layer_full_size(name):
    """Full workload size, in the launch configuration the benchmark times
    (same plan, whole-batch scratch), every output compared with the oracle.

    Besides the bound the tests hold every kernel to (tol * S' plus the final
    store's half ulp), the strict ratio max |err| / (tol * sum|w*x|) of the
    tolerance statement alone is computed, printed and required to be <= 1."""
    from expected_plans import EXPECTED_PLANS, layer_problem
    layer = workloads.BY_NAME[name]
    variant = cf.conv_describe_variant(layer_problem(cf, layer), layer.dtype)
    assert variant == EXPECTED_PLANS[name], variant
    _say(f"[parity-full] {name} n={layer.n} {variant}")
    inp = workloads.make_inputs(layer)
    g = geom_from_layer(layer)
    y = run_gpu(g, layer.dtype, inp.x, inp.w, inp.b, inp.r, transpose=layer.transpose,
                variant=layer.variant)
    assert y.shape == layer.out_shape
    yr, sr = oracle_ref(g, inp.x, inp.w, inp.b, inp.r, transpose=layer.transpose)
    q = assert_parity(layer.dtype, y, yr, sr, inp.b, inp.r, what=name, act=layer.act)
    err = np.abs(y.astype(np.float64) - yr)
    assert np.all(sr > 0)
    strict = float((err / (TOL[layer.dtype] * sr)).max())
    _say(f"  [strict] {name} max|err|/(tol*sum|w*x|) = {strict:.4g}; "
         f"max err/bound = {q:.4g}; outputs = {y.size}")
    assert strict <= 1.0, strict


# One specialised kernel per entry, in a geometry that kernel takes: (geometry,
# dtype, transpose, forced variant, text the variant name must contain).  The
# workload-sized runs above compare the persistent and multi-row paths in full;
# these pin each kernel's gather and scatter indexing bit for bit.
KERNELS = {
    "rowshift_r8": (oracle.Geom(4, 64, 8, 8, 64, 3, 3, pt=1, pl=1, pb=1, pr=1), "f16", False,
                    "implicit_gemm_halo", "rowshift.r8"),
    "rowshift_r14": (oracle.Geom(4, 64, 14, 14, 64, 3, 3, pt=1, pl=1, pb=1, pr=1), "f16",
                     False, "implicit_gemm_halo", "rowshift.r14"),
    "halo": (oracle.Geom(2, 32, 9, 40, 32, 3, 3, pt=1, pl=1, pb=1, pr=1), "f16", False,
             "implicit_gemm_halo", "implicit_gemm_halo.f16.r"),
    "rowband_partial": (oracle.Geom(32, 3, 30, 32, 64, 7, 7, sh=2, sw=2, pt=3, pl=3, pb=3, pr=3),
                        "f16", False, "implicit_gemm_rowband", "rows2"),
    "rowband_partial_elem": (oracle.Geom(32, 3, 30, 30, 64, 7, 7, sh=2, sw=2, pt=3, pl=3, pb=3,
                                         pr=3), "f16", False, "implicit_gemm_rowband", "rows2"),
    "grouped": (oracle.Geom(2, 64, 12, 12, 64, 3, 3, groups=8, dh=2, dw=2, pt=2, pl=2, pb=2, pr=2),
                "f16", False, "implicit_gemm_grouped", "c8"),
    "pointwise_f16_multitile": (oracle.Geom(2100, 16, 4, 4, 24, 1, 1), "f16", False,
                                "pointwise_gemm", "pointwise_gemm.f16"),
    "pointwise_f16": (oracle.Geom(3, 64, 12, 16, 200, 1, 1), "f16", False, "pointwise_gemm",
                      "pointwise_gemm.f16"),
    "pointwise_f32": (oracle.Geom(3, 24, 10, 12, 200, 1, 1), "f32", False, "pointwise_gemm",
                      "pointwise_gemm.f32.t64x80.k64"),
    "pointwise_f32_strip": (oracle.Geom(3, 240, 10, 12, 100, 1, 1), "f32", False, "pointwise_gemm",
                            "pointwise_gemm.f32.t256x16.strip"),
    "transpose_fused": (oracle.Geom(4, 64, 10, 12, 32, 2, 2, sh=2, sw=2), "f16", True,
                        "transpose_gemm_col2im", "fused_k2s2"),
    "transpose_col2im": (oracle.Geom(2, 24, 5, 6, 10, 3, 3, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1),
                         "f16", True, "transpose_gemm_col2im", "transpose_gemm_col2im.f16"),
    "depthwise_wave_5x5": (oracle.Geom(40, 256, 8, 8, 256, 5, 5, groups=256, pt=2, pl=2, pb=2,
                                       pr=2), "f32", False, "depthwise_direct", "wave.col14"),
    "depthwise_wave_3x3s2": (oracle.Geom(40, 256, 8, 8, 256, 3, 3, groups=256, sh=2, sw=2,
                                         pt=1, pl=1, pb=1, pr=1), "f32", False,
                             "depthwise_direct", "wave.col4"),
    "depthwise_wave_f16": (oracle.Geom(40, 256, 8, 8, 256, 5, 5, groups=256, pt=2, pl=2, pb=2,
                                       pr=2), "f16", False, "depthwise_direct", "wave"),
    "implicit_gemm": (oracle.Geom(2, 3, 9, 11, 16, 3, 3, pt=1, pl=1, pb=1, pr=1), "f32", False,
                      "implicit_gemm", "split1"),
    "implicit_gemm_split": (oracle.Geom(1, 128, 7, 7, 64, 3, 3, pt=1, pl=1, pb=1, pr=1), "f16",
                            False, "implicit_gemm", "split"),
}


def _kernel_run(kind, x, w, b=None, r=None, act="identity"):
    g, dtype, tr, variant, want = KERNELS[kind]
    g = dataclasses.replace(g, act=act)
    from gpu_harness import problem_from
    d = cf.conv_describe_variant(problem_from(g, transpose=tr, variant=variant,
                                              bias=b is not None, residual=r is not None), dtype)
    assert want in d, (kind, d)
    y = run_gpu(g, dtype, x, w, b, r, transpose=tr, variant=variant)
    yr, _ = oracle_ref(g, x, w, b, r, transpose=tr)
    return y, yr, d


def _w_shape(g, tr):
    return (g.c_in, g.c_out // g.groups, g.kh, g.kw) if tr else (g.c_out, g.c_in // g.groups, g.kh, g.kw)


@pytest.mark.parametrize("kind", list(KERNELS))
def test_kernel_index_probes(kind):
    """Integer-coded inputs (each value names its position, exact in fp16) and
    one-hot weights: output channel co reads tap t(co) = (co + j * Cout) mod T
    of its window (T = taps per group), for j over enough runs that every tap
    is read by some channel.  Each output must equal the addressed input
    value, or 0 where the tap is padding, bit for bit ('Convolutions',
    section 1: the worked example's windows)."""
    g, dtype, tr, _, _ = KERNELS[kind]
    npdt = np.float16 if dtype == "f16" else np.float32
    _say(f"[probe] {kind} {g}")
    x = (np.arange(g.n * g.c_in * g.h * g.w) % 1000 + 1).reshape(g.n, g.c_in, g.h, g.w).astype(npdt)
    ws = _w_shape(g, tr)
    T = ws[1] * ws[2] * ws[3] if not tr else (g.c_in // g.groups) * g.kh * g.kw
    runs = -(-T // g.c_out)
    for j in range(runs):
        w = np.zeros(ws, npdt)
        for co in range(g.c_out):
            t = (co + j * g.c_out) % T
            if tr:
                gi, jj = divmod(co, g.c_out // g.groups)
                ci, rest = divmod(t, g.kh * g.kw)
                w[gi * (g.c_in // g.groups) + ci, jj, rest // g.kw, rest % g.kw] = 1
            else:
                ci, rest = divmod(t, g.kh * g.kw)
                w[co, ci, rest // g.kw, rest % g.kw] = 1
        y, yr, _ = _kernel_run(kind, x, w)
        assert np.array_equal(y.astype(np.float64), yr), (kind, j)


@pytest.mark.parametrize("kind", list(KERNELS))
def test_kernel_integer_exact(kind):
    """Inputs, weights, bias and residual in {-1, 0, 1}: every partial sum is
    an integer below 2^11, exact in fp32 and in the fp16 store whatever the
    summation order, so each kernel's output must equal the oracle's exactly
    (ReLU fused, the common compiled activation)."""
    g, dtype, tr, _, _ = KERNELS[kind]
    npdt = np.float16 if dtype == "f16" else np.float32
    rng = np.random.default_rng(sum(map(ord, kind)))
    _say(f"[exact] {kind}")
    x = rng.integers(-1, 2, (g.n, g.c_in, g.h, g.w)).astype(npdt)
    w = rng.integers(-1, 2, _w_shape(g, tr)).astype(npdt)
    b = rng.integers(-1, 2, g.c_out).astype(npdt)
    from gpu_harness import problem_from
    ho, wo = cf.conv_output_extent(problem_from(g, transpose=tr))
    # the fused k = s = 2 ConvTranspose path takes no residual
    r = None if (tr and "fused" in KERNELS[kind][4]) else \
        rng.integers(-1, 2, (g.n, g.c_out, ho, wo)).astype(npdt)
    y, yr, _ = _kernel_run(kind, x, w, b, r, act="relu")
    assert np.array_equal(y.astype(np.float64), yr), kind


def _sweep_cases():
    rng = np.random.default_rng(2026)
    acts = list(cf.ACTIVATIONS)
    cases = []
    while len(cases) < 48:
        G = int(rng.choice([1, 1, 1, 2, 4]))
        cig = int(rng.choice([1, 2, 3, 5, 8, 16, 19, 40]))
        cog = int(rng.choice([1, 3, 8, 17, 64, 70]))
        if G > 1 and cig * G > 64:
            G = 1
        kh, kw = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        g = oracle.Geom(int(rng.integers(1, 4)), cig * G, int(rng.integers(1, 20)),
                        int(rng.integers(1, 20)), cog * G, kh, kw, groups=G,
                        sh=int(rng.integers(1, 4)), sw=int(rng.integers(1, 4)),
                        dh=int(rng.integers(1, 3)), dw=int(rng.integers(1, 3)),
                        pt=int(rng.integers(0, 3)), pl=int(rng.integers(0, 3)),
                        pb=int(rng.integers(0, 3)), pr=int(rng.integers(0, 3)),
                        act=acts[len(cases) % len(acts)])
        if g.act == "clip":
            g.alpha, g.beta = -0.3, 0.4
        elif g.act == "leaky_relu":
            g.alpha = 0.1
        elif g.act == "hard_sigmoid":
            g.alpha, g.beta = 0.2, 0.5
        try:
            oracle.out_shape(g)
        except ValueError:
            continue
        dtype = ("f32", "f16")[len(cases) % 2]
        cases.append((g, dtype, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: f"{c[1]}-{c[0].act}")
def test_random_shapes(case):
    g, dtype, has_b, has_r = case
    _say(f"[sweep] {dtype} {g}")
    rng = np.random.default_rng(g.n * 1000 + g.c_in * 10 + g.kh)
    npdt = np.float16 if dtype == "f16" else np.float32
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(npdt)
    w = (rng.standard_normal((g.c_out, g.c_in // g.groups, g.kh, g.kw)) * 0.3).astype(npdt)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(npdt) if has_b else None
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(npdt) if has_r else None
    yr, sr = oracle.conv2d(g, x, w, b, r)
    variants = ["auto", "implicit_gemm"]
    if g.c_in // g.groups == 1:
        variants.append("depthwise_direct")
    if _applicable(g, dtype, "implicit_gemm_halo"):
        variants.append("implicit_gemm_halo")
    for v in variants:
        y = run_gpu(g, dtype, x, w, b, r, variant=v)
        assert_parity(dtype, y, yr, sr, b, r, what=f"{v}", act=g.act)


def _applicable(g, dtype, variant):
    from gpu_harness import problem_from
    try:
        cf.conv_describe_variant(problem_from(g, variant=variant), dtype)
        return True
    except cf.ConvError:
        return False


HALO_CASES = [
    # (geometry, bias, residual)
    (oracle.Geom(2, 64, 14, 14, 64, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu"), True, True),
    (oracle.Geom(3, 32, 7, 7, 48, 3, 3, pt=1, pl=1, pb=1, pr=1, act="silu"), True, False),
    (oracle.Geom(1, 96, 15, 17, 40, 3, 3, sh=2, sw=2, pt=1, pl=0, pb=2, pr=1), False, True),
    (oracle.Geom(2, 16, 20, 30, 16, 3, 3, dh=2, dw=3, pt=2, pl=3, pb=2, pr=3, act="tanh"),
     True, False),
    (oracle.Geom(1, 24, 9, 64, 20, 3, 3, sh=1, sw=1, pt=0, pl=1, pb=0, pr=1), True, True),
    (oracle.Geom(2, 64, 10, 56, 64, 3, 3, groups=8, dh=2, dw=2, pt=2, pl=2, pb=2, pr=2,
                 act="sigmoid"), True, False),
    (oracle.Geom(2, 64, 12, 50, 256, 1, 1, act="relu"), True, False),
    (oracle.Geom(1, 48, 5, 5, 33, 1, 1, sh=2, sw=2, pt=1, pl=1, pb=0, pr=0), True, True),
    (oracle.Geom(4, 256, 14, 14, 256, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu"), True, True),
]


@pytest.mark.parametrize("case", HALO_CASES, ids=lambda c: f"{c[0].c_in}x{c[0].h}x{c[0].w}")
def test_halo_variant(case):
    g, has_b, has_r = case
    _say(f"[halo] {g}")
    assert _applicable(g, "f16", "implicit_gemm_halo")
    rng = np.random.default_rng(g.c_in + 31 * g.w)
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(np.float16)
    w = (rng.standard_normal((g.c_out, g.c_in // g.groups, g.kh, g.kw)) *
         np.sqrt(2.0 / (g.c_in // g.groups * g.kh * g.kw))).astype(np.float16)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(np.float16) if has_b else None
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(np.float16) if has_r else None
    yr, sr = oracle.conv2d(g, x, w, b, r)
    y = run_gpu(g, "f16", x, w, b, r, variant="implicit_gemm_halo")
    assert_parity("f16", y, yr, sr, b, r, what="halo", act=g.act)
    # same bits when chunked over images (no scratch: every image is independent)
    # and with misaligned weights (element-load path)
    y2 = run_gpu(g, "f16", x, w, b, r, variant="implicit_gemm_halo", offsets=(1, 3, 0, 0, 2))
    assert np.array_equal(_bits(y), _bits(y2))


ROWSHIFT_CASES = [
    (oracle.Geom(2, 64, 14, 14, 64, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu"), True, True),
    (oracle.Geom(3, 128, 7, 7, 40, 3, 3, pt=1, pl=1, pb=1, pr=1, act="silu"), True, False),
    (oracle.Geom(1, 64, 12, 11, 96, 3, 3, pt=0, pl=2, pb=2, pr=0), False, True),
    (oracle.Geom(2, 128, 10, 10, 64, 3, 3, groups=2, pt=1, pl=0, pb=1, pr=1, act="tanh"),
     True, False),
    (oracle.Geom(1, 192, 16, 16, 32, 3, 3), True, True),  # no pads: 14 x 14 out
    (oracle.Geom(2, 64, 5, 4, 48, 3, 3, pt=2, pl=2, pb=1, pr=2, act="hard_swish"), True, True),
    # five and six 64-channel stages: the steady-state loop of the pipeline
    (oracle.Geom(2, 320, 6, 6, 32, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu"), False, True),
    (oracle.Geom(1, 384, 9, 9, 64, 3, 3, pt=1, pl=1, pb=1, pr=1), True, True),
]


POINTWISE_CASES = [
    # (geometry, bias, residual): channel chunks with tails, channel tiles with
    # tails, pixel tiles with tails, several images, every epilogue term
    (oracle.Geom(2, 64, 12, 12, 256, 1, 1, act="relu"), True, False),
    (oracle.Geom(3, 24, 10, 6, 40, 1, 1, act="silu"), True, True),
    (oracle.Geom(1, 136, 16, 9, 200, 1, 1), False, True),
    (oracle.Geom(4, 72, 2, 2, 130, 1, 1, act="hard_swish"), True, True),
    (oracle.Geom(2, 256, 7, 4, 64, 1, 1, act="tanh"), True, False),
]


ROWBAND_CASES = [
    # (geometry, bias, residual): stem-like stride-2 layers with few input channels
    (oracle.Geom(2, 3, 30, 28, 64, 7, 7, sh=2, sw=2, pt=3, pl=3, pb=3, pr=3, act="relu"), True, False),
    (oracle.Geom(3, 3, 17, 23, 40, 7, 7, sh=2, sw=2, pt=3, pl=3, pb=3, pr=3), True, True),
    (oracle.Geom(2, 4, 20, 16, 24, 5, 5, sh=2, sw=2, pt=2, pl=2, pb=1, pr=2, act="hard_swish"),
     False, True),
    (oracle.Geom(1, 8, 33, 40, 64, 3, 3, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1, act="sigmoid"), True, False),
    (oracle.Geom(2, 3, 64, 64, 128, 7, 7, sh=2, sw=2, pt=3, pl=3, pb=3, pr=3, act="relu"), True, False),
]


GROUPED_CASES = [
    # (geometry, bias, residual): 8 input channels per group; dilation, stride,
    # asymmetric pads, 1x1 / 2x2 / 3x3 taps, up to 32 output channels per group,
    # planes whose pixel count is not a multiple of 4 (element loads)
    (oracle.Geom(2, 16, 9, 11, 48, 3, 3, groups=2, pt=1, pl=1, pb=1, pr=1), True, False),
    (oracle.Geom(3, 32, 12, 12, 32, 3, 3, groups=4, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1,
                 act="relu"), True, True),
    (oracle.Geom(1, 24, 20, 16, 96, 1, 1, groups=3, act="silu"), False, True),
    (oracle.Geom(2, 64, 16, 16, 16, 3, 3, groups=8, dh=3, dw=2, pt=3, pl=2, pb=2, pr=3,
                 act="hard_swish"), True, False),
    (oracle.Geom(2, 40, 13, 14, 40, 2, 2, groups=5, pt=1, pl=0, pb=0, pr=1, act="tanh"), True, True),
    (oracle.Geom(1, 256, 40, 40, 256, 3, 3, groups=32, dh=2, dw=2, pt=2, pl=2, pb=2, pr=2,
                 act="sigmoid"), True, False),
]


@pytest.mark.parametrize("case", GROUPED_CASES, ids=lambda c: f"g{c[0].groups}x{c[0].c_out}k{c[0].kh}x{c[0].kw}")
def test_grouped_variant(case):
    """The grouped (8 channels per group) implicit GEMM against the oracle;
    identical bits with misaligned operands and with y aliasing the residual."""
    g, has_b, has_r = case
    _say(f"[grouped] {g}")
    from gpu_harness import problem_from
    assert cf.conv_describe_variant(problem_from(g), "f16").startswith("implicit_gemm_grouped")
    rng = np.random.default_rng(g.c_in * 3 + g.h + 7 * g.c_out + g.kh)
    cig = g.c_in // g.groups
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(np.float16)
    w = (rng.standard_normal((g.c_out, cig, g.kh, g.kw)) *
         np.sqrt(2.0 / (cig * g.kh * g.kw))).astype(np.float16)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(np.float16) if has_b else None
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(np.float16) if has_r else None
    yr, sr = oracle.conv2d(g, x, w, b, r)
    y = run_gpu(g, "f16", x, w, b, r)
    assert_parity("f16", y, yr, sr, b, r, what="grouped", act=g.act)
    y2 = run_gpu(g, "f16", x, w, b, r, offsets=(1, 3, 1, 1, 1))
    assert np.array_equal(_bits(y), _bits(y2))
    if has_r:
        y3 = run_gpu(g, "f16", x, w, b, r, offsets=(0, 0, 0, 8, 8), alias_residual=True)
        assert np.array_equal(_bits(y), _bits(y3))
    y4 = run_gpu(g, "f16", x, w, b, r, variant="implicit_gemm")
    assert_parity("f16", y4, yr, sr, b, r, what="grouped-as-igemm", act=g.act)


POINTWISE_F32_CASES = [
    # (geometry, bias, residual): float32 1x1 on x as it lies; channel chunks with
    # tails, several channel tiles, tiles straddling images, tiny planes
    (oracle.Geom(3, 240, 14, 14, 80, 1, 1), True, False),
    (oracle.Geom(2, 36, 6, 10, 100, 1, 1, act="relu"), True, False),
    (oracle.Geom(1, 132, 5, 4, 17, 1, 1, act="silu"), False, True),
    (oracle.Geom(5, 8, 2, 2, 80, 1, 1, act="hard_swish"), True, True),
    # strips of 16 channels x 256 pixels: 12-step windows, whole (c_in 48, 144,
    # 240, 288) or with masked tail steps (c_in 16, 160, 256, 320), ragged
    # channel tiles, strips straddling images, a last strip with idle waves
    (oracle.Geom(2, 256, 7, 8, 90, 1, 1, act="relu"), True, True),
    (oracle.Geom(3, 160, 14, 14, 80, 1, 1, act="relu"), True, True),
    (oracle.Geom(2, 144, 6, 10, 100, 1, 1), False, True),
    (oracle.Geom(5, 48, 7, 4, 40, 1, 1, act="sigmoid"), True, False),
    (oracle.Geom(1, 16, 2, 2, 5, 1, 1, act="relu"), True, True),
    (oracle.Geom(2, 288, 6, 10, 40, 1, 1, act="relu"), True, True),
    (oracle.Geom(1, 320, 4, 4, 100, 1, 1), False, True),
]


@pytest.mark.parametrize("case", POINTWISE_F32_CASES, ids=lambda c: f"{c[0].c_in}to{c[0].c_out}x{c[0].h}x{c[0].w}")
def test_pointwise_f32_variant(case):
    """The float32 1x1 GEMM (MFMA f32) against the oracle; identical bits with
    misaligned operands (element loads) and with y aliasing the residual."""
    g, has_b, has_r = case
    _say(f"[pointwise-f32] {g}")
    from gpu_harness import problem_from
    assert cf.conv_describe_variant(problem_from(g), "f32").startswith("pointwise_gemm.f32")
    rng = np.random.default_rng(g.c_in + 17 * g.c_out + g.h)
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(np.float32)
    w = (rng.standard_normal((g.c_out, g.c_in, 1, 1)) * np.sqrt(2.0 / g.c_in)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(np.float32) if has_b else None
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(np.float32) if has_r else None
    yr, sr = oracle.conv2d(g, x, w, b, r)
    y = run_gpu(g, "f32", x, w, b, r)
    assert_parity("f32", y, yr, sr, b, r, what="pointwise-f32", act=g.act)
    y2 = run_gpu(g, "f32", x, w, b, r, offsets=(1, 3, 1, 1, 1))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    if has_r:
        y3 = run_gpu(g, "f32", x, w, b, r, offsets=(0, 0, 0, 4, 4), alias_residual=True)
        assert np.array_equal(y.view(np.uint32), y3.view(np.uint32))
    y4 = run_gpu(g, "f32", x, w, b, r, variant="implicit_gemm")
    assert_parity("f32", y4, yr, sr, b, r, what="pointwise-f32-as-igemm", act=g.act)


@pytest.mark.parametrize("case", ROWBAND_CASES, ids=lambda c: f"{c[0].c_in}x{c[0].h}x{c[0].w}k{c[0].kh}")
def test_rowband_variant(case):
    """The row-band stride-2 kernel against the oracle; identical bits with
    misaligned operands and with y aliasing the residual."""
    g, has_b, has_r = case
    _say(f"[rowband] {g}")
    from gpu_harness import problem_from
    assert cf.conv_describe_variant(problem_from(g), "f16").startswith("implicit_gemm_rowband")
    rng = np.random.default_rng(g.c_in * 7 + g.h + 5 * g.c_out)
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(np.float16)
    w = (rng.standard_normal((g.c_out, g.c_in, g.kh, g.kw)) *
         np.sqrt(2.0 / (g.c_in * g.kh * g.kw))).astype(np.float16)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(np.float16) if has_b else None
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(np.float16) if has_r else None
    yr, sr = oracle.conv2d(g, x, w, b, r)
    y = run_gpu(g, "f16", x, w, b, r)
    assert_parity("f16", y, yr, sr, b, r, what="rowband", act=g.act)
    y2 = run_gpu(g, "f16", x, w, b, r, offsets=(1, 3, 1, 1, 1))
    assert np.array_equal(_bits(y), _bits(y2))
    if has_r:
        y3 = run_gpu(g, "f16", x, w, b, r, offsets=(0, 0, 0, 8, 8), alias_residual=True)
        assert np.array_equal(_bits(y), _bits(y3))


@pytest.mark.parametrize("case", POINTWISE_CASES, ids=lambda c: f"{c[0].c_in}to{c[0].c_out}x{c[0].h}x{c[0].w}")
def test_pointwise_variant(case):
    """The 1x1 GEMM on x as it lies against the oracle; identical bits with
    misaligned operands (element loads and stores) and with y aliasing the
    residual."""
    g, has_b, has_r = case
    _say(f"[pointwise] {g}")
    from gpu_harness import problem_from
    assert cf.conv_describe_variant(problem_from(g), "f16").startswith("pointwise_gemm.f16")
    rng = np.random.default_rng(g.c_in + 31 * g.c_out + g.h)
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(np.float16)
    w = (rng.standard_normal((g.c_out, g.c_in, 1, 1)) * np.sqrt(2.0 / g.c_in)).astype(np.float16)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(np.float16) if has_b else None
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(np.float16) if has_r else None
    yr, sr = oracle.conv2d(g, x, w, b, r)
    y = run_gpu(g, "f16", x, w, b, r)
    assert_parity("f16", y, yr, sr, b, r, what="pointwise", act=g.act)
    y2 = run_gpu(g, "f16", x, w, b, r, offsets=(1, 3, 1, 1, 1))
    assert np.array_equal(_bits(y), _bits(y2))
    if has_r:
        y3 = run_gpu(g, "f16", x, w, b, r, offsets=(0, 0, 0, 4, 4), alias_residual=True)
        assert np.array_equal(_bits(y), _bits(y3))
    y4 = run_gpu(g, "f16", x, w, b, r, variant="implicit_gemm")
    assert_parity("f16", y4, yr, sr, b, r, what="pointwise-as-igemm", act=g.act)


@pytest.mark.parametrize("case", ROWSHIFT_CASES, ids=lambda c: f"{c[0].c_in}x{c[0].h}x{c[0].w}")
def test_rowshift_variant(case):
    g, has_b, has_r = case
    _say(f"[rowshift] {g}")
    from gpu_harness import problem_from
    assert "rowshift" in cf.conv_describe_variant(problem_from(g, variant="implicit_gemm_halo"),
                                                  "f16")
    rng = np.random.default_rng(g.c_in + 17 * g.w + g.h)
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(np.float16)
    w = (rng.standard_normal((g.c_out, g.c_in // g.groups, 3, 3)) *
         np.sqrt(2.0 / (g.c_in // g.groups * 9))).astype(np.float16)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(np.float16) if has_b else None
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(np.float16) if has_r else None
    yr, sr = oracle.conv2d(g, x, w, b, r)
    v = "implicit_gemm_halo"
    y = run_gpu(g, "f16", x, w, b, r, variant=v)
    assert_parity("f16", y, yr, sr, b, r, what="rowshift", act=g.act)
    y2 = run_gpu(g, "f16", x, w, b, r, variant=v, offsets=(5, 1, 2, 0, 3))  # misaligned w
    assert np.array_equal(_bits(y), _bits(y2))
    y3 = run_gpu(g, "f16", x, w, b, r, variant=v)
    assert np.array_equal(_bits(y), _bits(y3))
    if has_r:  # y aliasing the residual (16-byte aligned: the flat epilogue)
        y4 = run_gpu(g, "f16", x, w, b, r, variant=v, offsets=(0, 0, 0, 8, 8), alias_residual=True)
        assert np.array_equal(_bits(y), _bits(y4))


def _sweep_rowshift(seed):
    """A random 3x3 stride-1 geometry the row-shift kernel takes: whole
    64-channel stages per group, output rows of at most 14 columns."""
    rng = np.random.default_rng(seed)
    groups = int(rng.choice([1, 1, 2]))
    cig = 64 * int(rng.integers(1, 4))
    cog = int(rng.integers(1, 7)) * 8 * (1 if groups == 1 else 1)
    pt, pb, pl, pr = (int(v) for v in rng.integers(0, 3, 4))
    ho, wo = int(rng.integers(2, 15)), int(rng.integers(2, 15))
    h, w = ho + 2 - pt - pb, wo + 2 - pl - pr
    if h < 1 or w < 1:
        h, w, pt, pb, pl, pr = ho, wo, 1, 1, 1, 1
    act = str(rng.choice(["identity", "relu", "silu", "tanh", "hard_swish"]))
    g = oracle.Geom(int(rng.integers(1, 4)), cig * groups, h, w, cog * groups, 3, 3, groups=groups,
                    pt=pt, pl=pl, pb=pb, pr=pr, act=act)
    return g, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))


def _sweep_rowband(seed):
    """A random stride-2 geometry with few input channels (the row-band kernel)."""
    rng = np.random.default_rng(seed)
    k = int(rng.choice([3, 5, 7]))
    c_in = int(rng.integers(1, 5)) if k < 7 else int(rng.integers(1, 4))
    h, w = int(rng.integers(9, 41)), int(rng.integers(9, 41))
    p = [int(v) for v in rng.integers(0, k // 2 + 1, 4)]
    act = str(rng.choice(["identity", "relu", "sigmoid", "hard_swish"]))
    g = oracle.Geom(int(rng.integers(1, 3)), c_in, h, w, int(rng.integers(1, 17)) * 8, k, k, sh=2, sw=2,
                    pt=p[0], pl=p[1], pb=p[2], pr=p[3], act=act)
    return g, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))


def _sweep_more(kind, seed):
    """Random geometries for the pointwise (f16, f32), depthwise, grouped and
    fused ConvTranspose kernels: (geometry, dtype, bias, residual, transpose)."""
    rng = np.random.default_rng(seed)
    acts = ["identity", "relu", "sigmoid", "hard_swish", "silu"]
    act = str(rng.choice(acts))
    hb, hr = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    n = int(rng.integers(1, 4))
    if kind == "pointwise_f16":
        g = oracle.Geom(n, 8 * int(rng.integers(1, 25)), int(rng.integers(1, 20)), 4 * int(rng.integers(1, 10)),
                        int(rng.integers(1, 300)), 1, 1, act=act)
        return g, "f16", hb, hr, False
    if kind == "pointwise_f32":
        g = oracle.Geom(n, 4 * int(rng.integers(1, 40)), int(rng.integers(1, 16)), 4 * int(rng.integers(1, 8)),
                        int(rng.integers(1, 200)), 1, 1, act=act)
        return g, "f32", hb, hr, False
    if kind == "depthwise":
        k = int(rng.choice([3, 5, 7]))
        s = 1 if k == 7 else int(rng.choice([1, 2]))
        c = int(rng.integers(1, 40))
        h, w = int(rng.integers(k, 33)), 4 * int(rng.integers(2, 9))
        p = k // 2
        g = oracle.Geom(n, c, h, w, c, k, k, groups=c, sh=s, sw=s, pt=p, pl=p, pb=p, pr=p, act=act)
        return g, str(rng.choice(["f16", "f32"])), hb, hr, False
    if kind == "grouped":
        groups = int(rng.integers(2, 9))
        cog = int(rng.choice([4, 8, 16, 24, 32]))
        k = int(rng.choice([1, 2, 3]))
        d = int(rng.choice([1, 2]))
        s = int(rng.choice([1, 2]))
        h, w = int(rng.integers(3, 41)), int(rng.integers(3, 41))
        p = [int(v) for v in rng.integers(0, d * (k - 1) // 2 + 1, 4)]
        g = oracle.Geom(n, 8 * groups, h, w, cog * groups, k, k, groups=groups, sh=s, sw=s, dh=d, dw=d,
                        pt=p[0], pl=p[1], pb=p[2], pr=p[3], act=act)
        return g, "f16", hb, hr, False
    # fused ConvTranspose, kernel = stride = 2
    g = oracle.Geom(n, 8 * int(rng.integers(1, 20)), int(rng.integers(1, 12)), 4 * int(rng.integers(1, 11)),
                    int(rng.integers(1, 70)), 2, 2, sh=2, sw=2, act=act)  # fused path: w % 4 == 0
    return g, "f16", hb, False, True


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("kind", ["pointwise_f16", "pointwise_f32", "depthwise", "grouped", "transpose_fused"])
def test_random_sweep_more(kind, seed):
    """Seeded random geometries for the remaining specialised kernels against the
    oracle (a case the planner gives to another kernel is skipped)."""
    g, dtype, has_b, has_r, tr = _sweep_more(kind, 7919 * seed + len(kind))
    _say(f"[sweep {kind} {seed}] {dtype} {g} bias={has_b} res={has_r}")
    _check_more(kind, g, dtype, has_b, has_r, tr, seed)


def _check_more(kind, g, dtype, has_b, has_r, tr, seed):
    """Plan check (skip a case the planner gives to another kernel), seeded
    inputs, GPU call and element-wise parity against the oracle."""
    from gpu_harness import problem_from
    want = {"pointwise_f16": "pointwise_gemm.f16", "pointwise_f32": "pointwise_gemm.f32",
            "depthwise": "depthwise_direct", "grouped": "implicit_gemm_grouped",
            "transpose_fused": "transpose_gemm_col2im.f16.fused"}[kind]
    try:
        name = cf.conv_describe_variant(problem_from(g, transpose=tr), dtype)
    except Exception:
        pytest.skip("geometry not accepted")
    if not name.startswith(want):
        pytest.skip(f"planned as {name}")
    npdt = np.float16 if dtype == "f16" else np.float32
    rng = np.random.default_rng(seed + 1234)
    cig = g.c_in // g.groups
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(npdt)
    if tr:
        w = (rng.standard_normal((g.c_in, g.c_out, 2, 2)) * np.sqrt(2.0 / (4 * g.c_in))).astype(npdt)
        b = rng.uniform(-0.1, 0.1, g.c_out).astype(npdt) if has_b else None
        yr, sr = oracle.conv_transpose2d(g, x, w, b, None)
        y = run_gpu(g, dtype, x, w, b, None, transpose=True)
        assert_parity(dtype, y, yr, sr, b, None, what=f"sweep {kind}", act=g.act)
        return
    w = (rng.standard_normal((g.c_out, cig, g.kh, g.kw)) * np.sqrt(2.0 / (cig * g.kh * g.kw))).astype(npdt)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(npdt) if has_b else None
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(npdt) if has_r else None
    yr, sr = oracle.conv2d(g, x, w, b, r)
    y = run_gpu(g, dtype, x, w, b, r)
    assert_parity(dtype, y, yr, sr, b, r, what=f"sweep {kind}", act=g.act)


# Geometries on the vector paths of the kernels whose common activations are
# fixed at compile time (whole 16-byte vectors, no residual on the depthwise
# kernel), so that each compiled activation runs at least once.
_ACT_FIXED = [
    ("pointwise_f16", oracle.Geom(2, 64, 8, 8, 48, 1, 1), "f16", False),
    ("pointwise_f32", oracle.Geom(2, 24, 8, 8, 20, 1, 1), "f32", False),
    ("pointwise_f32", oracle.Geom(2, 32, 8, 8, 20, 1, 1), "f32", False),  # strip kernel
    ("depthwise", oracle.Geom(2, 6, 16, 16, 6, 3, 3, groups=6, pt=1, pl=1, pb=1, pr=1), "f32", False),
    ("depthwise", oracle.Geom(2, 6, 16, 16, 6, 3, 3, groups=6, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1),
     "f16", False),
    ("depthwise", oracle.Geom(2, 6, 16, 16, 6, 5, 5, groups=6, pt=2, pl=2, pb=2, pr=2), "f32", False),
    ("depthwise", oracle.Geom(2, 6, 16, 16, 6, 5, 5, groups=6, sh=2, sw=2, pt=2, pl=2, pb=2, pr=2),
     "f32", False),
    ("grouped", oracle.Geom(2, 64, 16, 16, 64, 3, 3, groups=8, dh=2, dw=2, pt=2, pl=2, pb=2, pr=2), "f16",
     False),
    ("transpose_fused", oracle.Geom(2, 32, 8, 8, 24, 2, 2, sh=2, sw=2), "f16", True),
]


@pytest.mark.parametrize("act", ["identity", "relu", "sigmoid", "hard_swish"])
@pytest.mark.parametrize("case", range(len(_ACT_FIXED)))
def test_compiled_activations(case, act):
    """Every activation the host may hand to a compile-time-activation kernel
    (and one it may not), on that kernel's vector path, against the oracle."""
    kind, g0, dtype, tr = _ACT_FIXED[case]
    g = dataclasses.replace(g0, act=act)
    _say(f"[act {kind} {case} {act}] {dtype} {g}")
    _check_more(kind, g, dtype, True, False, tr, 31 * case + len(act))


@pytest.mark.parametrize("seed", range(16))
@pytest.mark.parametrize("kind", ["rowshift", "rowband"])
def test_random_sweep(kind, seed):
    """Seeded random geometries for the row-shift and row-band kernels against
    the oracle (a case the planner gives to another kernel is skipped)."""
    g, has_b, has_r = (_sweep_rowshift if kind == "rowshift" else _sweep_rowband)(1000 * seed + 7)
    _say(f"[sweep {kind} {seed}] {g} bias={has_b} res={has_r}")
    from gpu_harness import problem_from
    v = "implicit_gemm_halo" if kind == "rowshift" else "auto"
    try:
        name = cf.conv_describe_variant(problem_from(g, variant=v), "f16")
    except Exception:
        pytest.skip("geometry not taken by the kernel")
    if kind not in name:
        pytest.skip(f"planned as {name}")
    rng = np.random.default_rng(seed + 99)
    cig = g.c_in // g.groups
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(np.float16)
    w = (rng.standard_normal((g.c_out, cig, g.kh, g.kw)) * np.sqrt(2.0 / (cig * g.kh * g.kw))).astype(np.float16)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(np.float16) if has_b else None
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(np.float16) if has_r else None
    yr, sr = oracle.conv2d(g, x, w, b, r)
    y = run_gpu(g, "f16", x, w, b, r, variant=v)
    assert_parity("f16", y, yr, sr, b, r, what=f"sweep {kind}", act=g.act)
    if kind == "rowshift":
        # whole k in one workgroup, and (when the planner splits this small
        # grid) the split through a one-image scratch: the same bits as the
        # whole-batch split
        y1 = run_gpu(g, "f16", x, w, b, r, variant=v, splits=1)
        assert_parity("f16", y1, yr, sr, b, r, what="sweep rowshift whole k", act=g.act)
        if ".split" in name:
            yc = run_gpu(g, "f16", x, w, b, r, variant=v, scratch_images=1)
            assert np.array_equal(_bits(y), _bits(yc))


DEPTHWISE_CASES = [
    (oracle.Geom(3, 5, 9, 11, 10, 3, 3, groups=5, pt=1, pl=1, pb=1, pr=1, act="relu"), "f32"),
    (oracle.Geom(2, 7, 13, 13, 7, 7, 7, groups=7, pt=3, pl=3, pb=3, pr=3), "f32"),
    (oracle.Geom(4, 6, 15, 14, 6, 5, 5, groups=6, sh=2, sw=2, pt=2, pl=2, pb=2, pr=1,
                 act="hard_swish"), "f32"),
    (oracle.Geom(2, 24, 28, 28, 24, 3, 3, groups=24, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1), "f16"),
    (oracle.Geom(5, 3, 7, 6, 9, 5, 5, groups=3, pt=2, pl=2, pb=2, pr=2, act="sigmoid"), "f16"),
    (oracle.Geom(1, 4, 30, 30, 4, 3, 3, groups=4, pt=0, pl=0, pb=0, pr=0), "f32"),
    # groups of planes that wrap from one image into the next, partial last group
    (oracle.Geom(7, 13, 20, 20, 13, 3, 3, groups=13, pt=1, pl=1, pb=1, pr=1), "f32"),
    # more plane groups than resident workgroups: each workgroup walks several
    (oracle.Geom(30, 70, 64, 64, 70, 3, 3, groups=70, pt=1, pl=1, pb=1, pr=1), "f32"),
]


@pytest.mark.parametrize("case", DEPTHWISE_CASES, ids=lambda c: f"{c[1]}-{c[0].kh}x{c[0].kw}s{c[0].sh}")
def test_depthwise_variants(case):
    """Whole-plane and tiled depthwise paths against the oracle; same bits when
    the input is misaligned (element loads) and from run to run."""
    g, dtype = case
    _say(f"[depthwise] {dtype} {g}")
    npdt = np.float16 if dtype == "f16" else np.float32
    rng = np.random.default_rng(g.c_out * 13 + g.kh)
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(npdt)
    w = (rng.standard_normal((g.c_out, 1, g.kh, g.kw)) * 0.3).astype(npdt)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(npdt)
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(npdt)
    yr, sr = oracle.conv2d(g, x, w, b, r)
    y = run_gpu(g, dtype, x, w, b, r)
    assert_parity(dtype, y, yr, sr, b, r, what="depthwise", act=g.act)
    y2 = run_gpu(g, dtype, x, w, b, r, offsets=(1, 0, 0, 2, 3))
    assert np.array_equal(_bits(y), _bits(y2))
    y3 = run_gpu(g, dtype, x, w, b, r, variant="implicit_gemm")
    assert_parity(dtype, y3, yr, sr, b, r, what="depthwise-as-igemm", act=g.act)


def _convt_cases():
    return [
        (oracle.Geom(2, 16, 5, 7, 8, 3, 3, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1, oph=1, opw=0), "f16"),
        (oracle.Geom(1, 8, 4, 4, 6, 4, 4, groups=2, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1), "f32"),
        (oracle.Geom(3, 40, 3, 6, 12, 2, 3, sh=2, sw=3, dh=1, dw=2, pt=0, pl=1, pb=0, pr=0,
                     act="tanh"), "f16"),
        (oracle.Geom(1, 5, 6, 5, 3, 3, 1, sh=1, sw=2, dh=2, pt=2, pl=0, pb=1, pr=0, opw=1,
                     act="sigmoid"), "f32"),
        (oracle.Geom(2, 64, 8, 8, 64, 2, 2, groups=4, sh=2, sw=2, act="relu"), "f16"),
    ]


@pytest.mark.parametrize("case", _convt_cases())
def test_conv_transpose_shapes(case):
    g, dtype = case
    _say(f"[convt] {dtype} {g}")
    rng = np.random.default_rng(g.c_in * 7 + g.kh)
    npdt = np.float16 if dtype == "f16" else np.float32
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(npdt)
    w = (rng.standard_normal((g.c_in, g.c_out // g.groups, g.kh, g.kw)) * 0.3).astype(npdt)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(npdt)
    r = rng.uniform(-1, 1, oracle.out_shape(g, transpose=True)).astype(npdt)
    yr, sr = oracle.conv_transpose2d(g, x, w, b, r)
    y = run_gpu(g, dtype, x, w, b, r, transpose=True)
    assert_parity(dtype, y, yr, sr, b, r, what="convt", act=g.act)
    # chunked through a one-image scratch: same bits
    y1 = run_gpu(g, dtype, x, w, b, r, transpose=True, scratch_images=1)
    assert np.array_equal(y.view(np.uint16 if dtype == "f16" else np.uint32),
                          y1.view(np.uint16 if dtype == "f16" else np.uint32))


CONVT_FUSED_CASES = [
    # (geometry, bias): kernel = stride = 2, no padding -- the GEMM epilogue
    # scatters straight into y.  Channel chunks with tails, channel tiles with
    # tails, tiles of several / one input rows, ragged last tiles.
    (oracle.Geom(1, 256, 40, 40, 64, 2, 2, sh=2, sw=2), True),
    (oracle.Geom(2, 24, 6, 12, 10, 2, 2, sh=2, sw=2, act="relu"), True),
    (oracle.Geom(3, 72, 9, 36, 6, 2, 2, sh=2, sw=2, act="silu"), False),
    (oracle.Geom(1, 16, 3, 128, 66, 2, 2, sh=2, sw=2, act="sigmoid"), True),
    (oracle.Geom(2, 8, 5, 4, 2, 2, 2, sh=2, sw=2, act="hard_swish"), True),
    (oracle.Geom(2, 130, 7, 20, 33, 2, 2, sh=2, sw=2, act="tanh"), True),
]


@pytest.mark.parametrize("case", CONVT_FUSED_CASES, ids=lambda c: f"{c[0].c_in}to{c[0].c_out}x{c[0].h}x{c[0].w}")
def test_conv_transpose_fused_k2s2(case):
    """ConvTranspose with kernel = stride = 2 through the fused GEMM + gather
    kernel against the oracle; identical bits with misaligned operands (element
    loads and stores)."""
    g, has_b = case
    _say(f"[convt-fused] {g}")
    from gpu_harness import problem_from
    name = cf.conv_describe_variant(problem_from(g, transpose=True), "f16")
    assert "fused_k2s2" in name, name
    rng = np.random.default_rng(g.c_in * 5 + g.w + 3 * g.c_out)
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(np.float16)
    w = (rng.standard_normal((g.c_in, g.c_out, 2, 2)) * np.sqrt(2.0 / g.c_in)).astype(np.float16)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(np.float16) if has_b else None
    yr, sr = oracle.conv_transpose2d(g, x, w, b, None)
    y = run_gpu(g, "f16", x, w, b, None, transpose=True)
    assert_parity("f16", y, yr, sr, b, None, what="convt-fused", act=g.act)
    y2 = run_gpu(g, "f16", x, w, b, None, transpose=True, offsets=(3, 1, 1, 0, 1))
    assert np.array_equal(_bits(y), _bits(y2))


def test_convt_checkerboard_counts():
    """All-ones input and kernel, stride 2 ('Convolutions' exercise 3): exact."""
    for k in (3, 4):
        g = oracle.Geom(1, 1, 6, 6, 1, k, k, sh=2, sw=2)
        y = run_gpu(g, "f32", np.ones((1, 1, 6, 6), np.float32), np.ones((1, 1, k, k), np.float32),
                    transpose=True)
        yr, _ = oracle.conv_transpose2d(g, np.ones((1, 1, 6, 6)), np.ones((1, 1, k, k)))
        assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_index_mapping_one_hot_probes(dtype):
    """Integer-coded inputs and one-hot weights: every output must be exactly the
    addressed input value (or 0 in padding), for each tap of the window."""
    npdt = np.float16 if dtype == "f16" else np.float32
    for g in [oracle.Geom(2, 3, 9, 11, 4, 3, 2, sh=2, sw=1, dh=1, dw=2, pt=2, pl=1, pb=0, pr=2),
              oracle.Geom(1, 4, 7, 6, 4, 2, 3, groups=2, sh=1, sw=3, dh=3, dw=1, pt=1, pl=0, pb=3, pr=1),
              oracle.Geom(1, 6, 8, 8, 12, 3, 3, groups=6, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1)]:
        x = (np.arange(g.n * g.c_in * g.h * g.w) % 1000 + 1).reshape(g.n, g.c_in, g.h, g.w)
        x = x.astype(npdt)
        assert np.all(x.astype(np.float64) == np.arange(x.size).reshape(x.shape) % 1000 + 1)
        cig = g.c_in // g.groups
        for c, u, v in itertools.product(range(cig), range(g.kh), range(g.kw)):
            w = np.zeros((g.c_out, cig, g.kh, g.kw), npdt)
            w[:, c, u, v] = 1
            y = run_gpu(g, dtype, x, w)
            yr, _ = oracle.conv2d(g, x, w)
            assert np.array_equal(y.astype(np.float64), yr), (g, c, u, v)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_integer_inputs_exact(dtype):
    """Small integers: every partial sum is exact in float32, so the GPU must
    equal the oracle exactly (identity activation, no bias)."""
    npdt = np.float16 if dtype == "f16" else np.float32
    rng = np.random.default_rng(5)
    for g, variant, splits in [
        (oracle.Geom(2, 32, 9, 9, 40, 3, 3, pt=1, pl=1, pb=1, pr=1), "implicit_gemm", 0),
        (oracle.Geom(1, 64, 6, 6, 16, 3, 3, pt=1, pl=1, pb=1, pr=1), "implicit_gemm", 3),
        (oracle.Geom(2, 8, 10, 10, 16, 5, 5, groups=8, pt=2, pl=2, pb=2, pr=2), "depthwise_direct", 0),
    ]:
        x = rng.integers(-2, 3, (g.n, g.c_in, g.h, g.w)).astype(npdt)
        w = rng.integers(-2, 3, (g.c_out, g.c_in // g.groups, g.kh, g.kw)).astype(npdt)
        y = run_gpu(g, dtype, x, w, variant=variant, splits=splits)
        yr, _ = oracle.conv2d(g, x, w)
        assert np.array_equal(y.astype(np.float64), yr.astype(npdt).astype(np.float64))


def _bits(a):
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


@pytest.mark.parametrize("name", ["w2_bottleneck3x3_f16", "w4a_depthwise5x5_f32",
                                  "w5a_dilated_grouped_f16", "w1_conv3x3_f32"])
def test_determinism_rerun(name):
    layer = workloads.BY_NAME[name].with_batch(2)
    inp = workloads.make_inputs(layer)
    g = geom_from_layer(layer)
    y1 = run_gpu(g, layer.dtype, inp.x, inp.w, inp.b, inp.r)
    y2 = run_gpu(g, layer.dtype, inp.x, inp.w, inp.b, inp.r)
    assert np.array_equal(_bits(y1), _bits(y2))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_split_k_forced_and_chunked(dtype):
    """Late-layer shape (small grid, long k): auto split, forced whole-k, forced
    R; chunking through a one-image scratch gives the same bits."""
    npdt = np.float16 if dtype == "f16" else np.float32
    g = oracle.Geom(3, 128, 7, 7, 96, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu")
    rng = np.random.default_rng(9)
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(npdt)
    w = (rng.standard_normal((g.c_out, g.c_in, 3, 3)) * 0.03).astype(npdt)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(npdt)
    r = rng.uniform(-1, 1, oracle.out_shape(g)).astype(npdt)
    yr, sr = oracle.conv2d(g, x, w, b, r)
    p = cf.make_problem(3, 128, 7, 7, 96, 3, 3, pads=(1, 1, 1, 1))
    assert int(re.search(r"split(\d+)", cf.conv_describe_variant(p, dtype)).group(1)) > 1
    outs = {}
    for splits in (0, 1, 2, 5, 16):
        y = run_gpu(g, dtype, x, w, b, r, splits=splits)
        assert_parity(dtype, y, yr, sr, b, r, what=f"splits={splits}", act=g.act)
        outs[splits] = y
        if splits != 1:
            yc = run_gpu(g, dtype, x, w, b, r, splits=splits, scratch_images=1)
            assert np.array_equal(_bits(y), _bits(yc)), splits


def test_offsets_and_alias():
    """Unaligned element offsets (arena placement) give the same bits, and y may
    alias the residual exactly."""
    layer = workloads.BY_NAME["w2_bottleneck3x3_f16"].with_batch(1)
    inp = workloads.make_inputs(layer)
    g = geom_from_layer(layer)
    y0 = run_gpu(g, "f16", inp.x, inp.w, inp.b, inp.r)
    y1 = run_gpu(g, "f16", inp.x, inp.w, inp.b, inp.r, offsets=(3, 5, 1, 7, 9))
    assert np.array_equal(_bits(y0), _bits(y1))
    y2 = run_gpu(g, "f16", inp.x, inp.w, inp.b, inp.r, offsets=(0, 0, 0, 4, 4),
                 alias_residual=True)
    assert np.array_equal(_bits(y0), _bits(y2))
    dl = workloads.BY_NAME["w4b_depthwise3x3s2_f32"].with_batch(1)
    di = workloads.make_inputs(dl)
    dg = geom_from_layer(dl)
    assert np.array_equal(_bits(run_gpu(dg, "f32", di.x, di.w, di.b)),
                          _bits(run_gpu(dg, "f32", di.x, di.w, di.b, offsets=(1, 2, 3, 0, 5))))
