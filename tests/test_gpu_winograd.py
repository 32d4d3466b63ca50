"""GPU parity of the Winograd F(2x2, 3x3) variant ("Convolutions", section 2.6;
include/conv.h, CONV_VARIANT_WINOGRAD, which a caller must ask for) against
the oracle's direct definition: integer-coded one-hot probes and small-integer
inputs (every transformed value is then exact in the 16-bit type, so the
result must be exact), seeded random geometries (odd output extents, whose
last tiles drop outputs; asymmetric pads; groups; every activation; bias and
residual) in float16 and bfloat16, reruns, and the allocation-free entry
point.  The workload-sized layer through this variant is compared in full in
test_gpu_parity.py."""
import dataclasses
import itertools

import numpy as np
import pytest

import convolution_forward_amd as cf
import oracle
import workloads
from gpu_harness import assert_parity, dev, problem_from, run_gpu, stream

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cf.lib()


def _q(a, dtype):
    return workloads.quantize(a, dtype)


def _planned(g, dtype):
    return cf.conv_describe_variant(problem_from(g, variant="winograd"), dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_index_probes_exact(dtype):
    """Integer-coded x and one-hot weights (U entries 0, +-1/4, +-1/2, 1): every
    V is a signed sum of four inputs, so x in 1..250 keeps |V| <= 1000, exact in
    float16, and x in 1..31 keeps |V| <= 124, exact in bfloat16's 8 bits; the
    products and sums are then exact and each output is the addressed input
    value (0 where the tap is padding)."""
    top = 250 if dtype == "f16" else 31
    g = oracle.Geom(2, 32, 9, 11, 48, 3, 3, pt=1, pl=2, pb=0, pr=1)
    assert _planned(g, dtype).startswith("winograd")
    x = (np.arange(g.n * g.c_in * g.h * g.w) % top + 1).reshape(g.n, g.c_in, g.h, g.w).astype(np.float32)
    T = g.c_in * 9
    for j in range(-(-T // g.c_out)):
        w = np.zeros((g.c_out, g.c_in, 3, 3), np.float32)
        for co in range(g.c_out):
            t = (co + j * g.c_out) % T
            w[co, t // 9, (t % 9) // 3, t % 3] = 1
        y = run_gpu(g, dtype, x, w, variant="winograd")
        yr, _ = oracle.conv2d(g, x, w)
        assert np.array_equal(y.astype(np.float64), yr), j


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_small_integer_inputs_exact(dtype):
    """x, w in {-1, 0, 1}, bias and residual in {-1, 0, 1}: U is a multiple of
    1/4 below 2.25 in magnitude and V an integer below 16, both exact; every
    product and sum is exact in float32, so the output equals the oracle's
    value rounded once to the type."""
    rng = np.random.default_rng(4)
    g = oracle.Geom(3, 48, 7, 10, 40, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu")
    x = rng.integers(-1, 2, (3, 48, 7, 10)).astype(np.float32)
    w = rng.integers(-1, 2, (40, 48, 3, 3)).astype(np.float32)
    b = rng.integers(-1, 2, 40).astype(np.float32)
    r = rng.integers(-1, 2, (3, 40, 7, 10)).astype(np.float32)
    y = run_gpu(g, dtype, x, w, b, r, variant="winograd")
    yr, _ = oracle.conv2d(g, x, w, b, r)
    assert np.all(np.abs(yr) < 2048)
    want = workloads.bf16_round(yr) if dtype == "bf16" else yr.astype(np.float16)
    assert np.array_equal(np.asarray(y, np.float64), np.asarray(want, np.float64))


def _sweep(seed):
    rng = np.random.default_rng(seed)
    acts = list(cf.ACTIVATIONS)
    G = int(rng.choice([1, 1, 1, 2]))
    g = oracle.Geom(int(rng.integers(1, 4)), G * 16 * int(rng.integers(1, 5)), int(rng.integers(1, 20)),
                    int(rng.integers(1, 20)), G * int(rng.choice([8, 32, 40, 64, 100])), 3, 3,
                    groups=G, pt=int(rng.integers(0, 3)), pl=int(rng.integers(0, 3)),
                    pb=int(rng.integers(0, 3)), pr=int(rng.integers(0, 3)),
                    act=acts[seed % len(acts)])
    if g.act == "clip":
        g.alpha, g.beta = -0.3, 0.4
    elif g.act == "leaky_relu":
        g.alpha = 0.1
    elif g.act == "hard_sigmoid":
        g.alpha, g.beta = 0.2, 0.5
    return g, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))


@pytest.mark.parametrize("seed", range(24))
def test_random_geometries(seed):
    g, has_b, has_r = _sweep(seed)
    try:
        shp = oracle.out_shape(g)
    except ValueError:
        pytest.skip("no window fits")
    dtype = ("f16", "bf16")[seed % 2]
    print(f"[winograd {seed}] {dtype} {_planned(g, dtype)} {g}", flush=True)
    rng = np.random.default_rng(seed + 50)
    cig = g.c_in // g.groups
    x = _q(rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)), dtype)
    w = _q(rng.standard_normal((g.c_out, cig, 3, 3)) * np.sqrt(2.0 / (9 * cig)), dtype)
    b = _q(rng.uniform(-0.1, 0.1, g.c_out), dtype) if has_b else None
    r = _q(rng.uniform(-1, 1, shp), dtype) if has_r else None
    y = run_gpu(g, dtype, x, w, b, r, variant="winograd")
    yr, sr = oracle.conv2d(g, x, w, b, r)
    assert_parity(dtype, y, yr, sr, b, r, what="winograd", act=g.act)


# Band shapes of the main kernel: a tile row longer than 32 tiles (segments of
# 32, the last one ragged), exactly 32, single-column images whose bands are 32
# tile rows, and windows whose staging needs the larger item count.
BAND_CASES = [
    oracle.Geom(1, 32, 6, 70, 40, 3, 3, pt=1, pl=1, pb=1, pr=1),
    oracle.Geom(1, 16, 5, 64, 24, 3, 3, pt=1, pl=1, pb=1, pr=1),
    oracle.Geom(1, 16, 4, 131, 8, 3, 3, pt=0, pl=2, pb=1, pr=0),
    oracle.Geom(2, 16, 80, 2, 24, 3, 3, pt=1, pl=1, pb=1, pr=1),
    oracle.Geom(2, 48, 20, 20, 32, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu"),
    oracle.Geom(3, 32, 13, 9, 72, 3, 3, pt=2, pl=0, pb=0, pr=2),
]


@pytest.mark.parametrize("case", range(len(BAND_CASES)))
def test_band_shapes(case):
    g = BAND_CASES[case]
    dtype = ("f16", "bf16")[case % 2]
    print(f"[winograd band {case}] {dtype} {_planned(g, dtype)} {g}", flush=True)
    shp = oracle.out_shape(g)
    rng = np.random.default_rng(700 + case)
    x = _q(rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)), dtype)
    w = _q(rng.standard_normal((g.c_out, g.c_in, 3, 3)) * np.sqrt(2.0 / (9 * g.c_in)), dtype)
    b = _q(rng.uniform(-0.1, 0.1, g.c_out), dtype)
    r = _q(rng.uniform(-1, 1, shp), dtype)
    y = run_gpu(g, dtype, x, w, b, r, variant="winograd")
    yr, sr = oracle.conv2d(g, x, w, b, r)
    assert_parity(dtype, y, yr, sr, b, r, what="winograd", act=g.act)


def test_rerun_bits_and_noalloc():
    layer = workloads.BY_NAME["x3_bottleneck3x3_f16_winograd"].with_batch(3)
    inp = workloads.make_inputs(layer)
    g = oracle.Geom(3, 256, 14, 14, 256, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu")
    y1 = run_gpu(g, "f16", inp.x, inp.w, inp.b, inp.r, variant="winograd")
    y2 = run_gpu(g, "f16", inp.x, inp.w, inp.b, inp.r, variant="winograd")
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    p = problem_from(g, bias=True, residual=True, variant="winograd")
    y3 = torch.empty((3, 256, 14, 14), dtype=torch.float16, device="cuda")
    cf.conv_forward_noalloc(p, "f16", dev(inp.x), dev(inp.w), dev(inp.b), dev(inp.r), y3, stream())
    torch.cuda.synchronize()
    assert np.array_equal(y1.view(np.uint16), y3.cpu().numpy().view(np.uint16))
