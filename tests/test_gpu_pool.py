"""GPU parity of the pooling forward (include/pool.h) against the fp64 oracle.

MaxPool and GlobalMaxPool are compared bit for bit (the result is one of the
inputs, the type's lowest finite value or NaN; NaN compares as NaN, and the
sign of zero is checked).  AveragePool and GlobalAveragePool are held to the
stated tolerance ("Convolution, pooling and resize", "Tolerances": 1e-5 for
float32, 2e-3 for half) scaled by the mean |x| over the divisor, plus half an
ulp of the output type for the final store; bfloat16 takes 1.6e-2 (4 units of
its roundoff, as for the convolution).  Cases: the workload pools at full
size, seeded random geometries (every dtype, floor and ceil mode, padding
counted or not, pads beyond the window so that windows are empty), NaN, +-0
and infinities, rows too wide to stage (direct kernel), planes above one
4096-element chunk, element offsets and reruns.
"""
import numpy as np
import pytest

import convolution_forward_amd as cf
import oracle
import workloads
from gpu_harness import TOL, NP, bound, dev, from_storage, stream, to_storage

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cf.lib()


def _say(*a):
    print(*a, flush=True)


def _problem(g, kind, offsets=(0, 0)):
    if kind.startswith("global"):
        return cf.make_pool_problem(g.n, g.c, g.h, g.w, kind, offsets=offsets)
    return cf.make_pool_problem(g.n, g.c, g.h, g.w, kind, kernel=(g.kh, g.kw),
                                stride=(g.sh, g.sw), dilation=(g.dh, g.dw),
                                pads=(g.pt, g.pl, g.pb, g.pr), ceil_mode=g.ceil_mode,
                                count_include_pad=g.count_include_pad, offsets=offsets)


def run_pool(g, kind, dtype, x, offsets=(0, 0)):
    p = _problem(g, kind, offsets)
    ho, wo = cf.pool_output_extent(p)
    npdt = NP[dtype]
    xs = np.zeros(offsets[0] + x.size, npdt)
    xs[offsets[0]:] = to_storage(x, dtype).ravel()
    ysize = g.n * g.c * ho * wo
    ys = np.zeros(offsets[1] + ysize, npdt)
    ys[offsets[1]:] = to_storage(np.full(ysize, 8192.0), dtype)  # a sentinel
    xd, yd = dev(xs), dev(ys)
    cf.pool_forward(p, dtype, xd, yd, stream())
    torch.cuda.synchronize()
    return from_storage(yd.cpu().numpy()[offsets[1]:], dtype).reshape(g.n, g.c, ho, wo)


def _stored(v, dtype):
    """Oracle values that are exact in the element type, as stored bits."""
    v = np.asarray(v, np.float64)
    if dtype == "bf16":  # exact in bfloat16: the upper half of the float32 bits
        b = v.astype(np.float32).view(np.uint32)
        assert not np.any(b & 0xFFFF)
        return b >> 16
    return v.astype(NP[dtype]).view(np.uint16 if dtype == "f16" else np.uint32)


def assert_max_exact(y, yr, dtype, what=""):
    y = np.asarray(y)
    nan_r, nan_g = np.isnan(yr), np.isnan(y.astype(np.float64))
    assert np.array_equal(nan_r, nan_g), f"{what}: NaN positions differ"
    ok = ~nan_r
    got = _stored(y.astype(np.float64)[ok], dtype)
    want = _stored(yr[ok], dtype)
    bad = got != want
    if bad.any():
        i = np.argwhere(bad)[0][0]
        raise AssertionError(f"{what}: {int(bad.sum())} max outputs differ; first gpu="
                             f"{y.astype(np.float64)[ok][i]!r} oracle={yr[ok][i]!r}")


def assert_avg(y, yr, scale, dtype, what=""):
    y = np.asarray(y, np.float64)
    nan_r = np.isnan(yr)
    assert np.array_equal(nan_r, np.isnan(y)), f"{what}: NaN positions differ"
    ok = ~nan_r
    lim = bound(dtype, yr[ok], scale[ok], act="identity")
    err = np.abs(y[ok] - yr[ok])
    assert np.all(err <= lim), f"{what}: max err/bound {float((err / lim).max()):.3g}"
    return float((err / np.maximum(lim, 1e-300)).max()) if err.size else 0.0


def check(g, kind, dtype, x, offsets=(0, 0)):
    y = run_pool(g, kind, dtype, x, offsets)
    if kind.startswith("global"):
        yr, sr = oracle.global_pool(kind.split("_")[1], x)
    else:
        g.kind = kind
        yr, sr = oracle.pool2d(g, x, dtype=dtype)
    if kind.endswith("max"):
        assert_max_exact(y, yr, dtype, what=f"{kind} {dtype}")
        return 0.0
    return assert_avg(y, yr, sr, dtype, what=f"{kind} {dtype}")


def _q(a, dtype):
    return workloads.quantize(a, dtype)


@pytest.mark.parametrize("name", [l.name for l in workloads.POOL_LAYERS])
def test_pool_workload_full_size(name):
    l = workloads.POOL_BY_NAME[name]
    x = workloads.make_pool_input(l)
    g = oracle.PoolGeom(l.n, l.c, l.h, l.w, l.kernel[0], l.kernel[1], l.stride[0], l.stride[1],
                        l.dilation[0], l.dilation[1], *l.pads, ceil_mode=l.ceil_mode,
                        count_include_pad=l.count_include_pad)
    _say(f"[pool-full] {name} {cf.pool_describe_variant(_problem(g, l.kind), l.dtype)}")
    q = check(g, l.kind, l.dtype, x)
    _say(f"  max err/bound {q:.3g}")


def _sweep(seed):
    rng = np.random.default_rng(seed)
    k = (int(rng.integers(1, 5)), int(rng.integers(1, 5)))
    g = oracle.PoolGeom(int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(1, 22)),
                        int(rng.integers(1, 22)), k[0], k[1], int(rng.integers(1, 4)),
                        int(rng.integers(1, 4)), int(rng.integers(1, 3)), int(rng.integers(1, 3)),
                        *(int(v) for v in rng.integers(0, 4, 4)),
                        ceil_mode=bool(rng.integers(0, 2)),
                        count_include_pad=bool(rng.integers(0, 2)))
    return g, ("f32", "f16", "bf16")[seed % 3], ("max", "average")[(seed // 3) % 2]


@pytest.mark.parametrize("seed", range(48))
def test_pool_random_geometries(seed):
    g, dtype, kind = _sweep(seed)
    try:
        oracle.pool_out_shape(g)
    except ValueError:
        pytest.skip("no window fits")
    _say(f"[pool sweep {seed}] {kind} {dtype} {g}")
    x = _q(np.random.default_rng(seed + 7).uniform(-2, 2, (g.n, g.c, g.h, g.w)), dtype)
    check(g, kind, dtype, x)


def _sweep_rowvec(seed):
    """A random geometry the row-vector kernel takes: windows of 2 or 3 taps,
    horizontal stride 1 or 2, rows of whole 16-byte vectors, a left pad and a
    right reach of at most one 32-bit word."""
    rng = np.random.default_rng(5000 + seed)
    dtype = ("f32", "f16", "bf16")[seed % 3]
    v, we = (4, 1) if dtype == "f32" else (8, 2)
    while True:
        kh, kw, sw = int(rng.integers(2, 4)), int(rng.integers(2, 4)), int(rng.integers(1, 3))
        pl = int(rng.integers(0, we + 1))
        if kw - sw - pl > we:
            continue
        g = oracle.PoolGeom(int(rng.integers(1, 4)), int(rng.integers(1, 6)),
                            int(rng.integers(1, 21)), v * int(rng.integers(1, 9)), kh, kw,
                            int(rng.integers(1, 4)), sw, 1, 1, int(rng.integers(0, 3)), pl,
                            int(rng.integers(0, 3)), int(rng.integers(0, 3)),
                            ceil_mode=bool(rng.integers(0, 2)),
                            count_include_pad=bool(rng.integers(0, 2)))
        try:
            _, _, _, wo = oracle.pool_out_shape(g)
        except ValueError:
            continue
        if -(-wo // (v // sw)) * v >= g.w:
            return g, dtype, ("max", "average")[(seed // 3) % 2]


@pytest.mark.parametrize("seed", range(36))
def test_pool_rowvec_geometries(seed):
    """The row-vector kernel over random geometries (several waves per row
    block, so that neighbour columns cross wave ends), with x and y at element
    offsets that break the vector alignment on every third case."""
    g, dtype, kind = _sweep_rowvec(seed)
    p = _problem(g, kind)
    assert ".rowvec" in cf.pool_describe_variant(p, dtype), cf.pool_describe_variant(p, dtype)
    offsets = ((0, 0), (1, 0), (0, 3))[seed % 3]
    _say(f"[pool rowvec {seed}] {kind} {dtype} {offsets} {g}")
    x = _q(np.random.default_rng(seed + 11).uniform(-2, 2, (g.n, g.c, g.h, g.w)), dtype)
    check(g, kind, dtype, x, offsets=offsets)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_pool_special_values(dtype):
    """NaN taps skipped unless all are NaN, -0 below +0, infinities, and windows
    that see only padding (pads wider than the window)."""
    rng = np.random.default_rng(3)
    x = _q(rng.uniform(-1, 1, (2, 3, 9, 10)), dtype).astype(np.float32)
    x[0, 0, :3, :3] = np.nan                  # an all-NaN window
    x[0, 1, ::2, 1::3] = np.nan               # NaN among numbers
    x[1, 0] = -0.0
    x[1, 0, 4, 4] = 0.0                       # +0 among -0
    x[1, 1, 2, :] = -np.inf
    x[1, 2, :, :] = -np.inf                   # only -inf: the max is -inf
    x[0, 2, 5, 5] = np.inf
    for kind in ("max", "average"):
        for cip in (False, True):
            g = oracle.PoolGeom(2, 3, 9, 10, 3, 3, 2, 2, 1, 1, 4, 4, 4, 4, ceil_mode=True,
                                count_include_pad=cip)
            _say(f"[pool special] {dtype} {kind} cip={cip}")
            y = run_pool(g, kind, dtype, x)
            g.kind = kind
            yr, sr = oracle.pool2d(g, x, dtype=dtype)
            if kind == "max":
                assert_max_exact(y, yr, dtype, "special max")
                assert np.all(y[yr == oracle.LOWEST[dtype]] == oracle.LOWEST[dtype])
            else:
                fin = np.isfinite(yr)
                assert np.array_equal(np.isnan(y), np.isnan(yr))
                assert np.array_equal(y[~fin & ~np.isnan(yr)], yr[~fin & ~np.isnan(yr)])
                assert_avg(np.where(fin, y, 0), np.where(fin, yr, 0), np.where(fin, sr, 0), dtype)
    for kind in ("global_max", "global_average"):
        xx = x.copy() if kind == "global_max" else np.nan_to_num(x, posinf=0.0, neginf=0.0)
        g = oracle.PoolGeom(2, 3, 9, 10)
        check(g, kind, dtype, xx)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_pool_rowvec_special_values(dtype):
    """NaN, +-0 and infinities on rows of whole 16-byte vectors (the row-vector
    kernel), x aligned and at an element offset: an all-NaN window, NaN among
    numbers at the row ends and in the middle, -0 beside +0, rows of -inf
    only, +inf; windows that reach past both row ends and past the last row."""
    v = 4 if dtype == "f32" else 8
    w = 3 * v
    rng = np.random.default_rng(31)
    x = _q(rng.uniform(-1, 1, (2, 3, 9, w)), dtype).astype(np.float32)
    x[0, 0, :2, :2] = np.nan                  # an all-NaN window (top-left corner)
    x[0, 1, ::2, ::3] = np.nan                # NaN among numbers
    x[0, 1, 4, w - 1] = np.nan                # NaN at a row's last column
    x[0, 2, :, 0] = np.nan                    # NaN down the first column
    x[1, 0] = -0.0
    x[1, 0, 4, 4] = 0.0                       # +0 among -0
    x[1, 1, 2, :] = -np.inf
    x[1, 2, :, :] = -np.inf                   # only -inf: the max is -inf
    x[0, 2, 5, 5] = np.inf
    for kind in ("max", "average"):
        for (k, s_, p, cm) in (((3, 3), 2, (1, 1, 1, 1), True), ((2, 2), 2, (0, 0, 1, 1), True),
                               ((3, 3), 1, (1, 1, 1, 1), False), ((3, 2), 2, (2, 0, 2, 0), True)):
            g = oracle.PoolGeom(2, 3, 9, w, k[0], k[1], s_, s_, 1, 1, *p, ceil_mode=cm,
                                count_include_pad=False)
            pp = _problem(g, kind)
            assert ".rowvec" in cf.pool_describe_variant(pp, dtype), cf.pool_describe_variant(pp, dtype)
            g.kind = kind
            yr, sr = oracle.pool2d(g, x, dtype=dtype)
            for off in ((0, 0), (1, 0)):
                _say(f"[pool rowvec special] {dtype} {kind} {k} s{s_} {p} ceil={cm} off={off}")
                y = run_pool(g, kind, dtype, x, offsets=off)
                if kind == "max":
                    assert_max_exact(y, yr, dtype, "rowvec special max")
                else:
                    fin = np.isfinite(yr)
                    assert np.array_equal(np.isnan(y), np.isnan(yr))
                    assert np.array_equal(y[~fin & ~np.isnan(yr)], yr[~fin & ~np.isnan(yr)])
                    assert_avg(np.where(fin, y, 0), np.where(fin, yr, 0), np.where(fin, sr, 0), dtype)


def test_pool_direct_kernel_wide_rows():
    for kind in ("max", "average"):
        # 6001 columns: not whole vectors (no row-vector kernel), and three
        # rows of them do not fit the band kernel's LDS
        g = oracle.PoolGeom(1, 2, 5, 6001, 3, 3, 1, 2, pt=1, pl=1, pb=1, pr=1)
        p = _problem(g, kind)
        assert cf.pool_describe_variant(p, "f32").endswith(".direct")
        x = np.random.default_rng(1).uniform(-1, 1, (1, 2, 5, 6001)).astype(np.float32)
        check(g, kind, "f32", x)


@pytest.mark.parametrize("hw", [(1, 1), (1, 7), (7, 7), (14, 14), (64, 64), (1, 4097),
                                (100, 100), (112, 112)])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_global_pools(hw, dtype):
    h, w = hw
    n, c = (2, 3) if h * w > 1000 else (3, 37)
    x = _q(np.random.default_rng(h * w).uniform(-1, 1, (n, c, h, w)), dtype)
    g = oracle.PoolGeom(n, c, h, w)
    for kind in ("global_max", "global_average"):
        _say(f"[global] {kind} {dtype} {hw} {cf.pool_describe_variant(_problem(g, kind), dtype)}")
        check(g, kind, dtype, x)


def test_offsets_and_rerun_bits():
    g = oracle.PoolGeom(4, 5, 13, 11, 3, 2, 2, 1, pt=1, pl=0, pb=1, pr=1)
    x = np.random.default_rng(9).uniform(-1, 1, (4, 5, 13, 11)).astype(np.float16)
    for kind in ("max", "average", "global_average"):
        a = run_pool(g, kind, "f16", x)
        b = run_pool(g, kind, "f16", x, offsets=(3, 5))
        c = run_pool(g, kind, "f16", x)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), kind
        assert np.array_equal(a.view(np.uint16), c.view(np.uint16)), kind
        check(g, kind, "f16", x, offsets=(1, 2))
