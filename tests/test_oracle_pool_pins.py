"""Pins of the pooling oracle ("Convolution, pooling and resize", section
"Pooling and resize": padding, dilation, ceil_mode dropping a last window that
starts inside the end padding, count_include_pad counting padding taps but not
taps beyond it, max skipping NaN unless all are NaN, the lowest finite value for
an empty max window, NaN for an empty average, global pools over a plane).

The oracle is compared with something other than itself: PyTorch's CPU pooling
in float64 (a library routine, symmetric pads only), a numpy formulation over
an explicitly padded array (asymmetric pads), brute-force window counts, hand
values and numpy reductions.  A wrong window start, a dropped or extra window,
a wrong divisor or a wrong NaN rule fails at least one of them.
"""
import itertools
import math
import warnings

import numpy as np
import pytest

import oracle
from oracle import PoolGeom

torch = pytest.importorskip("torch")
F = torch.nn.functional


def _brute_extent(n, k, s, d, pb, pe, ceil_mode):
    """Window starts 0, s, 2s, ... on the padded axis of length L = n+pb+pe.
    Floor mode keeps the windows whose last tap is inside the padded axis.
    Ceil mode takes windows until one reaches the end of the padded axis (the
    fewest windows that cover it), then drops that last window once if it
    starts inside the end padding (start - pb >= n)."""
    L, keff = n + pb + pe, d * (k - 1) + 1
    if keff > L:
        return None
    if not ceil_mode:
        return len([st for st in range(0, L, s) if st + keff <= L])
    taken = []
    st = 0
    while True:
        taken.append(st)
        if st + keff >= L:
            break
        st += s
    if taken[-1] - pb >= n:
        taken.pop()
    return len(taken) or None


def test_extent_brute_force():
    for n, k, s, d, pb, pe, cm in itertools.product(range(1, 10), range(1, 5), range(1, 4),
                                                    range(1, 3), range(0, 3), range(0, 3),
                                                    (False, True)):
        assert oracle.pool_extent(n, k, s, d, pb, pe, cm) == _brute_extent(n, k, s, d, pb, pe, cm), \
            (n, k, s, d, pb, pe, cm)


def test_extents_match_torch_shapes():
    for n, k, s, p, cm in itertools.product(range(2, 12), range(1, 5), range(1, 4), range(0, 3),
                                            (False, True)):
        if p > k // 2 or k > n + 2 * p:
            continue
        got = oracle.pool_extent(n, k, s, 1, p, p, cm)
        want = F.max_pool2d(torch.zeros(1, 1, n, n, dtype=torch.float64), k, s, p,
                            ceil_mode=cm).shape[-1]
        assert got == want, (n, k, s, p, cm)


def test_hand_values():
    x = np.arange(16, dtype=np.float64).reshape(1, 1, 4, 4)
    y, _ = oracle.pool2d(PoolGeom(1, 1, 4, 4, 2, 2, 2, 2, kind="max"), x)
    assert np.array_equal(y[0, 0], [[5, 7], [13, 15]])
    y, s = oracle.pool2d(PoolGeom(1, 1, 4, 4, 2, 2, 2, 2, kind="average"), x)
    assert np.array_equal(y[0, 0], [[2.5, 4.5], [10.5, 12.5]])
    assert np.array_equal(s, y)  # non-negative inputs: mean |x| = mean x
    ones = np.ones((1, 1, 3, 3))
    g = PoolGeom(1, 1, 3, 3, 3, 3, pt=1, pl=1, pb=1, pr=1, kind="average",
                 count_include_pad=True)
    y, _ = oracle.pool2d(g, ones)
    assert np.allclose(y[0, 0], [[4 / 9, 6 / 9, 4 / 9], [6 / 9, 1, 6 / 9], [4 / 9, 6 / 9, 4 / 9]])
    g.count_include_pad = False
    y, _ = oracle.pool2d(g, ones)
    assert np.array_equal(y[0, 0], np.ones((3, 3)))


def test_ceil_mode_drops_window_starting_in_end_padding():
    # 3 inputs, k2 s2 p1: windows start at -1, 1 and 3; the third starts in the
    # end padding and is dropped (2 outputs, not 3)
    assert oracle.pool_extent(3, 2, 2, 1, 1, 1, True) == 2
    x = np.array([1.0, 5.0, 3.0]).reshape(1, 1, 1, 3)
    y, _ = oracle.pool2d(PoolGeom(1, 1, 1, 3, 1, 2, 1, 2, pl=1, pr=1, kind="max", ceil_mode=True), x)
    assert np.array_equal(y.ravel(), [1.0, 5.0])
    # 5 inputs, k2 s2, no pads: ceil keeps the partial last window [x4]
    x = np.array([1.0, 2.0, 3.0, 4.0, 9.0]).reshape(1, 1, 1, 5)
    g = PoolGeom(1, 1, 1, 5, 1, 2, 1, 2, kind="average", ceil_mode=True)
    y, _ = oracle.pool2d(g, x)
    assert np.array_equal(y.ravel(), [1.5, 3.5, 9.0])
    # beyond the padding never counts, even with count_include_pad
    g.count_include_pad = True
    y, _ = oracle.pool2d(g, x)
    assert np.array_equal(y.ravel(), [1.5, 3.5, 9.0])


def test_nan_and_empty_windows():
    nan = float("nan")
    x = np.array([nan, 1.0, 2.0, nan]).reshape(1, 1, 2, 2)
    y, _ = oracle.pool2d(PoolGeom(1, 1, 2, 2, 2, 2, kind="max"), x)
    assert y.ravel()[0] == 2.0
    y, _ = oracle.pool2d(PoolGeom(1, 1, 2, 2, 2, 2, kind="max"), np.full((1, 1, 2, 2), nan))
    assert np.isnan(y.ravel()[0])
    # a 1x1 input with 2 of padding on each side and a 1x1 window: outputs at
    # the padding see no input element
    g = PoolGeom(1, 1, 1, 1, 1, 1, pt=2, pl=2, pb=2, pr=2, kind="max")
    for dt in ("f32", "f16", "bf16"):
        y, _ = oracle.pool2d(g, np.full((1, 1, 1, 1), 7.0), dtype=dt)
        assert y.shape == (1, 1, 5, 5)
        assert y[0, 0, 2, 2] == 7.0
        assert y[0, 0, 0, 0] == oracle.LOWEST[dt]
    assert oracle.LOWEST["f32"] == float(np.finfo(np.float32).min)
    assert oracle.LOWEST["f16"] == float(np.finfo(np.float16).min)
    assert oracle.LOWEST["bf16"] == float(torch.finfo(torch.bfloat16).min)
    g.kind = "average"
    y, _ = oracle.pool2d(g, np.full((1, 1, 1, 1), 7.0))
    assert y[0, 0, 2, 2] == 7.0 and np.isnan(y[0, 0, 0, 0])
    g.count_include_pad = True  # padding taps count: 0 / 1
    y, _ = oracle.pool2d(g, np.full((1, 1, 1, 1), 7.0))
    assert y[0, 0, 0, 0] == 0.0


def test_signed_zeros():
    for a, b in ((-0.0, 0.0), (0.0, -0.0)):
        x = np.array([a, b]).reshape(1, 1, 1, 2)
        y, _ = oracle.pool2d(PoolGeom(1, 1, 1, 2, 1, 2, kind="max"), x)
        assert y.ravel()[0] == 0.0 and not math.copysign(1.0, y.ravel()[0]) < 0
        y, _ = oracle.global_pool("max", x)
        assert not math.copysign(1.0, y.ravel()[0]) < 0


def _torch_cases():
    rng = np.random.default_rng(11)
    out = []
    while len(out) < 60:
        k = int(rng.integers(1, 5))
        p = int(rng.integers(0, k // 2 + 1))
        g = PoolGeom(int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(k, 13)),
                     int(rng.integers(k, 13)), k, k, *(int(rng.integers(1, 4)),) * 2,
                     pt=p, pl=p, pb=p, pr=p, ceil_mode=bool(rng.integers(0, 2)))
        out.append(g)
    return out


@pytest.mark.parametrize("i", range(60))
def test_max_and_average_match_torch(i):
    g = _torch_cases()[i]
    rng = np.random.default_rng(i)
    x = rng.standard_normal((g.n, g.c, g.h, g.w))
    xt = torch.from_numpy(x)
    d = int(rng.integers(1, 3))
    gm = PoolGeom(**{**g.__dict__, "dh": d, "dw": d, "kind": "max"})
    try:
        ym, _ = oracle.pool2d(gm, x)
        tm = F.max_pool2d(xt, g.kh, g.sh, g.pt, dilation=d, ceil_mode=g.ceil_mode).numpy()
        assert ym.shape == tm.shape and np.array_equal(ym, tm)
    except (ValueError, RuntimeError):
        pass  # no window fits at this dilation: both sides refuse
    for cip in (False, True):
        ga = PoolGeom(**{**g.__dict__, "kind": "average", "count_include_pad": cip})
        ya, _ = oracle.pool2d(ga, x)
        ta = F.avg_pool2d(xt, g.kh, g.sh, g.pt, ceil_mode=g.ceil_mode,
                          count_include_pad=cip).numpy()
        assert ya.shape == ta.shape
        assert np.allclose(ya, ta, rtol=1e-12, atol=1e-12), (g, cip)


def test_asymmetric_pads_match_padded_sliding_windows():
    """Floor mode with separate begin and end pads: pad the array explicitly
    (NaN marks padding), take every window with numpy's sliding view, and
    reduce: max over the real values, mean over real (+ padding) values."""
    rng = np.random.default_rng(5)
    for _ in range(40):
        kh, kw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        sh, sw, dh, dw = (int(v) for v in rng.integers(1, 3, 4))
        pt, pl, pb, pr = (int(v) for v in rng.integers(0, 3, 4))
        h, w = int(rng.integers(3, 9)), int(rng.integers(3, 9))
        g = PoolGeom(1, 2, h, w, kh, kw, sh, sw, dh, dw, pt, pl, pb, pr)
        try:
            shp = oracle.pool_out_shape(g)
        except ValueError:
            continue
        x = rng.standard_normal((1, 2, h, w))
        xp = np.pad(x, ((0, 0), (0, 0), (pt, pb), (pl, pr)), constant_values=np.nan)
        win = np.lib.stride_tricks.sliding_window_view(
            xp, ((kh - 1) * dh + 1, (kw - 1) * dw + 1), axis=(2, 3))
        win = win[:, :, ::sh, ::sw, ::dh, ::dw][:, :, :shp[2], :shp[3]]
        ym, _ = oracle.pool2d(g, x)
        empty = ~np.isfinite(win).any(axis=(4, 5))  # only padding under the window
        with np.errstate(invalid="ignore", divide="ignore"), warnings.catch_warnings():
            warnings.simplefilter("ignore")
            want = np.where(empty, oracle.LOWEST["f32"], np.nanmax(win, axis=(4, 5)))
            assert np.array_equal(ym, want)
            for cip in (False, True):
                g.kind, g.count_include_pad = "average", cip
                ya, _ = oracle.pool2d(g, x)
                real = np.nansum(win, axis=(4, 5))
                cnt = np.isfinite(win).sum(axis=(4, 5)) if not cip else win.shape[4] * win.shape[5]
                assert np.allclose(ya, real / cnt, rtol=1e-13, atol=1e-13, equal_nan=True)
                g.kind = "max"


def test_global_pools_match_numpy():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 5, 7, 9))
    x[0, 1, 2, 3] = np.nan
    x[1, 2] = np.nan
    y, s = oracle.global_pool("average", np.nan_to_num(x))
    assert np.allclose(y[:, :, 0, 0], np.nan_to_num(x).mean(axis=(2, 3)), rtol=1e-14)
    assert np.allclose(s[:, :, 0, 0], np.abs(np.nan_to_num(x)).mean(axis=(2, 3)), rtol=1e-14)
    y, _ = oracle.global_pool("max", x)
    with np.errstate(invalid="ignore"), __import__("warnings").catch_warnings():
        __import__("warnings").simplefilter("ignore")
        want = np.nanmax(x, axis=(2, 3))
    assert np.array_equal(y[:, :, 0, 0], want, equal_nan=True)
