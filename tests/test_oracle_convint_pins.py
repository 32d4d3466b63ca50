"""Pins of the ConvInteger oracle ("Convolution, pooling and resize", section
"ConvInteger": y = sum (x - xZero) * (w - wZero[m]) in int32 with wrap-around,
uint8 and int8 operands in any mix, one x zero point, w zero points per tensor
or per output channel, the geometry of the float convolution, a padded tap
being the quantized value xZero so that it adds nothing).

Compared with: the float oracle on the same integer values (zero points 0, no
wrap: a different code path), and a numpy int64 formulation that pads with
the zero point, gathers every window with a sliding view, multiplies and sums
exactly in Python integers, then wraps modulo 2^32 -- including extreme values
whose sums leave the int32 range.
"""
import numpy as np
import pytest

import oracle
from oracle import Geom


def _wrap32(v):
    v = np.asarray(v, dtype=object) % (1 << 32)
    return np.where(v >= (1 << 31), v - (1 << 32), v).astype(np.int64)


def _numpy_convinteger(g, x, w, xz, wz):
    """Pad with xz, gather windows, exact integer products."""
    xp = np.pad(x.astype(np.int64), ((0, 0), (0, 0), (g.pt, g.pb), (g.pl, g.pr)),
                constant_values=xz)
    win = np.lib.stride_tricks.sliding_window_view(
        xp, ((g.kh - 1) * g.dh + 1, (g.kw - 1) * g.dw + 1), axis=(2, 3))
    win = win[:, :, ::g.sh, ::g.sw, ::g.dh, ::g.dw]  # n, c, ho, wo, kh, kw
    n, c, ho, wo = win.shape[:4]
    cig, cog = g.c_in // g.groups, g.c_out // g.groups
    wzv = np.broadcast_to(np.asarray(wz, np.int64), (g.c_out,))
    y = np.zeros((n, g.c_out, ho, wo), dtype=object)
    for co in range(g.c_out):
        gi = co // cog
        xs = win[:, gi * cig:(gi + 1) * cig] - xz            # n, cig, ho, wo, kh, kw
        ws = w[co].astype(np.int64) - wzv[co]                 # cig, kh, kw
        y[:, co] = np.einsum("ncijab,cab->nij", xs.astype(object), ws.astype(object))
    return _wrap32(y)


def _case(rng, g, xt, wt, per_channel):
    lo = {"u8": 0, "i8": -128}
    x = rng.integers(lo[xt], lo[xt] + 256, (g.n, g.c_in, g.h, g.w))
    w = rng.integers(lo[wt], lo[wt] + 256, (g.c_out, g.c_in // g.groups, g.kh, g.kw))
    xz = int(rng.integers(lo[xt], lo[xt] + 256))
    wz = rng.integers(lo[wt], lo[wt] + 256, g.c_out) if per_channel else int(
        rng.integers(lo[wt], lo[wt] + 256))
    return x, w, xz, wz


@pytest.mark.parametrize("xt", ["u8", "i8"])
@pytest.mark.parametrize("wt", ["u8", "i8"])
def test_matches_numpy_padded_windows(xt, wt):
    rng = np.random.default_rng(len(xt + wt) * 7 + (xt == "u8") + 2 * (wt == "u8"))
    for i in range(12):
        G = int(rng.choice([1, 2]))
        g = Geom(int(rng.integers(1, 3)), G * int(rng.integers(1, 4)), int(rng.integers(1, 9)),
                 int(rng.integers(1, 9)), G * int(rng.integers(1, 4)), int(rng.integers(1, 4)),
                 int(rng.integers(1, 4)), groups=G, sh=int(rng.integers(1, 3)),
                 sw=int(rng.integers(1, 3)), dh=int(rng.integers(1, 3)), dw=int(rng.integers(1, 3)),
                 pt=int(rng.integers(0, 3)), pl=int(rng.integers(0, 3)), pb=int(rng.integers(0, 3)),
                 pr=int(rng.integers(0, 3)))
        try:
            oracle.out_shape(g)
        except ValueError:
            continue
        x, w, xz, wz = _case(rng, g, xt, wt, per_channel=bool(i % 2))
        y = oracle.conv_integer(g, x, w, xz, wz)
        assert np.array_equal(y, _numpy_convinteger(g, x, w, xz, wz)), (g, xz)


def test_zero_points_zero_is_the_float_convolution():
    rng = np.random.default_rng(4)
    for G in (1, 2, 4):
        g = Geom(2, 4 * G, 9, 7, 2 * G, 3, 2, groups=G, sh=2, pt=1, pl=0, pb=2, pr=1)
        x = rng.integers(0, 256, (g.n, g.c_in, g.h, g.w))
        w = rng.integers(-128, 128, (g.c_out, g.c_in // G, g.kh, g.kw))
        yf, _ = oracle.conv2d(g, x.astype(np.float64), w.astype(np.float64))
        assert np.array_equal(oracle.conv_integer(g, x, w, 0, 0), yf.astype(np.int64))


def test_padding_adds_nothing():
    """A zero point equal to every input value makes every term zero, padded
    taps included; a padded tap with a nonzero zero point is still skipped."""
    g = Geom(1, 2, 4, 4, 3, 3, 3, pt=2, pl=2, pb=2, pr=2)
    x = np.full((1, 2, 4, 4), 77)
    w = np.random.default_rng(0).integers(-128, 128, (3, 2, 3, 3))
    assert not oracle.conv_integer(g, x, w, 77, 5).any()
    # one real input element at the corner: only windows covering it are nonzero
    x = np.zeros((1, 1, 1, 1), np.int64)
    x[0, 0, 0, 0] = 9
    g = Geom(1, 1, 1, 1, 1, 3, 3, pt=1, pl=1, pb=1, pr=1)
    w = np.ones((1, 1, 3, 3), np.int64)
    y = oracle.conv_integer(g, x, w, 2, 0)
    assert y.shape == (1, 1, 1, 1) and y[0, 0, 0, 0] == 7


def test_wraps_modulo_2_32():
    """36864 taps of (255 - 0) * (-128 - 127) = -65025 each: -2,397,081,600,
    below -2^31; and of 255 * 127 each: +1,193,877,... above 2^31 with more."""
    g = Geom(1, 4096, 3, 3, 2, 3, 3, pt=1, pl=1, pb=1, pr=1)
    x = np.full((1, 4096, 3, 3), 255)
    w = np.empty((2, 4096, 3, 3), np.int64)
    w[0] = -128
    w[1] = 127
    y = oracle.conv_integer(g, x, w, 0, [127, -128])
    taps = np.array([[4, 6, 4], [6, 9, 6], [4, 6, 4]]) * 4096
    want0 = _wrap32(taps * 255 * (-128 - 127))
    want1 = _wrap32(taps * 255 * (127 + 128))
    assert np.array_equal(y[0, 0], want0) and np.array_equal(y[0, 1], want1)
    assert (taps * 255 * 255).max() > 2 ** 31  # the case does wrap
    assert y[0, 0, 1, 1] == int(_wrap32(9 * 4096 * 255 * -255))


def test_one_dimensional_as_height_one():
    rng = np.random.default_rng(8)
    g = Geom(2, 3, 1, 40, 5, 1, 3, sw=2, dw=2, pl=2, pr=1)
    x = rng.integers(-128, 128, (2, 3, 1, 40))
    w = rng.integers(0, 256, (5, 3, 1, 3))
    y = oracle.conv_integer(g, x, w, -3, 200)
    ref = np.zeros_like(y, dtype=np.int64)
    xp = np.pad(x, ((0, 0), (0, 0), (0, 0), (2, 1)), constant_values=-3)
    for n, co, ow in np.ndindex(2, 5, y.shape[3]):
        acc = 0
        for ci in range(3):
            for k in range(3):
                acc += (int(xp[n, ci, 0, ow * 2 + k * 2]) + 3) * (int(w[co, ci, 0, k]) - 200)
        ref[n, co, 0, ow] = acc
    assert np.array_equal(y, _wrap32(ref))
