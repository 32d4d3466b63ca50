"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics.

Each check compares the oracle with something other than itself: values the
pages print (tests/golden/, each file cites its passage), library routines
(scipy.signal correlate/convolve, numpy matmul/einsum), closed forms, brute
force on tiny inputs, and invariants (im2col-GEMM equivalence, adjointness of
Conv and ConvTranspose).  They are chosen so that a dropped term, a flipped
kernel, a wrong sign or index, a transposed operand or an off-by-one pad fails
at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy import signal

import oracle
from oracle import Geom

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


# ---------------------------------------------------------------- extents ---

def test_printed_extents():
    """'Convolutions' section 2.1 checks, section 6 output_padding, exercise 3."""
    n = 0
    for kind, *vals in _rows("extents.txt"):
        i, k, s, d, pb, pe, op, want = map(int, vals)
        if kind == "conv":
            assert oracle.conv_extent(i, k, s, d, pb, pe) == want, vals
        else:
            assert oracle.convt_extent(i, k, s, d, pb, pe, op) == want, vals
        n += 1
    assert n == 11


def test_extent_brute_force():
    """Section 2.1 derivation: count the window starts 0, s, 2s, ... whose last
    tap (start + d(k-1)) stays inside the padded axis."""
    for L, k, s, d, pb, pe in itertools.product(range(1, 9), range(1, 5), range(1, 4),
                                                range(1, 3), range(0, 3), range(0, 3)):
        padded = L + pb + pe
        count = sum(1 for st in range(0, padded, s) if st + d * (k - 1) <= padded - 1)
        got = oracle.conv_extent(L, k, s, d, pb, pe)
        if count == 0:
            assert got is None
        else:
            assert got == count, (L, k, s, d, pb, pe)


def test_convt_extent_inverts_conv_extent():
    """ConvTranspose's size is a preimage of Conv's size map, and output_padding
    ranges over the s preimages ('Convolutions' section 6 follow-up)."""
    for L, k, s, d, p in itertools.product(range(1, 7), range(1, 5), range(1, 4),
                                           range(1, 3), range(0, 2)):
        outs = set()
        for op in range(s):
            o = oracle.convt_extent(L, k, s, d, p, p, op)
            if o is None:
                continue
            assert oracle.conv_extent(o, k, s, d, p, p) == L
            outs.add(o)
        pre = {o for o in range(1, 40) if oracle.conv_extent(o, k, s, d, p, p) == L}
        # every output_padding gives a distinct preimage; the smallest preimage
        # is op = 0 whenever it is a valid size
        assert outs <= pre
        if outs:
            assert min(outs) == min(pre)
        assert oracle.convt_extent(L, k, s, d, p, p, s) is None


def test_auto_pad_invariants():
    """ONNX auto_pad reading (parity beyond these invariants is unpinned)."""
    for L, k, s, d in itertools.product(range(1, 12), range(1, 6), range(1, 4), range(1, 3)):
        assert oracle.auto_pad(False, "VALID", L, k, s, d) == (0, 0)
        assert oracle.auto_pad(False, "NOTSET", L, k, s, d, pads=(2, 1)) == (2, 1)
        for mode in ("SAME_UPPER", "SAME_LOWER"):
            pb, pe = oracle.auto_pad(False, mode, L, k, s, d)
            assert oracle.conv_extent(L, k, s, d, pb, pe) == -(-L // s)
            need = max(0, (-(-L // s) - 1) * s + d * (k - 1) + 1 - L)
            assert pb + pe == need
            if mode == "SAME_UPPER":
                assert pe - pb in (0, 1)
            else:
                assert pb - pe in (0, 1)
    # ConvTranspose with an explicit output shape reaches that shape
    for L, k, s, out in itertools.product(range(1, 6), range(1, 5), range(1, 4), range(1, 20)):
        for mode in ("SAME_UPPER", "SAME_LOWER", "NOTSET"):
            got = oracle.auto_pad(True, mode, L, k, s, 1, 0, out)
            if got is None:
                assert s * (L - 1) + k < out
                continue
            pb, pe = got
            assert abs(pb - pe) <= 1
            assert oracle.convt_extent(L, k, s, 1, pb, pe, 0) == out


# ------------------------------------------------------------ FLOP counts ---

def test_exercise1_counts():
    """'Convolutions' exercise 1 (section 2.3 equations), printed values."""
    rows = {r[0]: r[1:] for r in _rows("exercise1.txt")}
    macs = {}
    for name in ("std3x3", "dw3x3", "pw1x1", "bneck_a", "bneck_b", "bneck_c"):
        ci, co, k, g, params, mm, dec = rows[name]
        ci, co, k, g, params, dec = int(ci), int(co), int(k), int(g), int(params), int(dec)
        geo = Geom(1, ci, 56, 56, co, k, k, groups=g, pt=k // 2, pl=k // 2, pb=k // 2,
                   pr=k // 2)
        m = oracle.conv_macs(geo)
        macs[name] = m
        assert round(m / 1e6, dec) == float(mm), (name, m)
        if params >= 0:
            p = co * (ci // g) * k * k + (co if name == "std3x3" else 0)
            assert p == params
    ratio = (macs["dw3x3"] + macs["pw1x1"]) / macs["std3x3"]
    assert round(ratio, 3) == float(rows["ratio"][0])
    assert math.isclose(ratio, 1 / 128 + 1 / 9, rel_tol=1e-12)
    total = macs["bneck_a"] + macs["bneck_b"] + macs["bneck_c"]
    assert round(total / 1e6) == int(rows["bneck_total"][0])


# ------------------------------------------------------------ Conv values ---

def _rng(seed):
    return np.random.default_rng(seed)


def test_worked_example_windows():
    """'Convolutions' section 1: 4x4 * 3x3 -> 2x2 and the printed windows."""
    rows = list(_rows("worked_example.txt"))
    _, ih, iw, k, oh, ow = rows[0]
    g = Geom(1, 1, int(ih), int(iw), 1, int(k), int(k))
    assert oracle.out_shape(g) == (1, 1, int(oh), int(ow))
    # distinct powers of two mark every input cell: the all-ones kernel's output
    # names exactly the cells of each window
    x = (2.0 ** np.arange(16)).reshape(1, 1, 4, 4)
    w = np.ones((1, 1, 3, 3))
    y, _ = oracle.conv2d(g, x, w)
    for _, r, c, r0, r1, c0, c1 in rows[1:]:
        r, c, r0, r1, c0, c1 = map(int, (r, c, r0, r1, c0, c1))
        assert y[0, 0, r, c] == x[0, 0, r0:r1 + 1, c0:c1 + 1].sum()
    # the unfold is 9 x 4 and the 1 x 9 kernel row times it gives the outputs
    cols = np.stack([x[0, 0, i:i + 3, j:j + 3].ravel() for i in range(2) for j in range(2)],
                    axis=1)
    assert cols.shape == (9, 4)
    wr = _rng(3).standard_normal((1, 1, 3, 3))
    y2, _ = oracle.conv2d(g, x, wr)
    np.testing.assert_allclose(y2.ravel(), (wr.reshape(1, 9) @ cols).ravel(), rtol=1e-13)


@pytest.mark.parametrize("case", [
    # H, W, KH, KW, pads (t, l, b, r)
    (7, 9, 3, 3, (1, 1, 1, 1)),
    (6, 5, 2, 4, (0, 2, 1, 0)),
    (8, 8, 5, 5, (2, 2, 2, 2)),
    (5, 7, 1, 3, (0, 0, 0, 0)),
])
def test_single_channel_matches_scipy_correlate(case):
    """Conv is cross-correlation (no flip) with zero padding: scipy's
    correlate2d of the zero-padded input ('Convolutions' TL;DR and section 3)."""
    H, W, KH, KW, (pt, pl, pb, pr) = case
    rng = _rng(11)
    x = rng.standard_normal((1, 1, H, W))
    w = rng.standard_normal((1, 1, KH, KW))
    g = Geom(1, 1, H, W, 1, KH, KW, pt=pt, pl=pl, pb=pb, pr=pr)
    y, s = oracle.conv2d(g, x, w)
    xp = np.pad(x[0, 0], ((pt, pb), (pl, pr)))
    ref = signal.correlate2d(xp, w[0, 0], mode="valid")
    np.testing.assert_allclose(y[0, 0], ref, rtol=1e-12, atol=1e-12)
    # the scale is the same correlation of absolute values
    ref_s = signal.correlate2d(np.abs(xp), np.abs(w[0, 0]), mode="valid")
    np.testing.assert_allclose(s[0, 0], ref_s, rtol=1e-12, atol=1e-12)
    # and a flipped kernel (true convolution) is different
    conv = signal.convolve2d(xp, w[0, 0], mode="valid")
    assert not np.allclose(conv, ref)


def test_stride_is_subsampled_stride1_and_dilation_is_holey_kernel():
    rng = _rng(12)
    H, W = 11, 10
    x = rng.standard_normal((1, 1, H, W))
    w = rng.standard_normal((1, 1, 3, 3))
    for sh, sw, dh, dw, p in [(2, 3, 1, 1, 1), (1, 1, 2, 3, 2), (2, 2, 2, 1, 0), (3, 1, 1, 2, 3)]:
        g = Geom(1, 1, H, W, 1, 3, 3, sh=sh, sw=sw, dh=dh, dw=dw, pt=p, pl=p, pb=p, pr=p)
        y, _ = oracle.conv2d(g, x, w)
        wd = np.zeros((dh * 2 + 1, dw * 2 + 1))
        wd[::dh, ::dw] = w[0, 0]
        full = signal.correlate2d(np.pad(x[0, 0], p), wd, mode="valid")
        ref = full[::sh, ::sw]
        assert y.shape[2:] == ref.shape
        np.testing.assert_allclose(y[0, 0], ref, rtol=1e-12, atol=1e-12)


def test_channels_sum_and_groups_are_block_diagonal():
    """Multi-channel = sum of single-channel correlations; groups = independent
    convs on contiguous channel blocks ('Convolutions' TL;DR; exercise 4)."""
    rng = _rng(13)
    N, Ci, Co, G, H, W = 2, 6, 4, 2, 6, 7
    x = rng.standard_normal((N, Ci, H, W))
    w = rng.standard_normal((Co, Ci // G, 3, 3))
    b = rng.standard_normal(Co)
    g = Geom(N, Ci, H, W, Co, 3, 3, groups=G, pt=1, pl=1, pb=1, pr=1)
    y, _ = oracle.conv2d(g, x, w, b)
    cig, cog = Ci // G, Co // G
    for n in range(N):
        for co in range(Co):
            grp = co // cog
            ref = b[co] + sum(
                signal.correlate2d(np.pad(x[n, grp * cig + c], 1), w[co, c], mode="valid")
                for c in range(cig))
            np.testing.assert_allclose(y[n, co], ref, rtol=1e-12, atol=1e-12)


def test_depthwise_with_multiplier():
    """Depthwise (groups = Cin): output co reads input channel co // m."""
    rng = _rng(14)
    N, C, m, H, W = 2, 3, 2, 5, 6
    x = rng.standard_normal((N, C, H, W))
    w = rng.standard_normal((C * m, 1, 3, 3))
    g = Geom(N, C, H, W, C * m, 3, 3, groups=C, sh=2, sw=1, pt=1, pl=0, pb=1, pr=2)
    y, _ = oracle.conv2d(g, x, w)
    for n in range(N):
        for co in range(C * m):
            xp = np.pad(x[n, co // m], ((1, 1), (0, 2)))
            ref = signal.correlate2d(xp, w[co, 0], mode="valid")[::2, :]
            np.testing.assert_allclose(y[n, co], ref, rtol=1e-12, atol=1e-12)


def test_pointwise_is_matrix_product():
    """1x1, stride 1, no pad: Y_n = W X_n ('Convolutions' section 6)."""
    rng = _rng(15)
    N, Ci, Co, H, W = 3, 5, 7, 4, 6
    x = rng.standard_normal((N, Ci, H, W))
    w = rng.standard_normal((Co, Ci, 1, 1))
    g = Geom(N, Ci, H, W, Co, 1, 1)
    y, _ = oracle.conv2d(g, x, w)
    ref = np.matmul(w[:, :, 0, 0], x.reshape(N, Ci, H * W)).reshape(N, Co, H, W)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def _random_geoms():
    rng = _rng(16)
    out = []
    while len(out) < 24:
        G = int(rng.choice([1, 1, 2, 3]))
        cig, cog = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        kh, kw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        g = Geom(int(rng.integers(1, 3)), cig * G, int(rng.integers(1, 9)),
                 int(rng.integers(1, 9)), cog * G, kh, kw, groups=G,
                 sh=int(rng.integers(1, 4)), sw=int(rng.integers(1, 4)),
                 dh=int(rng.integers(1, 3)), dw=int(rng.integers(1, 3)),
                 pt=int(rng.integers(0, 3)), pl=int(rng.integers(0, 3)),
                 pb=int(rng.integers(0, 3)), pr=int(rng.integers(0, 3)))
        try:
            oracle.out_shape(g)
        except ValueError:
            continue
        out.append(g)
    return out


def test_direct_equals_im2col_gemm():
    """im2col-GEMM equivalence ('Convolutions' sections 1 and 2.4)."""
    rng = _rng(17)
    for g in _random_geoms():
        x = rng.standard_normal((g.n, g.c_in, g.h, g.w))
        w = rng.standard_normal((g.c_out, g.c_in // g.groups, g.kh, g.kw))
        b = rng.standard_normal(g.c_out)
        r = rng.standard_normal(oracle.out_shape(g))
        y, _ = oracle.conv2d(g, x, w, b, r)
        y2 = oracle.conv2d_im2col(g, x, w, b, r)
        np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)
        # integer-valued inputs: every partial sum is exact, so the two orders agree bit for bit
        xi = rng.integers(-3, 4, x.shape).astype(np.float64)
        wi = rng.integers(-3, 4, w.shape).astype(np.float64)
        assert np.array_equal(oracle.conv2d(g, xi, wi)[0], oracle.conv2d_im2col(g, xi, wi))


def test_brute_force_tiny():
    """Pure-Python loops on tiny problems (definition re-derived from ONNX Conv:
    x_pad[b, c, i*s + u*d, j*s + v*d] * w[o, c, u, v])."""
    rng = _rng(18)
    for g in _random_geoms()[:10]:
        x = rng.standard_normal((g.n, g.c_in, g.h, g.w))
        w = rng.standard_normal((g.c_out, g.c_in // g.groups, g.kh, g.kw))
        y, _ = oracle.conv2d(g, x, w)
        xp = np.zeros((g.n, g.c_in, g.h + g.pt + g.pb, g.w + g.pl + g.pr))
        xp[:, :, g.pt:g.pt + g.h, g.pl:g.pl + g.w] = x
        cig, cog = g.c_in // g.groups, g.c_out // g.groups
        for n, o, i, j in itertools.product(*(range(v) for v in y.shape)):
            grp = o // cog
            acc = 0.0
            for c, u, v in itertools.product(range(cig), range(g.kh), range(g.kw)):
                acc += xp[n, grp * cig + c, i * g.sh + u * g.dh, j * g.sw + v * g.dw] * w[o, c, u, v]
            assert math.isclose(y[n, o, i, j], acc, rel_tol=1e-12, abs_tol=1e-12)


def test_points_match_full():
    rng = _rng(19)
    g = Geom(2, 4, 9, 8, 6, 3, 2, groups=2, sh=2, dw=2, pt=1, pl=1, pb=1, pr=2, act="silu")
    x = rng.standard_normal((g.n, g.c_in, g.h, g.w))
    w = rng.standard_normal((g.c_out, 2, g.kh, g.kw))
    b = rng.standard_normal(g.c_out)
    r = rng.standard_normal(oracle.out_shape(g))
    y, s = oracle.conv2d(g, x, w, b, r)
    idx = rng.choice(y.size, 50, replace=False)
    yp, sp = oracle.conv2d_points(g, x, w, b, r, idx)
    np.testing.assert_array_equal(yp, y.ravel()[idx])
    np.testing.assert_array_equal(sp, s.ravel()[idx])


def test_epilogue_order_and_activations():
    """Sum, then bias, then residual, then activation ('Convolution, pooling and
    resize', 'Layout and operands'); activations at closed-form points."""
    a = oracle.activation
    assert a("relu", -1.5) == 0.0 and a("relu", 2.0) == 2.0
    assert a("sigmoid", 0.0) == 0.5 and a("tanh", 0.0) == 0.0
    assert a("hard_swish", -3.0) == 0.0 and a("hard_swish", 3.0) == 3.0
    assert a("hard_swish", 1.5) == 1.5 * (1.5 / 6 + 0.5)
    assert a("hard_sigmoid", -2.5, 0.2, 0.5) == 0.0 and a("hard_sigmoid", 2.5, 0.2, 0.5) == 1.0
    assert a("hard_sigmoid", 1.0, 0.2, 0.5) == 0.2 + 0.5
    assert a("silu", 0.0) == 0.0 and math.isclose(a("silu", 2.0), 2.0 / (1 + math.exp(-2.0)))
    assert a("clip", 5.0, -1.0, 2.0) == 2.0 and a("clip", -5.0, -1.0, 2.0) == -1.0
    assert a("leaky_relu", -2.0, 0.01) == -0.02 and a("leaky_relu", 3.0, 0.01) == 3.0
    assert math.isclose(a("tanh", 0.5), math.tanh(0.5)) and math.isclose(
        a("sigmoid", -1.0), 1 / (1 + math.e))
    # order: a 1x1 identity conv of x with weight 1 gives act(x + b + r)
    x = np.array([-0.7, 0.2, 1.3]).reshape(1, 1, 1, 3)
    w = np.ones((1, 1, 1, 1))
    b = np.array([0.25])
    r = np.array([0.5, -0.75, 0.1]).reshape(1, 1, 1, 3)
    for act in ("relu", "sigmoid", "hard_swish"):
        y, s = oracle.conv2d(Geom(1, 1, 1, 3, 1, 1, 1, act=act), x, w, b, r)
        ref = [a(act, v + 0.25 + rr) for v, rr in zip(x.ravel(), r.ravel())]
        np.testing.assert_allclose(y.ravel(), ref, rtol=1e-15)
        np.testing.assert_array_equal(s.ravel(), np.abs(x.ravel()))


# ----------------------------------------------------- ConvTranspose values ---

def _convt_geoms():
    return [
        Geom(1, 1, 5, 4, 1, 3, 3, sh=2, sw=2),
        Geom(2, 4, 4, 5, 6, 3, 2, groups=2, sh=2, sw=3, pt=1, pl=0, pb=1, pr=1, oph=1),
        Geom(1, 3, 3, 3, 2, 2, 2, sh=2, sw=2),
        Geom(2, 2, 4, 3, 4, 3, 3, groups=2, sh=1, sw=2, dh=2, dw=1, pt=2, pl=1, pb=1, pr=0,
             opw=1),
        Geom(1, 6, 3, 4, 3, 4, 4, groups=3, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1),
    ]


def test_convt_scatter_equals_gather():
    rng = _rng(21)
    for g in _convt_geoms():
        x = rng.standard_normal((g.n, g.c_in, g.h, g.w))
        w = rng.standard_normal((g.c_in, g.c_out // g.groups, g.kh, g.kw))
        b = rng.standard_normal(g.c_out)
        y, _ = oracle.conv_transpose2d(g, x, w, b)
        y2 = oracle.conv_transpose2d_gather(g, x, w, b)
        np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)


def test_convt_is_adjoint_of_conv():
    """<Conv(x; w), y> = <x, ConvT(y; w)> ('Convolutions' section 2.4: the input
    gradient of a correlation is what ConvTranspose computes)."""
    rng = _rng(22)
    for g in _convt_geoms():
        # ConvT maps (Cin_t, H) -> (Cout_t, Ho); the Conv with the same weights
        # maps (Cout_t, Ho) -> (Cin_t, H).
        _, cot, ho, wo = oracle.out_shape(g, transpose=True)
        gc = Geom(g.n, cot, ho, wo, g.c_in, g.kh, g.kw, groups=g.groups, sh=g.sh, sw=g.sw,
                  dh=g.dh, dw=g.dw, pt=g.pt, pl=g.pl, pb=g.pb, pr=g.pr)
        assert oracle.out_shape(gc) == (g.n, g.c_in, g.h, g.w)
        w = rng.standard_normal((g.c_in, g.c_out // g.groups, g.kh, g.kw))
        u = rng.standard_normal((g.n, cot, ho, wo))
        v = rng.standard_normal((g.n, g.c_in, g.h, g.w))
        cu, _ = oracle.conv2d(gc, u, w)
        tv, _ = oracle.conv_transpose2d(g, v, w)
        lhs, rhs = float(np.sum(cu * v)), float(np.sum(u * tv))
        assert math.isclose(lhs, rhs, rel_tol=1e-11, abs_tol=1e-11), (lhs, rhs)


def test_convt_single_channel_matches_scipy_full_convolution():
    """Stride-s ConvT of one channel = full convolution (kernel flipped) of the
    input with s-1 zeros inserted between samples, then cropped by the pads."""
    rng = _rng(23)
    for H, W, k, s, p, op in [(4, 5, 3, 1, 0, 0), (5, 4, 3, 2, 1, 1), (3, 3, 4, 2, 1, 0),
                              (4, 4, 2, 2, 0, 0), (3, 5, 3, 3, 2, 2)]:
        x = rng.standard_normal((1, 1, H, W))
        w = rng.standard_normal((1, 1, k, k))
        g = Geom(1, 1, H, W, 1, k, k, sh=s, sw=s, pt=p, pl=p, pb=p, pr=p, oph=op, opw=op)
        y, _ = oracle.conv_transpose2d(g, x, w)
        up = np.zeros(((H - 1) * s + 1, (W - 1) * s + 1))
        up[::s, ::s] = x[0, 0]
        full = signal.convolve2d(up, w[0, 0], mode="full")
        full = np.pad(full, ((0, op), (0, op)))
        ref = full[p:full.shape[0] - p, p:full.shape[1] - p]
        assert y.shape[2:] == ref.shape
        np.testing.assert_allclose(y[0, 0], ref, rtol=1e-12, atol=1e-12)


def test_checkerboard_counts():
    """'Convolutions' section 2.5 / exercise 3 (golden/checkerboard.txt)."""
    for k, ee, eo, oe, oo in (map(int, r) for r in _rows("checkerboard.txt")):
        g = Geom(1, 1, 6, 6, 1, k, k, sh=2, sw=2)
        y, _ = oracle.conv_transpose2d(g, np.ones((1, 1, 6, 6)), np.ones((1, 1, k, k)))
        y = y[0, 0]
        assert y.shape == ((6 - 1) * 2 + k,) * 2
        inner = range(k - 1, 2 * 6 - 1 - k + 1)  # positions every input window can reach
        for i in inner:
            for j in inner:
                want = {(0, 0): ee, (0, 1): eo, (1, 0): oe, (1, 1): oo}[(i % 2, j % 2)]
                assert y[i, j] == want, (k, i, j)


def test_convt_k_equals_s_is_pointwise_then_depth_to_space():
    """k = s, no pad: no overlap ('Convolutions' section 2.5), so each output is
    one tap: a 1x1 conv into Cout*k*k channels followed by depth-to-space."""
    rng = _rng(24)
    N, Ci, Co, H, W, k = 2, 5, 3, 3, 4, 2
    x = rng.standard_normal((N, Ci, H, W))
    w = rng.standard_normal((Ci, Co, k, k))
    b = rng.standard_normal(Co)
    y, s = oracle.conv_transpose2d(Geom(N, Ci, H, W, Co, k, k, sh=k, sw=k), x, w, b)
    ref = np.einsum("nchw,cjuv->njhuwv", x, w).reshape(N, Co, H * k, W * k) + b[None, :, None, None]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    ref_s = np.einsum("nchw,cjuv->njhuwv", np.abs(x), np.abs(w)).reshape(N, Co, H * k, W * k)
    np.testing.assert_allclose(s, ref_s, rtol=1e-12, atol=1e-12)


def test_rejects_bad_geometry():
    with pytest.raises(ValueError):
        oracle.out_shape(Geom(1, 1, 2, 2, 1, 5, 5))
    assert oracle.conv_extent(4, 3, 0, 1, 0, 0) is None
    assert oracle.convt_extent(4, 3, 2, 1, 0, 0, 2) is None
