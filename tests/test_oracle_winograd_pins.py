"""Pins of the Winograd F(2x2, 3x3) formulation of the oracle ("Convolutions",
section 2.6; Lavin and Gray 2016).  The transforms reach exactly the
cross-correlation, so in fp64 the formulation must equal the direct
definition to rounding (a wrong transform matrix, a flipped tile, a dropped
border tile or a wrong output index fails by O(1)); the 1-D F(2, 3)
identities are checked by hand, and shapes the method does not cover are
refused."""
import numpy as np
import pytest

import oracle
from oracle import Geom


def test_one_dimensional_f23_identities():
    """m1..m4 of F(2, 3) recombine to the 2 outputs of a 3-tap correlation:
    y0 = d0 g0 + d1 g1 + d2 g2, y1 = d1 g0 + d2 g1 + d3 g2 (the 2-D oracle on
    a 1 x 4 input with a 1-row kernel placed in the middle row)."""
    rng = np.random.default_rng(0)
    for _ in range(20):
        d = rng.standard_normal(4)
        gk = rng.standard_normal(3)
        x = np.zeros((1, 1, 3, 4))
        x[0, 0, 1] = d
        w = np.zeros((1, 1, 3, 3))
        w[0, 0, 1] = gk
        y = oracle.conv2d_winograd(Geom(1, 1, 3, 4, 1, 3, 3, pl=0, pt=0), x, w)
        assert y.shape == (1, 1, 1, 2)
        assert np.allclose(y.ravel(), [d[0] * gk[0] + d[1] * gk[1] + d[2] * gk[2],
                                       d[1] * gk[0] + d[2] * gk[1] + d[3] * gk[2]], rtol=1e-13,
                           atol=1e-13)


@pytest.mark.parametrize("seed", range(16))
def test_equals_direct_definition(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.choice([1, 1, 2]))
    g = Geom(int(rng.integers(1, 3)), G * int(rng.integers(1, 5)), int(rng.integers(1, 12)),
             int(rng.integers(1, 12)), G * int(rng.integers(1, 5)), 3, 3, groups=G,
             pt=int(rng.integers(0, 3)), pl=int(rng.integers(0, 3)), pb=int(rng.integers(0, 3)),
             pr=int(rng.integers(0, 3)), act=("identity", "relu", "sigmoid")[seed % 3])
    try:
        shp = oracle.out_shape(g)
    except ValueError:
        pytest.skip("no window fits")
    x = rng.standard_normal((g.n, g.c_in, g.h, g.w))
    w = rng.standard_normal((g.c_out, g.c_in // G, 3, 3))
    b = rng.standard_normal(g.c_out)
    r = rng.standard_normal(shp)
    yd, s = oracle.conv2d(g, x, w, b, r)
    yw = oracle.conv2d_winograd(g, x, w, b, r)
    assert np.all(np.abs(yw - yd) <= 1e-12 * (1 + s + np.abs(b)[None, :, None, None] + np.abs(r)))


def test_refuses_other_shapes():
    x = np.zeros((1, 1, 8, 8))
    for g in (Geom(1, 1, 8, 8, 1, 3, 3, sh=2), Geom(1, 1, 8, 8, 1, 3, 3, dh=2),
              Geom(1, 1, 8, 8, 1, 5, 5)):
        with pytest.raises(ValueError):
            oracle.conv2d_winograd(g, x, np.zeros((1, 1, g.kh, g.kw)))
