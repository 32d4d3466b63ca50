"""GPU parity of ConvInteger (include/conv_integer.h) against the oracle, bit
for bit ("Convolution, pooling and resize", "Tolerances": ConvInteger is
bit-exact int32): all four uint8/int8 mixes, per-tensor, per-channel and absent
zero points, seeded random geometries (groups, stride, dilation, asymmetric
pads, 1-D), extreme values whose sums wrap modulo 2^32, a reduction long
enough that the kernel's accumulator is flushed more than once, the workload
layer at full size, element offsets and reruns."""
import numpy as np
import pytest

import convolution_forward_amd as cf
import oracle
import workloads
from gpu_harness import dev, problem_from, stream

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

NPT = {"u8": np.uint8, "i8": np.int8}


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cf.lib()


def run_int(g, xt, wt, x, w, xz, wz, per_channel, offsets=(0, 0, 0)):
    """x, w: integer arrays of the operands' values; wz scalar or per channel;
    xz / wz None for an absent (zero) zero point."""
    p = problem_from(g, offsets=(offsets[0], offsets[1], 0, 0, offsets[2]))
    ho, wo = cf.conv_output_extent(p)
    xs = np.zeros(offsets[0] + x.size, np.uint8)
    xs[offsets[0]:] = np.asarray(x).astype(NPT[xt]).view(np.uint8).ravel()
    ws = np.zeros(offsets[1] + w.size, np.uint8)
    ws[offsets[1]:] = np.asarray(w).astype(NPT[wt]).view(np.uint8).ravel()
    ysize = g.n * g.c_out * ho * wo
    yd = dev(np.full(offsets[2] + ysize, 0x5A5A5A5A, np.int32))
    xzd = None if xz is None else dev(np.array([xz]).astype(NPT[xt]).view(np.uint8))
    wzd = None
    if wz is not None:
        wzv = np.asarray(wz).reshape(-1)
        wzd = dev(wzv.astype(NPT[wt]).view(np.uint8))
    cf.conv_integer_forward(p, xt, wt, dev(xs), dev(ws), xzd, wzd, per_channel, yd, stream())
    torch.cuda.synchronize()
    return yd.cpu().numpy()[offsets[2]:].reshape(g.n, g.c_out, ho, wo)


def check(g, xt, wt, x, w, xz, wz, per_channel, offsets=(0, 0, 0)):
    y = run_int(g, xt, wt, x, w, xz, wz, per_channel, offsets)
    yr = oracle.conv_integer(g, x, w, 0 if xz is None else xz,
                             0 if wz is None else (wz if per_channel else int(np.asarray(wz).reshape(-1)[0])))
    bad = y != yr
    assert not bad.any(), f"{int(bad.sum())} of {y.size} outputs differ; first at {np.argwhere(bad)[0]}"
    return y


LO = {"u8": 0, "i8": -128}


def _rand(rng, t, shape):
    return rng.integers(LO[t], LO[t] + 256, shape)


@pytest.mark.parametrize("seed", range(24))
def test_random_geometries_all_type_mixes(seed):
    rng = np.random.default_rng(seed)
    xt, wt = ("u8", "i8")[seed % 2], ("u8", "i8")[(seed // 2) % 2]
    G = int(rng.choice([1, 1, 2, 4]))
    g = oracle.Geom(int(rng.integers(1, 4)), G * int(rng.integers(1, 24)), int(rng.integers(1, 16)),
                    int(rng.integers(1, 16)), G * int(rng.integers(1, 40)), int(rng.integers(1, 5)),
                    int(rng.integers(1, 5)), groups=G, sh=int(rng.integers(1, 3)),
                    sw=int(rng.integers(1, 3)), dh=int(rng.integers(1, 3)), dw=int(rng.integers(1, 3)),
                    pt=int(rng.integers(0, 3)), pl=int(rng.integers(0, 3)), pb=int(rng.integers(0, 3)),
                    pr=int(rng.integers(0, 3)))
    try:
        oracle.out_shape(g)
    except ValueError:
        pytest.skip("no window fits")
    per_channel = seed % 3 == 0
    x = _rand(rng, xt, (g.n, g.c_in, g.h, g.w))
    w = _rand(rng, wt, (g.c_out, g.c_in // G, g.kh, g.kw))
    xz = None if seed % 5 == 4 else int(_rand(rng, xt, ()))
    wz = _rand(rng, wt, (g.c_out,)) if per_channel else (None if seed % 7 == 6 else int(_rand(rng, wt, ())))
    print(f"[convint {seed}] {xt}{wt} pc={per_channel} {g}", flush=True)
    check(g, xt, wt, x, w, xz, wz, per_channel)


def test_one_dimensional():
    g = oracle.Geom(2, 24, 1, 300, 40, 1, 5, sw=2, dw=3, pl=4, pr=1)
    rng = np.random.default_rng(1)
    check(g, "i8", "u8", _rand(rng, "i8", (2, 24, 1, 300)), _rand(rng, "u8", (40, 24, 1, 5)),
          -7, _rand(rng, "u8", (40,)), 1)


@pytest.mark.parametrize("types", [("u8", "i8"), ("u8", "u8"), ("i8", "i8"), ("i8", "u8")])
def test_extreme_values_wrap_around(types):
    """Every input and weight at an end of its range, the zero points at the other
    end: 36,864 taps of products of magnitude about 2^16 sum beyond 2^31, so
    the int32 results wrap."""
    xt, wt = types
    g = oracle.Geom(1, 4096, 3, 3, 4, 3, 3, pt=1, pl=1, pb=1, pr=1)
    hi = {"u8": 255, "i8": 127}
    x = np.full((1, 4096, 3, 3), hi[xt])
    w = np.empty((4, 4096, 3, 3), np.int64)
    w[0], w[1], w[2], w[3] = LO[wt], hi[wt], LO[wt] + 1, hi[wt] - 1
    wz = np.array([hi[wt], LO[wt], LO[wt], hi[wt]])
    y = check(g, xt, wt, x, w, LO[xt], wz, 1)
    assert np.abs(y.astype(np.int64)).max() > 2 ** 29


def test_long_reduction_flushes_accumulator():
    """147,456 taps (2,304 k-blocks): the MFMA accumulator is added into the
    wrapping totals twice before the end."""
    g = oracle.Geom(1, 16384, 2, 2, 3, 3, 3, pt=1, pl=1, pb=1, pr=1)
    rng = np.random.default_rng(2)
    x = _rand(rng, "u8", (1, 16384, 2, 2))
    x[:, : 8192] = 255
    w = _rand(rng, "i8", (3, 16384, 3, 3))
    w[0] = -128
    check(g, "u8", "i8", x, w, 0, np.array([127, 0, -3]), 1)


@pytest.mark.parametrize("seed", range(16))
def test_rowshift_geometries(seed):
    """The row-shift kernel (3x3 stride 1, rows of at most 14 outputs, 128k
    channels per group) over random pads, extents (both row counts, planes
    of pixel counts not a multiple of 4), groups, channel counts that leave a
    partial 32-channel tile, all type mixes and zero-point forms, and element
    offsets that break the x, w and y alignments."""
    rng = np.random.default_rng(900 + seed)
    xt, wt = ("u8", "i8")[seed % 2], ("u8", "i8")[(seed // 2) % 2]
    G = int(rng.choice([1, 2]))
    while True:
        g = oracle.Geom(int(rng.integers(1, 4)), G * 128 * int(rng.integers(1, 3)),
                        int(rng.integers(1, 15)), int(rng.integers(1, 15)),
                        G * int(rng.choice([8, 32, 40, 64])), 3, 3, groups=G,
                        pt=int(rng.integers(0, 3)), pl=int(rng.integers(0, 3)),
                        pb=int(rng.integers(0, 3)), pr=int(rng.integers(0, 3)))
        try:
            _, _, ho, wo = oracle.out_shape(g)
        except ValueError:
            continue
        if ho <= 14 and wo <= 14:
            break
    p = problem_from(g)
    assert ".rowshift." in cf.conv_integer_describe_variant(p, xt, wt)
    per_channel = seed % 3 != 2
    x = _rand(rng, xt, (g.n, g.c_in, g.h, g.w))
    w = _rand(rng, wt, (g.c_out, g.c_in // G, 3, 3))
    xz = None if seed % 5 == 4 else int(_rand(rng, xt, ()))
    wz = _rand(rng, wt, (g.c_out,)) if per_channel else (None if seed % 4 == 3 else int(_rand(rng, wt, ())))
    offsets = ((0, 0, 0), (1, 0, 0), (0, 3, 0), (0, 0, 1))[seed % 4]
    print(f"[convint rowshift {seed}] {xt}{wt} pc={per_channel} off={offsets} {g}", flush=True)
    check(g, xt, wt, x, w, xz, wz, per_channel, offsets=offsets)


@pytest.mark.parametrize("name", [l.name for l in workloads.INT_LAYERS])
def test_workload_layer_full_size(name):
    l = workloads.INT_BY_NAME[name]
    x, w, xz, wz = workloads.make_int_inputs(l)
    g = oracle.Geom(l.n, l.c_in, l.h, l.w, l.c_out, l.kh, l.kw, groups=l.groups, sh=l.stride[0],
                    sw=l.stride[1], dh=l.dilation[0], dw=l.dilation[1], pt=l.pads[0],
                    pl=l.pads[1], pb=l.pads[2], pr=l.pads[3])
    print(f"[convint-full] {name} {cf.conv_integer_describe_variant(problem_from(g), l.x_type, l.w_type)}",
          flush=True)
    check(g, l.x_type, l.w_type, x, w, xz, wz, 1)


def test_offsets_and_rerun():
    g = oracle.Geom(2, 20, 9, 7, 12, 3, 2, sh=2, pt=1, pl=0, pb=1, pr=1)
    rng = np.random.default_rng(3)
    x, w = _rand(rng, "u8", (2, 20, 9, 7)), _rand(rng, "i8", (12, 20, 3, 2))
    a = check(g, "u8", "i8", x, w, 17, -5, 0)
    b = check(g, "u8", "i8", x, w, 17, -5, 0, offsets=(3, 7, 5))
    c = run_int(g, "u8", "i8", x, w, 17, -5, 0)
    assert np.array_equal(a, b) and np.array_equal(a, c)
