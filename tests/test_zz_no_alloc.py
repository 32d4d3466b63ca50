"""conv_forward_noalloc (the library's static scratch, no allocation) against
conv_forward / conv_transpose_forward with caller scratch, through the C ABI.

Same plan and kernels, so the outputs must be bit-identical; each case makes
two calls in a row on the shared array, the second with a smaller input, so
the second finds the first's leftovers in it.  Also: a batch whose scratch
exceeds the 64 MiB array runs in chunks of whole images (same bits), a
problem whose single image needs more is refused before anything runs, and
the outputs meet the oracle's bound.
"""
import numpy as np
import pytest

import convolution_forward_amd as cf
import oracle
from gpu_harness import assert_parity, dev, problem_from, stream

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

LIMIT = 64 << 20


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cf.lib()


def _inputs(g, dtype, tr, seed):
    npdt = np.float16 if dtype == "f16" else np.float32
    rng = np.random.default_rng(seed)
    x = rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)).astype(npdt)
    ws = (g.c_in, g.c_out // g.groups, g.kh, g.kw) if tr else (g.c_out, g.c_in // g.groups, g.kh, g.kw)
    w = (rng.standard_normal(ws) * np.sqrt(2.0 / (ws[1] * g.kh * g.kw))).astype(npdt)
    b = rng.uniform(-0.1, 0.1, g.c_out).astype(npdt)
    return x, w, b


def _both(g, dtype, tr, seed, splits=0):
    """(y from the scratch-taking call, y from the no-alloc call, oracle check)."""
    print(f"[noalloc] {dtype} tr={tr} splits={splits} {g}", flush=True)
    x, w, b = _inputs(g, dtype, tr, seed)
    p = problem_from(g, transpose=tr, bias=True, splits=splits)
    print(f"  {cf.conv_describe_variant(p, dtype)} scratch {cf.conv_scratch_size(p, dtype)}",
          flush=True)
    ho, wo = cf.conv_output_extent(p)
    tdt = torch.float16 if dtype == "f16" else torch.float32
    xd, wd, bd = dev(x), dev(w), dev(b)
    y1 = torch.full((g.n, g.c_out, ho, wo), float("nan"), dtype=tdt, device="cuda")
    y2 = torch.full_like(y1, float("nan"))
    whole, _ = cf.conv_scratch_size(p, dtype)
    sc = torch.empty(max(whole, 16) // 4, dtype=torch.float32, device="cuda") if whole else None
    fn = cf.conv_transpose_forward if tr else cf.conv_forward
    fn(p, dtype, xd, wd, bd, None, y1, sc, whole if sc is not None else 0, stream())
    cf.conv_forward_noalloc(p, dtype, xd, wd, bd, None, y2, stream())
    torch.cuda.synchronize()
    a, c = y1.cpu().numpy(), y2.cpu().numpy()
    ref = oracle.conv_transpose2d if tr else oracle.conv2d
    yr, sr = ref(g, x, w, b)
    assert_parity(dtype, c, yr, sr, b, what="noalloc", act=g.act)
    return a, c, whole


def _bits(a):
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


CASES = [
    # (geometry, dtype, transpose, second call's batch, split ranges): split-k
    # Conv (forced R, so both batches keep the plan; R = 0 lets the planner
    # split the one-image call), general ConvTranspose (float32 columns), and a
    # plan without scratch
    (oracle.Geom(3, 512, 7, 7, 512, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu"), "f16", False, 1, 16),
    (oracle.Geom(1, 512, 7, 7, 512, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu"), "f16", False, 1, 0),
    (oracle.Geom(2, 128, 7, 7, 96, 3, 3, pt=1, pl=1, pb=1, pr=1), "f32", False, 1, 5),
    (oracle.Geom(4, 24, 9, 10, 16, 3, 3, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1), "f16", True, 2, 0),
    (oracle.Geom(3, 16, 6, 7, 8, 4, 4, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1), "f32", True, 1, 0),
    (oracle.Geom(4, 64, 14, 14, 64, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu"), "f16", False, 2, 0),
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: f"{c[1]}-{'convT' if c[2] else 'conv'}-{c[0].c_in}-r{c[4]}")
def test_noalloc_matches_scratch_call_twice(case):
    g, dtype, tr, n2, splits = case
    import dataclasses
    for i, n in enumerate((g.n, n2)):
        gi = dataclasses.replace(g, n=n)
        a, c, _ = _both(gi, dtype, tr, seed=100 + i, splits=splits)
        assert np.array_equal(_bits(a), _bits(c)), (i, n)


def test_noalloc_chunks_past_the_array():
    """1.6 MB of split-k planes per image: 50 images need 80 MB, more than the
    64 MiB array, so the call runs in chunks of whole images."""
    g = oracle.Geom(50, 512, 7, 7, 512, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu")
    a, c, whole = _both(g, "f16", False, seed=7, splits=16)
    assert whole > LIMIT
    assert np.array_equal(_bits(a), _bits(c))


def test_noalloc_refuses_images_beyond_the_array():
    """Forcing 16 ranges onto 18 k-blocks gives 9 ranges of 2048 x 32 x 32
    float32 sums, 72 MiB per image: refused before anything is enqueued."""
    p = cf.make_problem(1, 64, 32, 32, 2048, 3, 3, pads=(1, 1, 1, 1), splits=16)
    whole, per = cf.conv_scratch_size(p, "f16")
    assert per > LIMIT
    x = torch.zeros(64 * 32 * 32, dtype=torch.float16, device="cuda")
    w = torch.zeros(2048 * 64 * 9, dtype=torch.float16, device="cuda")
    y = torch.zeros(2048 * 32 * 32, dtype=torch.float16, device="cuda")
    st = cf.conv_forward_noalloc(p, "f16", x, w, None, None, y, stream(), check=False)
    assert st == cf.CONV_ERR_SCRATCH
