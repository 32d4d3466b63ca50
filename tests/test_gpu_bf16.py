"""GPU parity of the bfloat16 path (16-bit operands, float32 accumulation):
every kernel that serves float16 also serves bfloat16 with the bfloat16 MFMA
instructions, and is held to the same checks.

- Index mapping: integer-coded inputs (exact in bfloat16: 1..251) and one-hot
  weights through each specialised kernel, bit for bit.
- Exactness including the store's rounding: inputs in {-1, 0, 1}, so every sum
  is an exact integer in float32 and the output must be the oracle's exact
  value rounded once to nearest-even bfloat16, bit for bit.
- Values: seeded random geometries for each kernel and the split-k path
  against the oracle within 1.6e-2 * sum|w*x| (fp16's 4 units of roundoff,
  2e-3, taken at bfloat16's unit roundoff 2^-8; no page fixes a bfloat16
  tolerance), plus the final store's half ulp.
- Determinism and chunking (same bits).

The workload-sized bfloat16 layer (the bottleneck 3x3 of workload 2) is
compared in full in test_gpu_parity.py with the other full-size layers.
"""
import dataclasses

import numpy as np
import pytest

import convolution_forward_amd as cf
import oracle
import workloads
from gpu_harness import assert_parity, oracle_ref, problem_from, run_gpu

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import test_gpu_parity as P  # noqa: E402  (kernel table and sweep geometries)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cf.lib()


def _say(*a):
    print(*a, flush=True)


HALF_KERNELS = [k for k, v in P.KERNELS.items() if v[1] == "f16"]


def _run(kind, x, w, b=None, r=None, act="identity"):
    g, _, tr, variant, want = P.KERNELS[kind]
    g = dataclasses.replace(g, act=act)
    d = cf.conv_describe_variant(problem_from(g, transpose=tr, variant=variant,
                                              bias=b is not None, residual=r is not None), "bf16")
    assert want.replace("f16", "bf16") in d and ".bf16" in d, (kind, d)
    y = run_gpu(g, "bf16", x, w, b, r, transpose=tr, variant=variant)
    yr, _ = oracle_ref(g, x, w, b, r, transpose=tr)
    return y, yr


@pytest.mark.parametrize("kind", HALF_KERNELS)
def test_bf16_kernel_index_probes(kind):
    g, _, tr, _, _ = P.KERNELS[kind]
    _say(f"[bf16 probe] {kind} {g}")
    x = (np.arange(g.n * g.c_in * g.h * g.w) % 251 + 1).reshape(g.n, g.c_in, g.h, g.w)
    x = x.astype(np.float32)
    ws = P._w_shape(g, tr)
    T = (g.c_in // g.groups) * g.kh * g.kw
    for j in range(-(-T // g.c_out)):
        w = np.zeros(ws, np.float32)
        for co in range(g.c_out):
            t = (co + j * g.c_out) % T
            ci, rest = divmod(t, g.kh * g.kw)
            if tr:
                gi, jj = divmod(co, g.c_out // g.groups)
                w[gi * (g.c_in // g.groups) + ci, jj, rest // g.kw, rest % g.kw] = 1
            else:
                w[co, ci, rest // g.kw, rest % g.kw] = 1
        y, yr = _run(kind, x, w)
        assert np.array_equal(y.astype(np.float64), yr), (kind, j)


@pytest.mark.parametrize("kind", HALF_KERNELS)
def test_bf16_kernel_integer_exact_with_rounding(kind):
    g, _, tr, _, want = P.KERNELS[kind]
    rng = np.random.default_rng(sum(map(ord, kind)) + 1)
    _say(f"[bf16 exact] {kind}")
    x = rng.integers(-1, 2, (g.n, g.c_in, g.h, g.w)).astype(np.float32)
    w = rng.integers(-1, 2, P._w_shape(g, tr)).astype(np.float32)
    b = rng.integers(-1, 2, g.c_out).astype(np.float32)
    ho, wo = cf.conv_output_extent(problem_from(g, transpose=tr))
    r = None if (tr and "fused" in want) else \
        rng.integers(-1, 2, (g.n, g.c_out, ho, wo)).astype(np.float32)
    y, yr = _run(kind, x, w, b, r, act="relu")
    assert np.all(np.abs(yr) < 2 ** 24)
    assert np.array_equal(y, workloads.bf16_round(yr)), kind


def _bf16(a):
    return workloads.bf16_round(a)


def _check(g, has_b, has_r, seed, tr=False, variant="auto", splits=0):
    rng = np.random.default_rng(seed)
    cig = g.c_in // g.groups
    x = _bf16(rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)))
    ws = (g.c_in, g.c_out // g.groups, g.kh, g.kw) if tr else (g.c_out, cig, g.kh, g.kw)
    w = _bf16(rng.standard_normal(ws) * np.sqrt(2.0 / (ws[1] * g.kh * g.kw)))
    b = _bf16(rng.uniform(-0.1, 0.1, g.c_out)) if has_b else None
    shape = oracle.out_shape(g, transpose=tr)
    r = _bf16(rng.uniform(-1, 1, shape)) if has_r else None
    yr, sr = oracle_ref(g, x, w, b, r, transpose=tr)
    y = run_gpu(g, "bf16", x, w, b, r, transpose=tr, variant=variant, splits=splits)
    return assert_parity("bf16", y, yr, sr, b, r, what=f"bf16 {variant}", act=g.act), y


def _planned(g, tr=False, variant="auto", splits=0):
    try:
        return cf.conv_describe_variant(problem_from(g, transpose=tr, variant=variant,
                                                     splits=splits), "bf16")
    except cf.ConvError:
        return None


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("kind", ["rowshift", "rowband"])
def test_bf16_sweep_rowshift_rowband(kind, seed):
    g, has_b, has_r = (P._sweep_rowshift if kind == "rowshift" else P._sweep_rowband)(1000 * seed + 7)
    v = "implicit_gemm_halo" if kind == "rowshift" else "auto"
    name = _planned(g, variant=v)
    if name is None or kind not in name:
        pytest.skip(f"planned as {name}")
    _say(f"[bf16 sweep {kind} {seed}] {g} {name}")
    _check(g, has_b, has_r, seed + 99, variant=v)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("kind", ["pointwise_f16", "depthwise", "grouped", "transpose_fused"])
def test_bf16_sweep_more(kind, seed):
    g, _, has_b, has_r, tr = P._sweep_more(kind, 7919 * seed + len(kind))
    want = {"pointwise_f16": "pointwise_gemm.bf16", "depthwise": "depthwise_direct",
            "grouped": "implicit_gemm_grouped", "transpose_fused": "transpose_gemm_col2im.bf16.fused"}[kind]
    name = _planned(g, tr=tr)
    if name is None or not name.startswith(want):
        pytest.skip(f"planned as {name}")
    _say(f"[bf16 sweep {kind} {seed}] {g} {name}")
    _check(g, has_b, has_r and not tr, seed + 1234, tr=tr)


@pytest.mark.parametrize("case", range(10))
def test_bf16_generic_halo_depthwise_sweep(case):
    """The generic implicit GEMM, the halo kernel and the depthwise kernels on
    random small shapes (every activation), each variant that takes the shape."""
    g, _, has_b, has_r = P._sweep_cases()[case * 2 + 1]
    for v in ("auto", "implicit_gemm", "implicit_gemm_halo", "depthwise_direct"):
        name = _planned(g, variant=v)
        if name is None:
            continue
        _say(f"[bf16 generic {case}] {v} {name} {g}")
        _check(g, has_b, has_r, 31 + case, variant=v)


def test_bf16_split_k_and_chunks_and_rerun():
    g = oracle.Geom(3, 128, 7, 7, 96, 3, 3, pt=1, pl=1, pb=1, pr=1, act="relu")
    assert "split" in _planned(g)
    outs = {}
    for splits in (0, 1, 3, 16):
        _, y = _check(g, True, True, 5, splits=splits)
        outs[splits] = y
    _, y2 = _check(g, True, True, 5, splits=0)
    assert np.array_equal(outs[0].view(np.uint32), y2.view(np.uint32))
    # chunked through a one-image scratch: same bits
    rng = np.random.default_rng(5)
    x = _bf16(rng.uniform(-1, 1, (g.n, g.c_in, g.h, g.w)))
    w = _bf16(rng.standard_normal((g.c_out, g.c_in, 3, 3)) * 0.04)
    ya = run_gpu(g, "bf16", x, w, splits=4)
    yb = run_gpu(g, "bf16", x, w, splits=4, scratch_images=1)
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))


@pytest.mark.parametrize("case", [
    (oracle.Geom(2, 24, 5, 6, 10, 3, 3, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1, act="sigmoid"), True),
    (oracle.Geom(3, 16, 4, 8, 32, 2, 2, sh=2, sw=2), False),
    (oracle.Geom(1, 8, 6, 6, 4, 4, 4, sh=2, sw=2, pt=1, pl=1, pb=1, pr=1, oph=0, opw=0), True),
])
def test_bf16_conv_transpose(case):
    g, has_r = case
    _say(f"[bf16 convT] {g} {_planned(g, tr=True)}")
    _check(g, True, has_r, 77, tr=True)
