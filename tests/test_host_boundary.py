"""CPU tests of the C-ABI library's host half (no GPU is touched).

The library loads and exports every function include/conv.h declares; output
extents and auto_pad resolution are bit-exact against the oracle's own
independent code; every validation, overlap and scratch error path returns its
status before anything is enqueued; scratch sizes and variant names follow the
planner's shape-only rules.
"""
import itertools
import os
import re

import numpy as np
import pytest

import convolution_forward_amd as cf
import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 40  # never dereferenced: every call below fails validation first


def _header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, re.M))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert set(names) == set(cf.EXPORTS), names
    L = cf.lib()
    for n in names:
        assert hasattr(L, n), n


def test_struct_layout_matches_header():
    """Field order and sizes of the ctypes mirror equal the C struct."""
    src = open(os.path.join(ROOT, "include", "conv.h")).read()
    body = re.search(r"typedef struct conv_problem \{(.*?)\} conv_problem;", src, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        ctype, names = decl.split(None, 1)
        for nm in names.split(","):
            fields.append((nm.strip(), ctype))
    mirror = [(n, t) for n, t in cf.conv_problem._fields_]
    assert [f[0] for f in fields] == [m[0] for m in mirror]
    sizes = {"int64_t": 8, "int32_t": 4, "float": 4}
    import ctypes
    for (n, ct), (_, mt) in zip(fields, mirror):
        assert sizes[ct] == ctypes.sizeof(mt), n


def test_extents_bit_exact_vs_oracle():
    for H, k, s, d, pb, pe in itertools.product(range(1, 10), range(1, 5), range(1, 4),
                                                range(1, 3), range(0, 3), range(0, 3)):
        p = cf.make_problem(1, 1, H, 3, 1, k, 1, stride=(s, 1), dilation=(d, 1),
                            pads=(pb, 0, pe, 0))
        want = oracle.conv_extent(H, k, s, d, pb, pe)
        if want is None:
            with pytest.raises(cf.ConvError) as e:
                cf.conv_output_extent(p)
            assert e.value.status == cf.CONV_ERR_SHAPE
        else:
            assert cf.conv_output_extent(p)[0] == want
        for op in range(s):
            pt = cf.make_problem(1, 1, H, 3, 1, k, 1, stride=(s, 1), dilation=(d, 1),
                                 pads=(pb, 0, pe, 0), out_pad=(op, 0), transpose=True)
            want = oracle.convt_extent(H, k, s, d, pb, pe, op)
            if want is None:
                with pytest.raises(cf.ConvError):
                    cf.conv_output_extent(pt)
            else:
                assert cf.conv_output_extent(pt)[0] == want


def test_workload_extents_match_statements():
    for l in workloads.LAYERS:
        p = cf.make_problem(l.n, l.c_in, l.h, l.w, l.c_out, l.kh, l.kw, groups=l.groups,
                            stride=l.stride, dilation=l.dilation, pads=l.pads,
                            transpose=l.transpose)
        assert (l.n, l.c_out) + cf.conv_output_extent(p) == tuple(l.out_shape), l.name


def test_auto_pad_bit_exact_vs_oracle():
    for H, k, s, d in itertools.product(range(1, 12), range(1, 6), range(1, 4), range(1, 3)):
        for mode in ("NOTSET", "SAME_UPPER", "SAME_LOWER", "VALID"):
            p = cf.make_problem(1, 1, H, H, 1, k, k, stride=(s, s), dilation=(d, d),
                                pads=(1, 2, 2, 1))
            cf.conv_resolve_auto_pad(p, mode)
            want = oracle.auto_pad(False, mode, H, k, s, d, pads=(1, 2))
            assert (p.pad_top, p.pad_bottom) == want
            assert (p.pad_left, p.pad_right) == oracle.auto_pad(False, mode, H, k, s, d,
                                                                pads=(2, 1))
    for H, k, s, out in itertools.product(range(1, 6), range(1, 5), range(1, 4), range(1, 20)):
        for mode in ("NOTSET", "SAME_UPPER", "SAME_LOWER"):
            p = cf.make_problem(1, 1, H, H, 1, k, k, stride=(s, s), transpose=True)
            want = oracle.auto_pad(True, mode, H, k, s, 1, 0, out)
            if want is None:
                with pytest.raises(cf.ConvError):
                    cf.conv_resolve_auto_pad(p, mode, (out, out))
            else:
                cf.conv_resolve_auto_pad(p, mode, (out, out))
                assert (p.pad_top, p.pad_bottom) == want
                assert cf.conv_output_extent(p) == (out, out)
        for mode in ("SAME_UPPER", "SAME_LOWER"):
            p = cf.make_problem(1, 1, H, H, 1, k, k, stride=(s, s), transpose=True)
            want = oracle.auto_pad(True, mode, H, k, s, 1, 0, -1)
            if want is None:
                with pytest.raises(cf.ConvError):
                    cf.conv_resolve_auto_pad(p, mode)
            else:
                cf.conv_resolve_auto_pad(p, mode)
                assert (p.pad_top, p.pad_bottom) == want


def _good(**kw):
    base = dict(n=2, c_in=8, h=9, w=9, c_out=16, kh=3, kw=3)
    base.update({k: kw.pop(k) for k in list(kw) if k in base})
    return cf.make_problem(base["n"], base["c_in"], base["h"], base["w"], base["c_out"],
                           base["kh"], base["kw"], **kw)


def _fwd(p, dtype="f16", x=FAKE, w=FAKE + (1 << 30), b=None, r=None, y=FAKE + (2 << 30),
         scratch=None, sbytes=0, transpose=False):
    """Status of a forward call, from the host-only pre-flight (never enqueues).
    When the pre-flight rejects the call, the forward entry point itself is
    called too and must return the same status (it cannot launch then)."""
    p.transpose = int(bool(p.transpose))
    st = cf.conv_check(p, dtype, x, w, b, r, y, scratch, sbytes)
    if st != cf.CONV_OK:
        fn = cf.conv_transpose_forward if transpose else cf.conv_forward
        if (p.transpose == 1) == transpose:
            assert fn(p, dtype, x, w, b, r, y, scratch, sbytes, None, check=False) == st
    return st


@pytest.mark.parametrize("mut,status", [
    (dict(n=0), cf.CONV_ERR_SHAPE),
    (dict(c_in=7, groups=2), cf.CONV_ERR_SHAPE),
    (dict(c_out=15, groups=2, c_in=8), cf.CONV_ERR_SHAPE),
    (dict(stride=(0, 1)), cf.CONV_ERR_SHAPE),
    (dict(dilation=(1, 0)), cf.CONV_ERR_SHAPE),
    (dict(pads=(-1, 0, 0, 0)), cf.CONV_ERR_SHAPE),
    (dict(kh=12), cf.CONV_ERR_SHAPE),                 # no window fits
    (dict(out_pad=(1, 0)), cf.CONV_ERR_SHAPE),        # output padding on Conv
    (dict(n=1 << 20, c_in=1 << 10, h=64, w=64), cf.CONV_ERR_SHAPE),  # > 2^31-1 elements
    (dict(n=1 << 62, c_in=4), cf.CONV_ERR_SHAPE),     # int64 overflow
    (dict(act="relu", variant="transpose_gemm_col2im"), cf.CONV_ERR_ARG),
    (dict(variant="depthwise_direct"), cf.CONV_ERR_ARG),  # 8 channels per group
    (dict(variant=17), cf.CONV_ERR_ARG),
    (dict(splits=-1), cf.CONV_ERR_ARG),
    (dict(splits=99), cf.CONV_ERR_ARG),
    (dict(offsets=(-1, 0, 0, 0, 0)), cf.CONV_ERR_ARG),
])
def test_validation_errors(mut, status):
    p = _good(**mut)
    assert _fwd(p) == status
    if status == cf.CONV_ERR_SHAPE:
        with pytest.raises(cf.ConvError):
            cf.conv_scratch_size(p, "f16")


def test_bad_enums_and_pointers():
    p = _good()
    assert _fwd(p, dtype=3) == cf.CONV_ERR_ARG
    assert _fwd(p, dtype=-1) == cf.CONV_ERR_ARG
    p.activation = 9
    assert _fwd(p) == cf.CONV_ERR_ARG
    p = _good()
    p.has_bias = 2
    assert _fwd(p) == cf.CONV_ERR_ARG
    p = _good()
    assert _fwd(p, x=None) == cf.CONV_ERR_ARG
    assert _fwd(p, y=None) == cf.CONV_ERR_ARG
    p = _good(bias=True)
    assert _fwd(p) == cf.CONV_ERR_ARG  # has_bias without a bias pointer
    p = _good(residual=True)
    assert _fwd(p) == cf.CONV_ERR_ARG
    # transpose flag mismatch, both directions (the entry points reject it)
    assert cf.conv_forward(_good(transpose=True), "f16", FAKE, FAKE + (1 << 30), None, None,
                           FAKE + (2 << 30), check=False) == cf.CONV_ERR_ARG
    assert cf.conv_transpose_forward(_good(), "f16", FAKE, FAKE + (1 << 30), None, None,
                                     FAKE + (2 << 30), check=False) == cf.CONV_ERR_ARG
    assert cf.lib().conv_forward(None, 0, FAKE, FAKE, None, None, FAKE, None, 0, None) == cf.CONV_ERR_ARG


def test_overlap_rules():
    p = _good()  # x 2*8*9*9 halves, w 16*8*3*3, y 2*16*7*7 (no pads)
    assert cf.conv_check(p, "f16", FAKE, FAKE + (1 << 30), None, None, FAKE + (2 << 30)) == 0
    xs = 2 * 8 * 81 * 2
    assert _fwd(p, x=FAKE, y=FAKE + xs - 2) == cf.CONV_ERR_OVERLAP        # y over x tail
    assert _fwd(p, w=FAKE + (2 << 30) + 64) == cf.CONV_ERR_OVERLAP         # y over w
    pb = _good(bias=True)
    assert _fwd(pb, b=FAKE + (2 << 30) + 10) == cf.CONV_ERR_OVERLAP        # y over bias
    pr = _good(residual=True)
    assert _fwd(pr, r=FAKE + (2 << 30) + 2) == cf.CONV_ERR_OVERLAP         # partial y/r overlap
    # element offsets move the ranges: in one arena, x placed on y's last element
    ys = 2 * 16 * 7 * 7 * 2
    po = _good(offsets=(ys // 2 - 1, 0, 0, 0, 0))
    assert _fwd(po, x=FAKE, y=FAKE, w=FAKE + (1 << 30)) == cf.CONV_ERR_OVERLAP
    po = _good(offsets=(ys // 2, 0, 0, 0, 0))
    assert _fwd(po, x=FAKE, y=FAKE, w=FAKE + (1 << 30)) == cf.CONV_OK
    # y aliasing the residual exactly is allowed
    pr = _good(residual=True, offsets=(0, 0, 0, 3, 3))
    assert _fwd(pr, r=FAKE + (2 << 30), y=FAKE + (2 << 30)) == cf.CONV_OK


def test_scratch_rules():
    # a small-grid, long-k layer splits k, so it needs scratch
    p = cf.make_problem(2, 512, 7, 7, 512, 3, 3, pads=(1, 1, 1, 1))
    whole, per = cf.conv_scratch_size(p, "f32")
    desc = cf.conv_describe_variant(p, "f32")
    R = int(re.search(r"split(\d+)", desc).group(1))
    assert R > 1 and per == R * 512 * 49 * 4 and whole == 2 * per
    assert _fwd(p, "f32") == cf.CONV_ERR_SCRATCH                    # none given
    assert _fwd(p, "f32", scratch=FAKE + (3 << 30), sbytes=per - 4) == cf.CONV_ERR_SCRATCH
    assert _fwd(p, "f32", scratch=FAKE + (3 << 30) + 4, sbytes=per) == cf.CONV_ERR_ARG  # misaligned
    # scratch overlapping an operand
    assert _fwd(p, "f32", scratch=FAKE + 16, sbytes=whole) == cf.CONV_ERR_OVERLAP
    assert _fwd(p, "f32", scratch=FAKE + (2 << 30) - 64, sbytes=whole) == cf.CONV_ERR_OVERLAP
    # forced whole-k needs no scratch
    p1 = cf.make_problem(2, 512, 7, 7, 512, 3, 3, pads=(1, 1, 1, 1), splits=1)
    assert cf.conv_scratch_size(p1, "f32") == (0, 0)
    # ConvTranspose columns: c_out*kh*kw*h*w floats per image (float32 here; the
    # float16 kernel = stride = 2 case is fused and needs none)
    pt = cf.make_problem(8, 256, 40, 40, 64, 2, 2, stride=(2, 2), transpose=True)
    assert cf.conv_scratch_size(pt, "f32") == (8 * 64 * 4 * 1600 * 4, 64 * 4 * 1600 * 4)
    assert cf.conv_scratch_size(pt, "f16") == (0, 0)
    assert _fwd(pt, "f32", transpose=True) == cf.CONV_ERR_SCRATCH
    assert _fwd(pt, "f16", transpose=True) == cf.CONV_OK
    # depthwise and unsplit implicit need none
    for l in workloads.LAYERS:
        if l.transpose:
            continue
        q = cf.make_problem(l.n, l.c_in, l.h, l.w, l.c_out, l.kh, l.kw, groups=l.groups,
                            stride=l.stride, dilation=l.dilation, pads=l.pads)
        d = cf.conv_describe_variant(q, l.dtype)
        if "split1" in d or d.startswith(("depthwise", "pointwise", "implicit_gemm_halo")):
            assert cf.conv_scratch_size(q, l.dtype) == (0, 0), d


def test_split_cut_is_shape_only_and_deterministic():
    """The cut depends on the full-batch shape only, never on the scratch size."""
    for dt, n in (("f32", 4), ("f16", 1), ("bf16", 1)):
        p = cf.make_problem(n, 512, 7, 7, 512, 3, 3, pads=(1, 1, 1, 1))
        a = cf.conv_describe_variant(p, dt)
        assert a == cf.conv_describe_variant(p, dt)
        assert ".split" in a and not a.endswith("split1"), a
        whole, per = cf.conv_scratch_size(p, dt)
        R = int(re.search(r"split(\d+)", a).group(1))
        assert per == R * 512 * 49 * 4 and whole == n * per, (a, whole, per)


def test_rowshift_split_plans():
    """A 16-bit row-shift layer whose grid fills at most half the CUs splits k
    into equal ranges of whole 64-channel stages, the largest count that keeps
    the grid at one workgroup per CU; a forced count must divide the stages."""
    p = cf.make_problem(1, 512, 7, 7, 512, 3, 3, pads=(1, 1, 1, 1))
    assert cf.conv_describe_variant(p, "f16") == "implicit_gemm_halo.f16.rowshift.r8.n32.split8"
    assert cf.conv_describe_variant(p, "bf16") == "implicit_gemm_halo.bf16.rowshift.r8.n32.split8"
    p = cf.make_problem(3, 128, 7, 7, 96, 3, 3, pads=(1, 1, 1, 1))  # 9 tiles, 2 stages
    assert cf.conv_describe_variant(p, "f16").endswith("rowshift.r8.n32.split2")
    p = cf.make_problem(8, 512, 7, 7, 512, 3, 3, pads=(1, 1, 1, 1))  # 128 tiles
    assert cf.conv_describe_variant(p, "f16") == "implicit_gemm_halo.f16.rowshift.r8.n32.split2"
    # more than half the CUs' worth of tiles: whole k
    p = cf.make_problem(16, 512, 7, 7, 512, 3, 3, pads=(1, 1, 1, 1))
    assert cf.conv_describe_variant(p, "f16") == "implicit_gemm_halo.f16.rowshift.r8.n32"
    for s, want in ((4, "rowshift.r14.n32.split4"), (1, "rowshift.r14.n32")):
        p = cf.make_problem(1, 256, 14, 14, 64, 3, 3, pads=(1, 1, 1, 1), splits=s,
                            variant="implicit_gemm_halo")
        assert cf.conv_describe_variant(p, "f16").endswith(want)
    for s in (3, 5):  # not a divisor of the 4 stages
        p = cf.make_problem(1, 256, 14, 14, 64, 3, 3, pads=(1, 1, 1, 1), splits=s,
                            variant="implicit_gemm_halo")
        with pytest.raises(cf.ConvError):
            cf.conv_describe_variant(p, "f16")
    # a forced count the stages do not divide, variant left to the planner:
    # the generic implicit GEMM splits instead
    p = cf.make_problem(1, 256, 14, 14, 64, 3, 3, pads=(1, 1, 1, 1), splits=3)
    assert cf.conv_describe_variant(p, "f16") == "implicit_gemm.f16.t64x64.split3"


def test_variant_names_for_workloads():
    names = {}
    for l in workloads.LAYERS:
        q = cf.make_problem(l.n, l.c_in, l.h, l.w, l.c_out, l.kh, l.kw, groups=l.groups,
                            stride=l.stride, dilation=l.dilation, pads=l.pads,
                            transpose=l.transpose)
        names[l.name] = cf.conv_describe_variant(q, l.dtype)
    assert names["w4a_depthwise5x5_f32"].startswith("depthwise_direct.f32")
    assert names["w4b_depthwise3x3s2_f32"].startswith("depthwise_direct.f32")
    assert names["w5b_convtranspose2x2s2_f16"].startswith("transpose_gemm_col2im.f16.fused_k2s2")
    assert names["w3b_pointwise_f16"].startswith("pointwise_gemm.f16")
    assert names["w3a_stem7x7s2_f16"].startswith("implicit_gemm_rowband.f16")
    for n in ("w1_conv3x3_f32", "w2_bottleneck3x3_f16", "w5a_dilated_grouped_f16"):
        assert names[n].startswith("implicit_gemm"), names[n]
    buf_small = cf.conv_describe_variant  # too-small buffer path
    import ctypes
    b = ctypes.create_string_buffer(4)
    q = cf.make_problem(1, 3, 32, 32, 16, 3, 3, pads=(1, 1, 1, 1))
    assert cf.lib().conv_describe_variant(ctypes.byref(q), 0, b, 4) == cf.CONV_ERR_ARG
    assert buf_small(q, "f32")


def test_workload_plans_fixed():
    """Each workload layer's variant string, as the GPU tier asserts it on the
    device: the plan depends on the shape only."""
    from expected_plans import EXPECTED_PLANS, layer_problem
    for name, want in EXPECTED_PLANS.items():
        l = workloads.BY_NAME[name]
        assert cf.conv_describe_variant(layer_problem(cf, l), l.dtype) == want, name


def test_planner_references_no_hip_symbol(tmp_path):
    """The planner (validation, plan, describe, scratch, check, status text) is
    plain C++: it compiles without the HIP headers on the include path and its
    object references no HIP runtime symbol, so nothing it answers can depend
    on the device a call runs on (its compute-unit count included)."""
    import shutil
    import subprocess
    if shutil.which("g++") is None or shutil.which("nm") is None:
        pytest.skip("no host toolchain")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(root, "convolution_forward_amd", "csrc")
    obj = str(tmp_path / "plan.o")
    subprocess.check_call(["g++", "-std=c++17", "-c", "-I", os.path.join(root, "include"), "-I",
                           csrc, os.path.join(csrc, "conv_plan.cpp"), "-o", obj])
    undefined = subprocess.check_output(["nm", "-u", "-C", obj], text=True)
    assert "hip" not in undefined.lower(), undefined
    for name in ("conv_describe_variant", "conv_scratch_size", "conv_check",
                 "conv_output_extent", "conv_resolve_auto_pad", "conv_status_string"):
        assert name in subprocess.check_output(["nm", "-g", "--defined-only", obj], text=True)


def test_convt_fused_plan_rules():
    """Kernel = stride = 2 without padding, float16, one group, no residual takes
    the fused GEMM + gather path with no scratch; anything else keeps the float32
    column matrix."""
    base = dict(stride=(2, 2), transpose=True)
    for co in (32, 31):
        p = cf.make_problem(2, 64, 10, 12, co, 2, 2, **base)
        assert "fused_k2s2" in cf.conv_describe_variant(p, "f16")
        assert cf.conv_scratch_size(p, "f16") == (0, 0)
    unfused = [
        (cf.make_problem(2, 64, 10, 12, 32, 2, 2, **base), "f32"),
        (cf.make_problem(2, 64, 10, 12, 32, 2, 2, residual=True, **base), "f16"),
        (cf.make_problem(2, 64, 10, 12, 32, 2, 2, groups=2, **base), "f16"),
        (cf.make_problem(2, 64, 10, 10, 32, 2, 2, **base), "f16"),        # w % 4 != 0
        (cf.make_problem(2, 64, 10, 132, 32, 2, 2, **base), "f16"),       # w > 128
        (cf.make_problem(2, 64, 10, 12, 32, 3, 3, **base), "f16"),
        (cf.make_problem(2, 64, 10, 12, 32, 2, 2, pads=(1, 1, 1, 1), **base), "f16"),
    ]
    for q, dt in unfused:
        d = cf.conv_describe_variant(q, dt)
        assert d.startswith("transpose_gemm_col2im") and "fused" not in d, d
        assert cf.conv_scratch_size(q, dt)[0] > 0


def test_status_strings():
    for s in range(6):
        assert cf.status_string(s) and cf.status_string(s) != "unknown status"
    assert cf.status_string(42) == "unknown status"


def test_bf16_plans_mirror_f16():
    """bfloat16 takes every kernel float16 takes (same 16-bit data movement,
    the bfloat16 MFMA): the plan names differ only in the type."""
    for l in workloads.LAYERS + workloads.EXTRA_LAYERS:
        if l.dtype != "f16":
            continue
        q = cf.make_problem(l.n, l.c_in, l.h, l.w, l.c_out, l.kh, l.kw, groups=l.groups,
                            stride=l.stride, dilation=l.dilation, pads=l.pads,
                            transpose=l.transpose, residual=l.residual)
        a = cf.conv_describe_variant(q, "f16")
        b = cf.conv_describe_variant(q, "bf16")
        assert b == a.replace(".f16", ".bf16"), (a, b)
        assert cf.conv_scratch_size(q, "f16") == cf.conv_scratch_size(q, "bf16")
    p = cf.make_problem(1, 3, 8, 8, 4, 3, 3)
    with pytest.raises(cf.ConvError):
        cf.conv_describe_variant(p, 3)


def test_bf16_input_rounding_is_nearest_even_once():
    """The inputs' bfloat16 rounding (float64 -> 8 significant bits, ties to
    even, no double rounding through float32) against a brute-force nearest
    search over the two bfloat16 neighbours."""
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.standard_normal(20000) * 4, rng.uniform(-1, 1, 20000)])
    # exact ties and near-ties: midpoints of adjacent bfloat16 values, and the
    # float32 neighbours of a midpoint
    lo = workloads.bf16_round(rng.uniform(0.5, 2, 2000)).astype(np.float64)
    step = np.ldexp(1.0, np.frexp(lo)[1] - 8)
    mid = lo + step / 2
    a = np.concatenate([a, mid, np.nextafter(mid, 0), np.nextafter(mid, 10)])
    r = workloads.bf16_round(a).astype(np.float64)
    m, e = np.frexp(a)
    down = np.ldexp(np.floor(np.ldexp(m, 8)), e - 8)
    up = np.ldexp(np.floor(np.ldexp(m, 8)) + 1, e - 8)
    dd, du = np.abs(a - down), np.abs(up - a)
    even_down = (np.floor(np.ldexp(m, 8)) % 2) == 0
    want = np.where(dd < du, down, np.where(du < dd, up, np.where(even_down, down, up)))
    assert np.array_equal(r, want)
    bits = workloads.bf16_bits(r)
    assert np.array_equal(workloads.bf16_from_bits(bits).astype(np.float64), r)


def test_winograd_band_plans():
    """The Winograd variant's workgroup bands, from the shape alone: whole tile
    rows of one image while a tile row has at most 32 tiles (4 x 7 tiles on
    14 x 14 outputs), 32-tile segments of one row beyond that, 32 rows of
    one-tile-wide images; 64-channel blocks when the bands fill the GPU;
    refused where it does not apply (float32, 5 x 5, stride 2, input channels
    per group not a multiple of 16) or where x would pass 2 GiB."""
    def plan(n, c, h, w, co, dtype="f16", **kw):
        p = cf.make_problem(n, c, h, w, co, kw.pop("k", 3), kw.pop("k2", 3), variant="winograd", **kw)
        return cf.conv_describe_variant(p, dtype)
    assert plan(32, 256, 14, 14, 256, pads=(1, 1, 1, 1)) == "winograd_f2x2_3x3.f16.band4x7.c64"
    assert plan(1, 32, 6, 70, 40, "bf16", pads=(1, 1, 1, 1)) == "winograd_f2x2_3x3.bf16.band1x32.c32"
    assert plan(2, 16, 80, 2, 24, pads=(1, 1, 1, 1)) == "winograd_f2x2_3x3.f16.band32x1.c32"
    assert plan(2, 48, 20, 20, 32, pads=(1, 1, 1, 1)) == "winograd_f2x2_3x3.f16.band3x10.c32"
    for bad in (dict(dtype="f32", pads=(1, 1, 1, 1)), dict(k=5, k2=5, pads=(2, 2, 2, 2)),
                dict(stride=(2, 2), pads=(1, 1, 1, 1))):
        with pytest.raises(cf.ConvError):
            plan(2, 32, 14, 14, 32, **bad)
    with pytest.raises(cf.ConvError):
        plan(2, 24, 14, 14, 32, pads=(1, 1, 1, 1))
    with pytest.raises(cf.ConvError):  # 2^30 input elements
        plan(1024, 256, 64, 64, 16, pads=(1, 1, 1, 1))
