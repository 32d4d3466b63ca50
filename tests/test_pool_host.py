"""CPU tests of the pooling ABI's host half (include/pool.h; no GPU is touched).

Output extents (floor and ceil mode) and auto_pad are compared bit for bit with
the oracle's own independent code; validation, overlap and variant naming
follow the planner's shape-only rules; the ctypes mirror matches the header.
"""
import ctypes
import itertools
import os
import re

import pytest

import convolution_forward_amd as cf
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 40  # never dereferenced: pool_check does range arithmetic only


def test_struct_layout_matches_header():
    src = open(os.path.join(ROOT, "include", "pool.h")).read()
    body = re.search(r"typedef struct pool_problem \{(.*?)\} pool_problem;", src, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if decl:
            ctype, names = decl.split(None, 1)
            fields += [(nm.strip(), ctype) for nm in names.split(",")]
    mirror = cf.pool_problem._fields_
    assert [f[0] for f in fields] == [m[0] for m in mirror]
    sizes = {"int64_t": 8, "int32_t": 4}
    for (_, ct), (_, mt) in zip(fields, mirror):
        assert sizes[ct] == ctypes.sizeof(mt)


def test_extents_bit_exact_vs_oracle():
    for h, k, s, d, pb, pe, cm in itertools.product(range(1, 12), range(1, 5), range(1, 4),
                                                    range(1, 3), range(0, 3), range(0, 3),
                                                    (False, True)):
        p = cf.make_pool_problem(1, 1, h, 5, "max", kernel=(k, 1), stride=(s, 1),
                                 dilation=(d, 1), pads=(pb, 0, pe, 0), ceil_mode=cm)
        want = oracle.pool_extent(h, k, s, d, pb, pe, cm)
        if want is None:
            with pytest.raises(cf.ConvError):
                cf.pool_output_extent(p)
        else:
            assert cf.pool_output_extent(p) == (want, 5), (h, k, s, d, pb, pe, cm)


def test_global_extent_and_ignored_window():
    p = cf.make_pool_problem(2, 3, 7, 9, "global_average", kernel=(99, 99), pads=(5, 5, 5, 5))
    assert cf.pool_output_extent(p) == (1, 1)


def test_auto_pad_matches_oracle():
    for h, k, s, d in itertools.product(range(1, 10), range(1, 5), range(1, 4), range(1, 3)):
        for mode in ("SAME_UPPER", "SAME_LOWER", "VALID"):
            p = cf.make_pool_problem(1, 1, h, h, "max", kernel=(k, k), stride=(s, s),
                                     dilation=(d, d), pads=(1, 1, 1, 1))
            cf.pool_resolve_auto_pad(p, mode)
            pb, pe = oracle.auto_pad(False, mode, h, k, s, d)
            assert (p.pad_top, p.pad_bottom) == (pb, pe), (h, k, s, d, mode)


@pytest.mark.parametrize("field,value", [
    ("n", 0), ("c", -1), ("h", 0), ("kh", 0), ("stride_w", 0), ("dil_h", 0), ("pad_left", -1),
    ("h", 1 << 40), ("kw", 10 ** 6),
])
def test_validation_errors(field, value):
    p = cf.make_pool_problem(2, 3, 8, 8, "max", kernel=(3, 3), stride=(2, 2), pads=(1, 1, 1, 1))
    setattr(p, field, value)
    assert cf.pool_check(p, "f16", FAKE, FAKE + (1 << 32)) == cf.CONV_ERR_SHAPE


def test_bad_enums_pointers_and_overlap():
    good = lambda: cf.make_pool_problem(2, 3, 8, 8, "average", kernel=(2, 2), stride=(2, 2))
    assert cf.pool_check(good(), "f32", FAKE, FAKE + (1 << 32)) == cf.CONV_OK
    for dt in (3, -1):
        assert cf.pool_check(good(), dt, FAKE, FAKE + (1 << 32)) == cf.CONV_ERR_ARG
    for f, v in (("kind", 4), ("ceil_mode", 2), ("count_include_pad", -1), ("reserved", 1),
                 ("x_off", -1)):
        p = good()
        setattr(p, f, v)
        assert cf.pool_check(p, "f32", FAKE, FAKE + (1 << 32)) == cf.CONV_ERR_ARG, f
    assert cf.pool_check(good(), "f32", None, FAKE) == cf.CONV_ERR_ARG
    assert cf.pool_check(good(), "f32", FAKE, None) == cf.CONV_ERR_ARG
    # x is 2*3*8*8 floats; y 2*3*4*4 floats
    assert cf.pool_check(good(), "f32", FAKE, FAKE + 4 * 383) == cf.CONV_ERR_OVERLAP
    assert cf.pool_check(good(), "f32", FAKE, FAKE + 4 * 384) == cf.CONV_OK
    assert cf.pool_check(good(), "f32", FAKE + 4 * 95, FAKE) == cf.CONV_ERR_OVERLAP
    assert cf.pool_check(good(), "f32", FAKE + 4 * 96, FAKE) == cf.CONV_OK


def test_variant_names():
    p = cf.make_pool_problem(32, 64, 112, 112, "max", kernel=(3, 3), stride=(2, 2),
                             pads=(1, 1, 1, 1))
    assert cf.pool_describe_variant(p, "f16") == "pool.max.f16.rowvec4"
    # 3x3 stride 1 on rows of whole vectors: 8 (f16) or 4 (f32) outputs a thread
    p = cf.make_pool_problem(2, 3, 16, 16, "average", kernel=(3, 3), pads=(1, 1, 1, 1))
    assert cf.pool_describe_variant(p, "f16") == "pool.average.f16.rowvec8"
    assert cf.pool_describe_variant(p, "f32") == "pool.average.f32.rowvec4"
    # rows that are not whole 16-byte vectors, dilation, a wide left pad or a
    # large window: the band kernel
    for kw in ({"kernel": (3, 3), "stride": (2, 2), "w": 113},
               {"kernel": (3, 3), "dilation": (2, 2)},
               {"kernel": (3, 3), "pads": (2, 2, 2, 2)},
               {"kernel": (5, 5)}):
        w = kw.pop("w", 112)
        p = cf.make_pool_problem(32, 64, 112, w, "max", **kw)
        assert cf.pool_describe_variant(p, "f32").startswith("pool.max.f32.band"), kw
    # a row too wide to stage three input rows in 64 KiB: the direct kernel
    p = cf.make_pool_problem(1, 1, 4, 6000, "average", kernel=(3, 3))
    assert cf.pool_describe_variant(p, "f32") == "pool.average.f32.direct"
    p = cf.make_pool_problem(32, 2048, 7, 7, "global_average")
    assert cf.pool_describe_variant(p, "bf16") == "pool.global_average.bf16.tree.planes64"
    p = cf.make_pool_problem(64, 80, 14, 14, "global_max")
    assert cf.pool_describe_variant(p, "f32") == "pool.global_max.f32.tree.planes4"
    p = cf.make_pool_problem(2, 3, 100, 100, "global_max")
    assert cf.pool_describe_variant(p, "f32") == "pool.global_max.f32.tree.chunks3"
