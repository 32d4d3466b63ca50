"""CPU tests of the ConvInteger ABI's host half (include/conv_integer.h): the
fields ConvInteger does not use must be zero, types and pointers are checked,
y may not overlap an operand or a zero point, and the variant name is
shape-only.  No GPU is touched (pointers are compared, never read)."""
import pytest

import convolution_forward_amd as cf

FAKE = 1 << 40


def _p(**kw):
    return cf.make_problem(2, 16, 8, 8, 32, 3, 3, pads=(1, 1, 1, 1), **kw)


def _chk(p, xt="u8", wt="i8", x=FAKE, w=FAKE + (1 << 30), xz=None, wz=None, pc=0, y=FAKE + (2 << 30)):
    return cf.conv_integer_check(p, xt, wt, x, w, xz, wz, pc, y)


def test_good_and_names():
    assert _chk(_p()) == cf.CONV_OK
    for xt in ("u8", "i8"):
        for wt in ("u8", "i8"):
            assert cf.conv_integer_describe_variant(_p(), xt, wt) == \
                f"conv_integer.{xt}{wt}.implicit_gemm.i8mfma.t64x64"
    # 3x3 stride 1, rows of at most 14 outputs, 128k channels per group: row shift
    p = cf.make_problem(32, 256, 14, 14, 256, 3, 3, pads=(1, 1, 1, 1))
    assert cf.conv_integer_describe_variant(p, "u8", "i8") == "conv_integer.u8i8.rowshift.r14.i8mfma32"
    p = cf.make_problem(2, 512, 7, 7, 64, 3, 3, pads=(1, 1, 1, 1), groups=2)
    assert cf.conv_integer_describe_variant(p, "i8", "i8") == "conv_integer.i8i8.rowshift.r8.i8mfma32"
    for kw in (dict(c_in=192), dict(h=15, w=15), dict(stride=(2, 2)), dict(dilation=(2, 2))):
        a = dict(c_in=256, h=14, w=14, stride=(1, 1), dilation=(1, 1))
        a.update(kw)
        p = cf.make_problem(2, a["c_in"], a["h"], a["w"], 64, 3, 3, pads=(1, 1, 1, 1),
                            stride=a["stride"], dilation=a["dilation"])
        assert cf.conv_integer_describe_variant(p, "u8", "u8").endswith("implicit_gemm.i8mfma.t64x64"), kw


@pytest.mark.parametrize("kw", [dict(act="relu"), dict(bias=True), dict(residual=True),
                                dict(transpose=True), dict(splits=2), dict(variant="implicit_gemm")])
def test_unused_fields_must_be_zero(kw):
    assert _chk(_p(**kw)) == cf.CONV_ERR_ARG


def test_types_pointers_overlap():
    assert _chk(_p(), xt=2) == cf.CONV_ERR_ARG
    assert _chk(_p(), wt=-1) == cf.CONV_ERR_ARG
    assert _chk(_p(), x=None) == cf.CONV_ERR_ARG
    assert _chk(_p(), y=None) == cf.CONV_ERR_ARG
    assert _chk(_p(), pc=2) == cf.CONV_ERR_ARG
    # x is 2*16*8*8 = 2048 bytes; y 2*32*8*8 int32
    assert _chk(_p(), y=FAKE + 2044) == cf.CONV_ERR_OVERLAP
    assert _chk(_p(), y=FAKE + 2048) == cf.CONV_OK
    assert _chk(_p(), xz=FAKE + (2 << 30) + 100) == cf.CONV_ERR_OVERLAP
    assert _chk(_p(), wz=FAKE + (2 << 30) - 31, pc=1) == cf.CONV_ERR_OVERLAP
    assert _chk(_p(), wz=FAKE + (2 << 30) - 32, pc=1) == cf.CONV_OK
    p = _p()
    p.groups = 3  # 16 input channels are not divisible into 3 groups
    assert _chk(p) == cf.CONV_ERR_SHAPE
