"""CPU tests of the C boundary: the library loads, exports every declared
symbol, and rejects bad arguments with the documented status codes before any
HIP call.  No GEMM is launched here (there is no GPU in this container)."""
import ctypes
import os
import re

import pytest

import bit_integer_gemm_amd as lb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lb_gemm.h")


@pytest.fixture(scope="module")
def lib():
    from bit_integer_gemm_amd import _build
    _build.ensure_built()
    return lb.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lb_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(lb.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_library_carries_the_source_hash(lib):
    """The loaded library was built from the sources in this tree."""
    from bit_integer_gemm_amd import _build
    assert _build.built_sha() == _build.source_sha() == lb.build_id()
    assert len(lb.build_id()) == 16


def test_header_constants_match_binding():
    text = open(HEADER).read()
    def define(name):
        return int(re.search(rf"#define {name} \(?(-?\d+)\)?", text).group(1))
    assert define("LB_AUTO") == lb.LB_AUTO
    assert define("LB_NUM_VARIANTS") == lb.LB_NUM_VARIANTS
    assert define("LB_DEFAULT_VARIANT") == lb.LB_DEFAULT_VARIANT
    assert define("LB_S8_K_ALIGN") == lb.K_ALIGN[lb.LB_S8]
    assert define("LB_S4_K_ALIGN") == lb.K_ALIGN[lb.LB_S4]
    assert define("LB_B1_K_ALIGN") == lb.K_ALIGN[lb.LB_B1]
    assert define("LB_S8_K_MAX") == lb.K_MAX[lb.LB_S8]
    assert define("LB_B1_K_MAX") == lb.K_MAX[lb.LB_B1]
    assert define("LB_CONV_S8_C_ALIGN") == lb.CONV_C_ALIGN[lb.LB_S8]
    assert define("LB_CONV_S4_C_ALIGN") == lb.CONV_C_ALIGN[lb.LB_S4]
    assert define("LB_PLAN_LINEAR") == lb.LB_PLAN_LINEAR


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation
NULL = ctypes.c_void_p(0)


@pytest.mark.parametrize("fn,align,kmax", [("lb_gemm_s8", 16, 131071), ("lb_gemm_s4", 32, 131071),
                                           ("lb_gemm_b1", 128, 134217600)])
def test_gemm_argument_checks(lib, fn, align, kmax):
    f = getattr(lib, fn)
    assert f(NULL, FAKE, FAKE, 4, 4, align, -1, NULL) == lb.LB_ERR_NULL
    assert f(FAKE, NULL, FAKE, 4, 4, align, -1, NULL) == lb.LB_ERR_NULL
    assert f(FAKE, FAKE, NULL, 4, 4, align, -1, NULL) == lb.LB_ERR_NULL
    assert f(FAKE, FAKE, FAKE, 0, 4, align, -1, NULL) == lb.LB_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 4, -1, align, -1, NULL) == lb.LB_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 4, 0, -1, NULL) == lb.LB_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 2**31, 4, align, -1, NULL) == lb.LB_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 4, 4, align + align // 2, -1, NULL) == lb.LB_ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, 4, 4, align, 9, NULL) == lb.LB_ERR_VARIANT
    assert f(FAKE, FAKE, FAKE, 4, 4, align, -2, NULL) == lb.LB_ERR_VARIANT
    over = (kmax // align + 1) * align
    assert f(FAKE, FAKE, FAKE, 4, 4, over, 0, NULL) == lb.LB_ERR_OVERFLOW


def test_linear_argument_checks(lib):
    f = lib.lb_gemm_s8_linear
    assert f(FAKE, FAKE, NULL, FAKE, FAKE, 4, 4, 16, -1, NULL) == lb.LB_ERR_NULL
    assert f(FAKE, FAKE, FAKE, NULL, FAKE, 4, 4, 16, -1, NULL) == lb.LB_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, NULL, 4, 4, 16, -1, NULL) == lb.LB_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 24, -1, NULL) == lb.LB_ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 131072, -1, NULL) == lb.LB_ERR_OVERFLOW


CONV_OK = dict(N=2, H=8, W=9, C=128, Co=16, Kh=3, Kw=3, sh=1, sw=1, ph=1, pw=1)


def conv_args(**kw):
    d = dict(CONV_OK, **kw)
    return [d[k] for k in ("N", "H", "W", "C", "Co", "Kh", "Kw", "sh", "sw", "ph", "pw")]


@pytest.mark.parametrize("fn,calign", [("lb_conv2d_s8", 16), ("lb_conv2d_s4", 32)])
def test_conv_argument_checks(lib, fn, calign):
    f = getattr(lib, fn)
    assert f(NULL, FAKE, FAKE, *conv_args(), -1, NULL) == lb.LB_ERR_NULL
    assert f(FAKE, NULL, FAKE, *conv_args(), -1, NULL) == lb.LB_ERR_NULL
    assert f(FAKE, FAKE, NULL, *conv_args(), -1, NULL) == lb.LB_ERR_NULL
    for bad in (dict(N=0), dict(H=-1), dict(C=0), dict(Co=0), dict(Kh=0), dict(sw=0), dict(sh=-2),
                dict(ph=-1), dict(Kh=11), dict(Kw=12, pw=1), dict(H=2**31)):
        assert f(FAKE, FAKE, FAKE, *conv_args(**bad), -1, NULL) == lb.LB_ERR_SHAPE, bad
    assert f(FAKE, FAKE, FAKE, *conv_args(C=calign // 2), -1, NULL) == lb.LB_ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, *conv_args(C=calign + calign // 2), -1, NULL) == lb.LB_ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, *conv_args(), 9, NULL) == lb.LB_ERR_VARIANT
    assert f(FAKE, FAKE, FAKE, *conv_args(), -2, NULL) == lb.LB_ERR_VARIANT
    # window longer than the exact-int32 K limit
    assert f(FAKE, FAKE, FAKE, *conv_args(C=calign * 8192, Kh=1, Kw=1, ph=0, pw=0), 0, NULL) == lb.LB_ERR_OVERFLOW
    # padded image of 2^31 bytes or more cannot be addressed with 32-bit offsets
    # 32 bytes per pixel: 1024 x 256 x 256 x 32 = 2^31
    big = dict(N=1024, H=256, W=256, C=32 if calign == 16 else 64, Kh=1, Kw=1, ph=0, pw=0)
    assert f(FAKE, FAKE, FAKE, *conv_args(**big), 0, NULL) == lb.LB_ERR_OVERFLOW


def test_conv_out_dims_formula():
    assert lb.conv_out_dims(56, 56, 3, 3, (1, 1), (1, 1)) == (56, 56)
    assert lb.conv_out_dims(28, 28, 3, 3, (2, 2), (1, 1)) == (14, 14)
    assert lb.conv_out_dims(7, 9, 1, 7, (3, 2), (0, 3)) == (3, 5)
    import oracle
    for args in [(56, 56, 3, 3, (1, 1), (1, 1)), (11, 13, 5, 5, (2, 2), (2, 2)), (7, 9, 1, 7, (3, 2), (0, 3))]:
        assert lb.conv_out_dims(*args) == oracle.conv_out_dims(*args)


def test_overflow_bound_is_the_int32_limit():
    # 16384 * K_MAX fits int32, one more K step does not
    assert 16384 * lb.K_MAX[lb.LB_S8] <= 2**31 - 1 < 16384 * (lb.K_MAX[lb.LB_S8] + 1)


def test_status_strings(lib):
    for s in range(7):
        assert lb.status_string(s) and lb.status_string(s) != "unknown status"
    assert lb.status_string(99) == "unknown status"


def test_variant_info(lib):
    seen = set()
    for d in (lb.LB_S8, lb.LB_S4, lb.LB_B1):
        for v in range(9):
            info = lb.lb_variant_info(d, v)
            assert info["stages"] == 2 + v % 3
            assert info["tile_m"] > 0 and info["tile_n"] > 0 and info["tile_k"] > 0
            seen.add((d, info["tile_m"] * info["tile_n"]))
        sizes = [lb.lb_variant_info(d, 3 * t)["tile_m"] * lb.lb_variant_info(d, 3 * t)["tile_n"]
                 for t in range(3)]
        assert sizes[0] < sizes[1] < sizes[2]   # small < medium < large
    # int4 tiles cover twice the K elements of int8 tiles (same bytes)
    assert lb.lb_variant_info(lb.LB_S4, 7)["tile_k"] == 2 * lb.lb_variant_info(lb.LB_S8, 7)["tile_k"]
    with pytest.raises(lb.LbError):
        lb.lb_variant_info(lb.LB_S8, 9)
    with pytest.raises(lb.LbError):
        lb.lb_variant_info(3, 0)


def test_auto_plan_argument_checks(lib):
    """lb_auto_plan rejects an unknown op and non-positive sizes before it asks
    the device anything (the launches it reports are checked on the GPU)."""
    out = [ctypes.c_int(0) for _ in range(4)]
    refs = [ctypes.byref(v) for v in out]
    assert lib.lb_auto_plan(4, 64, 64, 64, 256, *refs) == lb.LB_ERR_VARIANT
    assert lib.lb_auto_plan(-1, 64, 64, 64, 256, *refs) == lb.LB_ERR_VARIANT
    for op in (lb.LB_S8, lb.LB_S4, lb.LB_B1, lb.LB_PLAN_LINEAR):
        assert lib.lb_auto_plan(op, 0, 64, 64, 256, *refs) == lb.LB_ERR_SHAPE
        assert lib.lb_auto_plan(op, 64, -1, 64, 256, *refs) == lb.LB_ERR_SHAPE
        assert lib.lb_auto_plan(op, 64, 64, 0, 256, *refs) == lb.LB_ERR_SHAPE
    # K below one byte of a packed type
    assert lib.lb_auto_plan(lb.LB_S4, 64, 64, 1, 256, *refs) == lb.LB_ERR_SHAPE
    assert lib.lb_auto_plan(lb.LB_B1, 64, 64, 7, 256, *refs) == lb.LB_ERR_SHAPE
