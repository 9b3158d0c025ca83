"""The automatic path's launch planning, on the CPU: lb_auto_plan with an
explicit CU count runs the same host code an LB_AUTO call runs (variant
choice, two-launch split, K bands, the four-wave kernel's narrow tiles)
without a GPU.  The rules are restated here from the header's description and
checked on shapes chosen to sit on either side of each rule's boundary."""
import os

import numpy as np
import pytest

import bit_integer_gemm_amd as lb

CU = 256


@pytest.fixture(scope="module", autouse=True)
def built():
    from bit_integer_gemm_amd import _build
    _build.ensure_built()
    lb.load()


@pytest.fixture
def forced():
    old = os.environ.get("LB_AUTO_VARIANT")

    def force(v):
        if v is None:
            os.environ.pop("LB_AUTO_VARIANT", None)
        else:
            os.environ["LB_AUTO_VARIANT"] = str(v)
    yield force
    if old is None:
        os.environ.pop("LB_AUTO_VARIANT", None)
    else:
        os.environ["LB_AUTO_VARIANT"] = old


def plan(op, M, N, K, cu=CU):
    p = lb.lb_auto_plan(op, M, N, K, cu)
    return p["launches"], (p["tile_m"], p["tile_n"]), p["k_bands"]


def cdiv(a, b):
    return -(-a // b)


def narrow_tile(op, M, N, cu=CU):
    """The narrow tile a variant-6 product takes on one partial round (the
    header's rule), or None."""
    if cdiv(M, 256) * cdiv(N, 256) >= cu:
        return None
    wide, tall = cdiv(M, 256) * cdiv(N, 192), cdiv(M, 192) * cdiv(N, 256)
    only_wide = op in (lb.LB_S4, lb.LB_B1)
    if wide <= cu and (only_wide or tall > cu or wide <= tall):
        return (256, 192)
    if tall <= cu and not only_wide:
        return (192, 256)
    return None


@pytest.mark.parametrize("op,M,N,K,tile", [
    (lb.LB_S8, 512, 380, 1040, (256, 192)), (lb.LB_S8, 380, 512, 1040, (192, 256)),
    (lb.LB_PLAN_LINEAR, 300, 200, 131056, (192, 256)), (lb.LB_PLAN_LINEAR, 8192, 1376, 4096, (256, 192)),
    (lb.LB_S4, 380, 512, 1056, (256, 192)), (lb.LB_B1, 380, 512, 8320, (256, 192)),
    (lb.LB_S8, 4096, 3072, 4096, (256, 192)), (lb.LB_S8, 3072, 4096, 4096, (192, 256)),
    (lb.LB_S4, 3072, 4096, 4096, (256, 256)),          # int4 has no 192x256 tile
    (lb.LB_S8, 3584, 3584, 4096, (256, 256)),          # neither narrow grid fits in one round
    (lb.LB_S8, 4096, 4096, 4096, (256, 256)),          # a full round already
])
def test_forced_variant_6_takes_the_narrow_tile(forced, op, M, N, K, tile):
    forced(6)
    assert plan(op, M, N, K) == (1, tile, 1)
    assert narrow_tile(op, M, N) in (tile, None)


def test_narrow_rule_matches_its_statement_on_random_shapes(forced):
    forced(6)
    rng = np.random.default_rng(77)
    seen = set()
    for _ in range(300):
        M, N = (int(v) for v in rng.integers(200, 6000, 2))
        op = (lb.LB_S8, lb.LB_S4, lb.LB_B1, lb.LB_PLAN_LINEAR)[int(rng.integers(0, 4))]
        K = {lb.LB_S8: 1024, lb.LB_S4: 1024, lb.LB_B1: 4096, lb.LB_PLAN_LINEAR: 1024}[op]
        t256 = cdiv(M, 256) * cdiv(N, 256)
        if t256 > CU or 4 * t256 <= CU:     # the split and K-band rules own these
            continue
        want = narrow_tile(op, M, N) or (256, 256)
        assert plan(op, M, N, K) == (1, want, 1), (op, M, N)
        seen.add(want)
    assert seen == {(256, 256), (256, 192), (192, 256)}


def test_cu_count_moves_the_boundaries(forced):
    forced(6)
    # 192 tiles of 256x256: one partial round on 256 CUs (narrow tile), but 1.5
    # rounds on 128 CUs, which the two-launch split turns into one whole round
    # and a remainder
    assert plan(lb.LB_S8, 4096, 3072, 4096, 256) == (1, (256, 192), 1)
    assert plan(lb.LB_S8, 4096, 3072, 4096, 128)[0] == 2
    # a grid that fills 304 CUs exactly is a whole round there: no narrow tile
    assert plan(lb.LB_S8, 4096, 4864, 4096, 304) == (1, (256, 256), 1)


def test_split_and_k_bands_keep_the_256x256_tile(forced):
    forced(6)
    # 16 x 19 tiles: 1.19 rounds, the last under half full -> two launches
    launches, tile, _ = plan(lb.LB_S8, 4096, 4864, 4096)
    assert launches == 2 and tile == (256, 256)
    # one tile, long K: K bands, not a narrow tile
    launches, tile, bands = plan(lb.LB_S8, 256, 256, 8192)
    assert launches == 1 and tile == (256, 256) and bands >= 2
    # the linear layer never cuts K
    assert plan(lb.LB_PLAN_LINEAR, 256, 256, 8192)[2] == 1


@pytest.mark.parametrize("op,M,N,K,narrow", [
    (lb.LB_S4, 4096, 3072, 2048, True), (lb.LB_S4, 5120, 2304, 2048, True),
    (lb.LB_B1, 8192, 1536, 8192, True), (lb.LB_B1, 2816, 4096, 16384, True),
    (lb.LB_S4, 2048, 4096, 2048, False), (lb.LB_B1, 2304, 2400, 8192, False),
])
def test_nearly_full_narrow_round_overrides_the_selector(forced, op, M, N, K, narrow):
    forced(None)
    launches, tile, bands = plan(op, M, N, K)
    ntiles = cdiv(M, 256) * cdiv(N, 192)
    assert narrow == (8 * ntiles >= 7 * CU)
    if narrow:
        assert (launches, tile, bands) == (1, (256, 192), 1)
    else:
        info = lb.lb_variant_info(op, lb.lb_select_variant(op, M, N, K, CU)[0])
        assert tile == (info["tile_m"], info["tile_n"])


def test_forcing_a_variant_disables_the_override(forced):
    forced(4)
    assert plan(lb.LB_S4, 4096, 3072, 2048)[1] == tuple(
        lb.lb_variant_info(lb.LB_S4, 4)[k] for k in ("tile_m", "tile_n"))
