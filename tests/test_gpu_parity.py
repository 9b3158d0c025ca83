"""GPU parity: every kernel variant against the CPU oracle, element by element.

All results are integers (the int32 accumulators) and must match bit-exactly;
the linear layer's fp32 output must be within 1e-6 relative of the oracle's
fp64 value.  Derivation of that bound: the kernel rounds three times in fp32
(int32 -> float, times sx, times sw), each with relative error at most 2^-24,
so the total stays below 3 * 2^-24 + O(2^-48) ~= 1.8e-7 < 1e-6.

Outputs are written into buffers with guard bands on both sides that must come
back untouched.  Small shapes cover ragged M, N (not multiples of any tile), K
shorter than one pipeline stage, K not a multiple of the stage, and single rows
and columns.  The full-size workloads run in the launch configuration the
benchmark times (automatic variant choice) and are checked element by element
against the oracle, plus a Freivalds product check.  The variant sweep's whole
shape grid (324 shapes per bit width) runs with the automatic choice: compared
with the oracle in full up to 2^30 multiply-adds, and above that on sampled
whole rows and columns plus a Freivalds check of all of C on the device.
"""
import functools
import os

import numpy as np
import pytest

import inputs
import oracle

torch = pytest.importorskip("torch")
import bit_integer_gemm_amd as lb  # noqa: E402

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINEL = 0x5A5A5A5A


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def guarded(M, N, dtype=torch.int32):
    flat = torch.full((M * N + 2 * GUARD,), SENTINEL if dtype == torch.int32 else float("nan"),
                      dtype=dtype, device="cuda")
    return flat, flat[GUARD:GUARD + M * N].view(M, N)


def check_guards(flat):
    head, tail = flat[:GUARD].cpu(), flat[-GUARD:].cpu()
    if flat.dtype == torch.int32:
        assert (head == SENTINEL).all() and (tail == SENTINEL).all(), "write outside C"
    else:
        assert torch.isnan(head).all() and torch.isnan(tail).all(), "write outside out"


def run(kind, A, B, variant, K=None):
    M, N = A.shape[0], B.shape[0]
    flat, C = guarded(M, N)
    dA, dB = to_dev(A), to_dev(B)
    if kind == "s8":
        lb.lb_gemm_s8(dA, dB, C, variant)
    elif kind == "s4":
        lb.lb_gemm_s4(dA, dB, C, variant)
    else:
        lb.lb_gemm_b1(dA.view(torch.int32), dB.view(torch.int32), C, variant)
    torch.cuda.synchronize()
    check_guards(flat)
    return C.cpu().numpy()


def make(kind, M, N, K, seed):
    if kind == "s8":
        return inputs.s8_rows(M, K, seed), inputs.s8_rows(N, K, seed + 1)
    if kind == "s4":
        return inputs.s4_rows(M, K, seed), inputs.s4_rows(N, K, seed + 1)
    return inputs.b1_rows(M, K, seed), inputs.b1_rows(N, K, seed + 1)


def ref(kind, A, B, K):
    if kind == "s8":
        return oracle.gemm_s8(A, B)
    if kind == "s4":
        return oracle.gemm_s4(A, B, K)
    return oracle.gemm_b1(A, B, K)


SMALL = {
    "s8": [(256, 256, 256), (1, 1, 16), (63, 65, 48), (257, 129, 272), (130, 300, 112),
           (64, 64, 2048), (17, 513, 1040), (300, 70, 64)],
    "s4": [(1, 1, 32), (63, 65, 96), (257, 129, 544), (130, 300, 224), (64, 64, 4096),
           (17, 513, 2080)],
    "b1": [(1, 1, 128), (63, 65, 384), (257, 129, 1152), (130, 300, 256), (64, 64, 8192),
           (17, 513, 2176)],
}


@pytest.mark.parametrize("kind", ["s8", "s4", "b1"])
@pytest.mark.parametrize("variant", list(range(9)))
def test_small_shapes_every_variant(kind, variant):
    for i, (M, N, K) in enumerate(SMALL[kind]):
        print(f"[parity] {kind} v{variant} M={M} N={N} K={K}", flush=True)
        A, B = make(kind, M, N, K, 100 + 10 * i)
        got = run(kind, A, B, variant, K)
        np.testing.assert_array_equal(got, ref(kind, A, B, K), err_msg=f"{kind} v{variant} {M}x{N}x{K}")


@pytest.mark.parametrize("variant", [lb.LB_AUTO, 0, 4, 7, 8])
def test_auto_and_variants_mid_size_s8(variant):
    M, N, K = 520, 776, 1040
    A, B = make("s8", M, N, K, 900)
    np.testing.assert_array_equal(run("s8", A, B, variant), oracle.gemm_s8(A, B))


def test_extreme_values_at_max_k():
    """Largest-magnitude operands at the largest K the boundary accepts, on the
    three int8 kernels the variants use (variant 6 is the four-wave tile whose
    MFMAs are inline assembly on tied accumulators) and the int4 kernels: all
    -128 gives 16384*K, and for int4 all -8 gives the largest sum, 64*K."""
    M, N = 33, 47
    K = 131056  # largest multiple of 16 <= 131071
    A = np.full((M, K), -128, np.int8)
    B = np.full((N, K), -128, np.int8)
    for v in (6, 7, 2, 5):
        print(f"[parity] s8 extreme v{v}", flush=True)
        got = run("s8", A, B, v)
        assert (got == 16384 * K).all()
    K4 = 131040  # largest multiple of 32 <= 131071
    A4 = inputs.pack_s4(np.full((M, K4), -8, np.int8))
    B4 = inputs.pack_s4(np.full((N, K4), 7, np.int8))
    for v in (7, 2):
        got = run("s4", A4, B4, v)
        assert (got == -56 * K4).all()
    B4m = inputs.pack_s4(np.full((N, K4), -8, np.int8))
    for v in (6, 7, 2):
        print(f"[parity] s4 extreme all -8 v{v}", flush=True)
        got = run("s4", A4, B4m, v)
        assert (got == 64 * K4).all()
    Kb = 8192
    ones = np.full((M, Kb // 32), 0xFFFFFFFF, np.uint32)
    for v in (7, 0):
        assert (run("b1", ones, ones[:1].repeat(N, 0), v) == Kb).all()
        fives = np.full((M, Kb // 32), 0x55555555, np.uint32)
        aas = np.full((N, Kb // 32), 0xAAAAAAAA, np.uint32)
        assert (run("b1", fives, aas, v) == 0).all()


@pytest.fixture
def b1_route():
    """Select the 1-bit route (LB_B1_ROUTE) for one test and restore it after."""
    old = os.environ.get("LB_B1_ROUTE")

    def use(route):
        os.environ["LB_B1_ROUTE"] = route
    yield use
    if old is None:
        os.environ.pop("LB_B1_ROUTE", None)
    else:
        os.environ["LB_B1_ROUTE"] = old


@functools.lru_cache(maxsize=2)
def b1_pass_k_case(route):
    M, N, K = 17, 9, lb.B1_PASS_K[route]
    A, B = inputs.b1_rows(M, K, 31), inputs.b1_rows(N, K, 32)
    return A, B, oracle.gemm_b1(A, B, K)


@pytest.mark.parametrize("route", ["fp4", "int8"])
@pytest.mark.parametrize("variant", list(range(9)))
def test_b1_at_longest_single_pass_k(b1_route, route, variant):
    """The longest 1-bit K one kernel pass covers, on both routes: on the FP4
    route the fp32 accumulator reaches 2^24, the last integer fp32 counts
    exactly; on the int8 route the accumulator (64 per matching bit pair) comes
    within 8192 of the int32 limit.  All ones give K exactly, and random bits
    match the oracle."""
    b1_route(route)
    A, B, want = b1_pass_k_case(route)
    M, N, K = A.shape[0], B.shape[0], lb.B1_PASS_K[route]
    print(f"[parity] b1 {route} K={K} v{variant}", flush=True)
    ones = np.full((M, K // 32), 0xFFFFFFFF, np.uint32)
    assert (run("b1", ones, ones[:N], variant) == K).all()
    np.testing.assert_array_equal(run("b1", A, B, variant), want)


@pytest.mark.parametrize("variant", [lb.LB_AUTO] + list(range(9)))
def test_b1_int8_route_small_shapes(b1_route, variant):
    """The int8 route of the 1-bit GEMM (weighted bit planes on the int8
    instruction), kept for A/B measurement, against the oracle."""
    b1_route("int8")
    for i, (M, N, K) in enumerate(SMALL["b1"] + [(256, 300, 8192)]):
        print(f"[parity] b1 int8 route v{variant} M={M} N={N} K={K}", flush=True)
        A, B = make("b1", M, N, K, 600 + 10 * i)
        np.testing.assert_array_equal(run("b1", A, B, variant, K), ref("b1", A, B, K),
                                      err_msg=f"b1 int8 route v{variant} {M}x{N}x{K}")


B1_LONG_K_CASE = (17, 9, (1 << 26) + 384)   # five K bands on the FP4 route, three on the int8 route


@functools.lru_cache(maxsize=1)
def b1_long_k_case():
    M, N, K = B1_LONG_K_CASE
    A, B = inputs.b1_rows(M, K, 33), inputs.b1_rows(N, K, 34)
    return A, B, oracle.gemm_b1(A, B, K)


@pytest.mark.parametrize("route", ["fp4", "int8"])
@pytest.mark.parametrize("variant", [lb.LB_AUTO] + list(range(9)))
def test_b1_long_k_runs_as_bands(b1_route, route, variant):
    """1-bit K beyond one pass (here 2^26 + 384 bits), for every variant and
    the automatic choice, on both routes: the bands' counts add up exactly."""
    b1_route(route)
    M, N, K = B1_LONG_K_CASE
    print(f"[parity] b1 {route} long K={K} v{variant}", flush=True)
    A, B, want = b1_long_k_case()
    np.testing.assert_array_equal(run("b1", A, B, variant), want)


@pytest.mark.parametrize("variant", [lb.LB_AUTO, 0, 6, 7])
def test_b1_at_max_k(variant):
    """The largest 1-bit K the boundary accepts (2^27 - 128 bits, eight bands):
    all ones give K, and complementary bit patterns give 0 and K/2."""
    M, N, K = 17, 9, lb.K_MAX[lb.LB_B1]
    print(f"[parity] b1 K={K} v{variant}", flush=True)
    ones = np.full((M, K // 32), 0xFFFFFFFF, np.uint32)
    assert (run("b1", ones, ones[:N], variant) == K).all()
    fives = np.full((M, K // 32), 0x55555555, np.uint32)
    assert (run("b1", fives, np.full((N, K // 32), 0xAAAAAAAA, np.uint32), variant) == 0).all()
    assert (run("b1", fives, fives[:N], variant) == K // 2).all()


@pytest.mark.parametrize("M,N,K", [(200, 300, 1024), (128, 128, 512), (1, 257, 2048), (333, 64, 8192)])
def test_probe_valu_b1_matches_oracle(M, N, K):
    """The vector-ALU popcount 1-bit GEMM of the probe module (the measured
    baseline the matrix-core routes replace) is exact against the oracle on
    ragged shapes."""
    from bit_integer_gemm_amd import probe
    if not os.path.exists(probe.LIB):
        pytest.fail(f"{probe.LIB} not built: run __graft_entry__.build()")
    A, B = inputs.b1_rows(M, K, 71), inputs.b1_rows(N, K, 72)
    C = torch.full((M, N), 7, dtype=torch.int32, device="cuda")
    probe.valu_b1(to_dev(A.view(np.int32)), to_dev(B.view(np.int32)), C)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(C.cpu().numpy(), oracle.gemm_b1(A, B, K))


def test_b1_equals_int8_gemm_of_unpacked_bits():
    """The 1-bit route against the int8 route on the GPU: unpacking the bits to
    0/1 bytes and running the int8 GEMM must give the same C, for K values that
    end inside a 16-byte piece, a 64-byte block and a pipeline stage."""
    g = inputs.rng(91)
    for (M, N, K) in [(37, 53, 128), (70, 90, 640), (300, 130, 4224), (256, 256, 8192)]:
        Ab = g.integers(0, 2, (M, K), dtype=np.uint8)
        Bb = g.integers(0, 2, (N, K), dtype=np.uint8)
        A1, B1 = inputs.pack_b1(Ab), inputs.pack_b1(Bb)
        C8 = torch.empty((M, N), dtype=torch.int32, device="cuda")
        lb.lb_gemm_s8(to_dev(Ab.astype(np.int8)), to_dev(Bb.astype(np.int8)), C8)
        torch.cuda.synchronize()
        for v in [lb.LB_AUTO] + list(range(lb.LB_NUM_VARIANTS)):
            np.testing.assert_array_equal(run("b1", A1, B1, v), C8.cpu().numpy(), err_msg=f"{M}x{N}x{K} v{v}")


def test_loaded_library_matches_sources():
    """The library the GPU tests run was built from this tree's sources."""
    from bit_integer_gemm_amd import _build
    assert lb.build_id() == _build.source_sha()


def test_transpose_identity_on_gpu():
    M, N, K = 200, 333, 528
    A, B = make("s8", M, N, K, 77)
    np.testing.assert_array_equal(run("s8", B, A, 4), run("s8", A, B, 7).T)


# ---------------------------------------------------------------------------
# full-size workloads, automatic variant (the benchmark's launch configuration)
# ---------------------------------------------------------------------------

def sampled_check(kind, A, B, K, C, rng, nrows=6, ncols=6):
    M, N = C.shape
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, nrows, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, ncols, replace=False)]))
    np.testing.assert_array_equal(C[rows], ref(kind, np.ascontiguousarray(A[rows]), B, K))
    np.testing.assert_array_equal(C[:, cols], ref(kind, A, np.ascontiguousarray(B[cols]), K))


def decode(kind, X):
    if kind == "s8":
        return X.astype(np.int64)
    if kind == "s4":
        p = X.astype(np.uint8)
        out = np.empty((p.shape[0], p.shape[1] * 2), np.int64)
        out[:, 0::2] = ((p << 4).astype(np.int8) >> 4)
        out[:, 1::2] = (p.astype(np.int8) >> 4)
        return out
    by = np.ascontiguousarray(X.astype("<u4")).view(np.uint8)
    return np.unpackbits(by, axis=1, bitorder="little").astype(np.int64)


def freivalds(kind, A, B, C, rng, reps=2):
    """C x == A (B^T x) for random integer vectors x (exact in int64)."""
    Ad, Bd = decode(kind, A), decode(kind, B)
    for _ in range(reps):
        x = rng.integers(-1000, 1000, C.shape[1]).astype(np.int64)
        np.testing.assert_array_equal(C.astype(np.int64) @ x, Ad @ (Bd.T @ x))


@pytest.mark.parametrize("kind,M,N,K,seeds", [
    ("s8", 256, 256, 256, inputs.SEEDS["s8_256"]),
    ("s4", 4096, 4096, 4096, inputs.SEEDS["s4_4096"]),
    ("b1", 4096, 4096, 8192, inputs.SEEDS["b1_4096"]),
    ("s8", 4096, 4096, 4096, (4_000_001, 4_500_001)),
])
def test_full_size_exact(kind, M, N, K, seeds):
    """The benchmark workloads at their full sizes, automatic variant: every
    element of C against the oracle, plus a Freivalds product check."""
    print(f"[parity] full {kind} {M}x{N}x{K}", flush=True)
    if kind == "s8":
        A, B = inputs.s8_rows(M, K, seeds[0]), inputs.s8_rows(N, K, seeds[1])
    elif kind == "s4":
        A, B = inputs.s4_rows(M, K, seeds[0]), inputs.s4_rows(N, K, seeds[1])
    else:
        A, B = inputs.b1_rows(M, K, seeds[0]), inputs.b1_rows(N, K, seeds[1])
    C = run(kind, A, B, lb.LB_AUTO, K)
    np.testing.assert_array_equal(C, ref(kind, A, B, K))
    freivalds(kind, A, B, C, inputs.rng(12345))


# The shape grid of the variant sweep (M, N over 64 .. 16384, four K per bit
# width: all 324 shapes per bit width), on the sweep's own operands, with the
# library's automatic choice.  Shapes up to 2^30 multiply-adds are compared
# with the oracle element by element.  Larger ones (up to 16384^2 x 8192, and
# 1-bit K up to 32768) are compared with the oracle on sampled whole rows and
# columns (the first and last of each, plus random ones), and all of C is
# checked by Freivalds' test on the device: C x == A (B^T x) for random integer
# vectors x, in fp64, where every product and partial sum is an integer below
# 2^53 and therefore exact in any summation order (|C x| and |A (B^T x)| are
# at most 128 * 64 * 16384 * 128 * 8192 < 2^48 here).
GRID_MN = [2 ** e for e in range(6, 15)]
GRID_K = {"s8": [256, 1024, 4096, 8192], "s4": [256, 1024, 4096, 8192], "b1": [1024, 4096, 8192, 32768]}
DTYPE_CODE = {"s8": 0, "s4": 1, "b1": 2}
FULL_COMPARE_MACS = 1 << 30


def decode_dev(kind, X, r0, r1):
    """Rows r0..r1 of a device operand as fp64 values (int8 bytes, signed
    nibbles with the even k in the low nibble, or bits with k in bit k % 32)."""
    x = X[r0:r1]
    if kind == "s8":
        return x.to(torch.float64)
    if kind == "s4":
        p = x.to(torch.int32)
        lo = ((p & 15) ^ 8) - 8
        hi = (((p >> 4) & 15) ^ 8) - 8
        return torch.stack((lo, hi), dim=2).reshape(x.shape[0], -1).to(torch.float64)
    shifts = torch.arange(32, device=x.device, dtype=torch.int32)
    bits = (x.unsqueeze(-1) >> shifts) & 1
    return bits.reshape(x.shape[0], -1).to(torch.float64)


def freivalds_dev(kind, dA, dB, C, seed, reps=2, chunk=2048):
    """C x == A (B^T x) on the device, exactly (see above), for `reps` random
    vectors x with entries in [-64, 64]."""
    M, N = C.shape
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for _ in range(reps):
        x = torch.randint(-64, 65, (N,), generator=g, device="cuda").to(torch.float64)
        v = None
        for r in range(0, N, chunk):
            part = decode_dev(kind, dB, r, min(N, r + chunk)).T @ x[r:r + chunk]
            v = part if v is None else v + part
        for r in range(0, M, chunk):
            lhs = C[r:r + chunk].to(torch.float64) @ x
            rhs = decode_dev(kind, dA, r, min(M, r + chunk)) @ v
            bad = (lhs != rhs).nonzero()
            assert bad.numel() == 0, f"Freivalds check fails on {bad.numel()} rows from row {r}"


def sampled_check_dev(kind, A, B, K, C, rng, nrows=3, ncols=3):
    """Whole rows and columns of a device C against the oracle (sliced on the
    device, so only the sampled outputs are copied back)."""
    M, N = C.shape
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, nrows, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, ncols, replace=False)]))
    got_r = C[torch.from_numpy(rows).cuda()].cpu().numpy()
    got_c = C[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    np.testing.assert_array_equal(got_r, ref(kind, np.ascontiguousarray(A[rows]), B, K))
    np.testing.assert_array_equal(got_c, ref(kind, A, np.ascontiguousarray(B[cols]), K))


@pytest.mark.parametrize("kidx", range(4))
@pytest.mark.parametrize("kind", ["s8", "s4", "b1"])
def test_sweep_grid_selected_variant(kind, kidx):
    shapes = [(M, N) for M in GRID_MN for N in GRID_MN]
    Mmax, Nmax = max(GRID_MN), max(GRID_MN)
    g = inputs.rng(777 + kidx)
    for K in GRID_K[kind][kidx:kidx + 1]:
        sa = 4_000_000 + 100 * DTYPE_CODE[kind] + kidx
        sb = 4_500_000 + 100 * DTYPE_CODE[kind] + kidx
        rows = {"s8": inputs.s8_rows, "s4": inputs.s4_rows, "b1": inputs.b1_rows}[kind]
        A, B = rows(Mmax, K, sa), rows(Nmax, K, sb)
        dA, dB = to_dev(A), to_dev(B)
        if kind == "b1":
            dA, dB = dA.view(torch.int32), dB.view(torch.int32)
        call = {"s8": lb.lb_gemm_s8, "s4": lb.lb_gemm_s4, "b1": lb.lb_gemm_b1}[kind]
        n_full = sum(1 for M, N in shapes if M * N * K <= FULL_COMPARE_MACS)
        print(f"[parity] grid {kind} K={K}: {len(shapes)} shapes, {n_full} compared in full, "
              f"{len(shapes) - n_full} sampled + Freivalds", flush=True)
        for M, N in shapes:
            C = torch.empty(M, N, dtype=torch.int32, device="cuda")
            call(dA[:M], dB[:N], C, lb.LB_AUTO)
            torch.cuda.synchronize()
            if M * N * K <= FULL_COMPARE_MACS:
                np.testing.assert_array_equal(C.cpu().numpy(), ref(kind, A[:M], B[:N], K),
                                              err_msg=f"{M}x{N}x{K}")
            else:
                sampled_check_dev(kind, A[:M], B[:N], K, C, g)
                freivalds_dev(kind, dA[:M], dB[:N], C, seed=M * 131 + N * 7 + K)
            del C
        del dA, dB
        torch.cuda.empty_cache()


def test_freivalds_dev_detects_a_wrong_element():
    """The device Freivalds check fails when one element of C is off by one."""
    M, N, K = 300, 260, 512
    A, B = make("s8", M, N, K, 4711)
    dA, dB = to_dev(A), to_dev(B)
    C = to_dev(oracle.gemm_s8(A, B))
    freivalds_dev("s8", dA, dB, C, seed=1)
    for kind in ("s4", "b1"):
        A2, B2 = make(kind, M, N, 1024, 4712)
        d2A, d2B = to_dev(A2), to_dev(B2)
        if kind == "b1":
            d2A, d2B = d2A.view(torch.int32), d2B.view(torch.int32)
        freivalds_dev(kind, d2A, d2B, to_dev(ref(kind, A2, B2, 1024)), seed=2)
    C[123, 45] += 1
    with pytest.raises(AssertionError):
        freivalds_dev("s8", dA, dB, C, seed=1)


# ---------------------------------------------------------------------------
# linear layer
# ---------------------------------------------------------------------------

def run_linear(X, W, sx, sw, variant):
    M, N = X.shape[0], W.shape[0]
    flat, out = guarded(M, N, torch.float32)
    lb.lb_gemm_s8_linear(to_dev(X), to_dev(W), to_dev(sx), to_dev(sw), out, variant)
    torch.cuda.synchronize()
    check_guards(flat)
    return out.cpu().numpy()


def assert_rel(got, want, rtol=1e-6):
    err = np.abs(got.astype(np.float64) - want)
    bad = err > rtol * np.abs(want)
    assert not bad.any(), f"{bad.sum()} elements beyond {rtol} relative; worst {err.max()}"


@pytest.mark.parametrize("variant", list(range(9)))
def test_linear_small_every_variant(variant):
    for i, (M, N, K) in enumerate([(64, 64, 256), (67, 130, 208), (1, 5, 16), (300, 257, 1040)]):
        X, W = inputs.s8_rows(M, K, 40 + i), inputs.s8_rows(N, K, 50 + i)
        sx, sw = inputs.scales(M, 60 + i), inputs.scales(N, 70 + i)
        assert_rel(run_linear(X, W, sx, sw, variant), oracle.linear_s8(X, W, sx, sw))


def test_linear_full_size_exact():
    """The linear layer 8192 x 11008 x 4096, automatic variant: every output
    against the oracle within the relative bound."""
    M, K, N = 8192, 4096, 11008
    s = inputs.SEEDS["linear"]
    print("[parity] linear full 8192x11008x4096", flush=True)
    X, W = inputs.s8_rows(M, K, s[0]), inputs.s8_rows(N, K, s[1])
    sx, sw = inputs.scales(M, s[2]), inputs.scales(N, s[3])
    out = run_linear(X, W, sx, sw, lb.LB_AUTO)
    assert_rel(out, oracle.linear_s8(X, W, sx, sw))


def test_linear_large_ragged_sampled():
    """A linear layer of ragged size with a K tail, 8000 x 11000 x 4000: the
    automatic path splits it into whole rounds of large tiles and a remainder,
    with partial edge tiles and a short last K stage.  Whole sampled rows and
    columns (first, last and four random of each) against the oracle."""
    M, N, K = 8000, 11000, 4000
    print("[parity] linear ragged 8000x11000x4000", flush=True)
    X, W = inputs.s8_rows(M, K, 5101), inputs.s8_rows(N, K, 5102)
    sx, sw = inputs.scales(M, 5103), inputs.scales(N, 5104)
    out = run_linear(X, W, sx, sw, lb.LB_AUTO)
    rng = inputs.rng(5105)
    rows = sorted({0, M - 1, *rng.integers(0, M, 4).tolist()})
    cols = sorted({0, N - 1, *rng.integers(0, N, 4).tolist()})
    assert_rel(out[rows], oracle.linear_s8(X[rows], W, sx[rows], sw))
    assert_rel(out[:, cols], oracle.linear_s8(X, W[cols], sx, sw[cols]))


@pytest.mark.parametrize("M,N", [(8192, 1376), (1024, 11008)])
def test_linear_shard_of_eight_exact(M, N):
    """One GPU's share of the linear layer split over eight GPUs, by columns of
    W (8192 x 1376 x 4096) or by rows of X (1024 x 11008 x 4096), with the
    automatic variant: every output against the oracle within the relative
    bound."""
    K = 4096
    s = inputs.SEEDS["linear"]
    print(f"[parity] linear shard {M}x{N}x{K}: {lb.lb_auto_plan(lb.LB_PLAN_LINEAR, M, N, K)}", flush=True)
    X, W = inputs.s8_rows(M, K, s[0]), inputs.s8_rows(N, K, s[1])
    sx, sw = inputs.scales(M, s[2]), inputs.scales(N, s[3])
    out = run_linear(X, W, sx, sw, lb.LB_AUTO)
    assert_rel(out, oracle.linear_s8(X, W, sx, sw))


def test_graph_capture_replays_match_eager():
    """The library's launches are captured into a HIP graph (the sweep times
    short kernels that way); every replay, with eager work in between, must
    reproduce the eager result exactly."""
    M, N, K = 300, 520, 1040
    A, B = make("s8", M, N, K, 4242)
    dA, dB = to_dev(A), to_dev(B)
    eager = torch.empty(M, N, dtype=torch.int32, device="cuda")
    lb.lb_gemm_s8(dA, dB, eager, 6)
    torch.cuda.synchronize()
    want = oracle.gemm_s8(A, B)
    np.testing.assert_array_equal(eager.cpu().numpy(), want)
    C = torch.zeros(M, N, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lb.lb_gemm_s8(dA, dB, C, 6)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lb.lb_gemm_s8(dA, dB, C, 6)
        lb.lb_gemm_s8(dA, dB, C, 0)
    for r in range(3):
        C.fill_(-1)
        other = torch.empty(M, M, dtype=torch.int32, device="cuda")
        lb.lb_gemm_s8(dA, dA, other, 3)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(C.cpu().numpy(), want, err_msg=f"replay {r}")


# ---------------------------------------------------------------------------
# automatic choice run as two launches (a band of whole rounds of large tiles,
# then the remaining columns)
# ---------------------------------------------------------------------------

def splits(dtype_code, M, N, K, v=None):
    """Whether the library's automatic choice runs (M, N, K) as two launches:
    a large-tile variant (v, when LB_AUTO_VARIANT forces it) whose last round of
    tiles fills at most half the CUs."""
    if v is None:
        v = lb.lb_select_variant(dtype_code, M, N, K, 0)[0]
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    T = -(-M // 256) * -(-N // 256)
    return v >= 6 and T > cu and T % cu != 0 and 2 * (T % cu) <= cu


# Column bands (19 tile columns over 16 tile rows), and row bands (19 tile rows
# over 16 tile columns, where no column band fills whole rounds); ragged edges.
# The selector avoids a large tile whose last round is nearly empty, so the
# large tiles (the 2-stage one, variant 6, and the default, 7) are forced.
@pytest.mark.parametrize("kind,M,N,K,v", [
    ("s8", 4096, 4864, 4096, 6), ("s8", 4000, 4810, 4096, 7),
    ("s4", 4096, 4864, 4096, 6), ("s4", 4000, 4810, 4096, 7),
    ("b1", 4000, 4810, 4096, 6),
    ("s8", 4864, 4096, 4096, 6), ("s8", 4810, 4000, 4096, 7),
    ("s4", 4810, 4000, 4096, 6), ("b1", 4810, 4000, 4096, 7),
])
def test_auto_split_launches_match_oracle(forced_auto_variant, kind, M, N, K, v):
    print(f"[parity] split {kind} {M}x{N}x{K} v{v}", flush=True)
    forced_auto_variant(v)
    code = {"s8": lb.LB_S8, "s4": lb.LB_S4, "b1": lb.LB_B1}[kind]
    assert splits(code, M, N, K, v), "shape no longer exercises the two-launch path"
    A, B = make(kind, M, N, K, 2024)
    got = run(kind, A, B, lb.LB_AUTO, K)
    np.testing.assert_array_equal(got, ref(kind, A, B, K))


@pytest.mark.parametrize("M,N", [(4000, 4810), (4810, 4000)])
def test_auto_split_linear_matches_oracle(forced_auto_variant, M, N):
    K = 4096
    forced_auto_variant(6)
    assert splits(lb.LB_S8, M, N, K, 6)
    X, W = inputs.s8_rows(M, K, 71), inputs.s8_rows(N, K, 72)
    sx, sw = inputs.scales(M, 73), inputs.scales(N, 74)
    assert_rel(run_linear(X, W, sx, sw, lb.LB_AUTO), oracle.linear_s8(X, W, sx, sw))


# ---------------------------------------------------------------------------
# automatic choice with K cut into bands (few tiles, long K): each band adds its
# exact partial sums into C
# ---------------------------------------------------------------------------

KB_PER = {"s8": 1, "s4": 2, "b1": 8}   # elements per byte
ALPHA = {"s8": 2.5, "s4": 2.3, "b1": 0.83}   # 1-bit: the FP4 route (the default)


def k_bands(kind, M, N, K, v=None):
    """Number of K bands the library's automatic choice uses for (M, N, K)
    (with variant v when LB_AUTO_VARIANT forces it): the cost model of the
    header's split-K rule, restated."""
    code = {"s8": lb.LB_S8, "s4": lb.LB_S4, "b1": lb.LB_B1}[kind]
    if v is None:
        v = lb.lb_select_variant(code, M, N, K, 0)[0]
    info = lb.lb_variant_info(code, v)
    tm, tn = info["tile_m"], info["tile_n"]
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = -(-M // tm) * -(-N // tn)
    kb = K // KB_PER[kind]
    if 4 * tiles > cu:
        return 1
    t0 = ALPHA[kind] * K
    smax = min(cu // tiles, 16, kb // 128)
    best, best_t = 1, t0
    for S in range(2, smax + 1):
        t = t0 / S + 3000.0 + 0.015 * M * N * S
        if t < best_t:
            best, best_t = S, t
    if best < 2 or best_t * 1.3 > t0:
        return 1
    length = -(-(-(-kb // best)) // 128) * 128
    return -(-kb // length)


@pytest.mark.parametrize("kind,M,N,K", [
    ("s8", 64, 64, 8192), ("s8", 100, 70, 4112), ("s8", 256, 512, 16384), ("s8", 1, 1, 2048),
    ("s4", 64, 64, 8192), ("s4", 100, 70, 4128),
    ("b1", 64, 64, 32768), ("b1", 100, 70, 16512),
])
def test_auto_k_bands_match_oracle(kind, M, N, K):
    bands = k_bands(kind, M, N, K)
    print(f"[parity] k bands {kind} {M}x{N}x{K}: {bands}", flush=True)
    assert bands >= 2, "shape no longer exercises the K-band path"
    A, B = make(kind, M, N, K, 3030)
    np.testing.assert_array_equal(run(kind, A, B, lb.LB_AUTO, K), ref(kind, A, B, K))


def test_auto_k_bands_extreme_values():
    """Largest-magnitude operands at the largest K, K cut into bands: every
    band's partial sum and every running total of C stays exact."""
    M, N = 33, 47
    K = 131056
    assert k_bands("s8", M, N, K) >= 2
    A = np.full((M, K), -128, np.int8)
    got = run("s8", A, np.full((N, K), -128, np.int8), lb.LB_AUTO)
    assert (got == 16384 * K).all()
    got = run("s8", A, np.full((N, K), 127, np.int8), lb.LB_AUTO)
    assert (got == -16256 * K).all()
    K4 = 131040
    A4 = inputs.pack_s4(np.full((M, K4), -8, np.int8))
    got = run("s4", A4, inputs.pack_s4(np.full((N, K4), 7, np.int8)), lb.LB_AUTO)
    assert (got == -56 * K4).all()


@pytest.fixture
def forced_auto_variant():
    """Set LB_AUTO_VARIANT for one test and restore the environment after it."""
    old = os.environ.get("LB_AUTO_VARIANT")

    def force(v):
        os.environ["LB_AUTO_VARIANT"] = str(v)
    yield force
    if old is None:
        os.environ.pop("LB_AUTO_VARIANT", None)
    else:
        os.environ["LB_AUTO_VARIANT"] = old


# The selection table sends no few-tile product to the large tiles, so the K
# bands of the four-wave int8 tile (variant 6) and of the other large tiles are
# reached by forcing the automatic path's variant.  Ragged M and N, and a band
# length that leaves a short last band, are among the cases.
@pytest.mark.parametrize("kind,v,M,N,K", [
    ("s8", 6, 256, 256, 8192), ("s8", 6, 200, 330, 16384), ("s8", 6, 64, 512, 12288),
    ("s8", 7, 256, 256, 8192), ("s8", 8, 200, 330, 16384),
    ("s4", 6, 256, 256, 16384), ("b1", 6, 256, 256, 65536),
])
def test_forced_large_tile_k_bands_match_oracle(forced_auto_variant, kind, v, M, N, K):
    forced_auto_variant(v)
    bands = k_bands(kind, M, N, K, v)
    print(f"[parity] forced variant {v} k bands {kind} {M}x{N}x{K}: {bands} bands", flush=True)
    assert bands >= 2, "shape no longer exercises the K bands"
    A, B = make(kind, M, N, K, 3100 + v)
    np.testing.assert_array_equal(run(kind, A, B, lb.LB_AUTO, K), ref(kind, A, B, K))


def test_forced_variant_reaches_the_linear_layer(forced_auto_variant):
    """LB_AUTO_VARIANT also fixes the variant of the linear layer's automatic
    path (here the four-wave kernel, on its 256x192 tile, on ragged M and N)."""
    forced_auto_variant(6)
    M, N, K = 300, 520, 1024
    X, W = inputs.s8_rows(M, K, 81), inputs.s8_rows(N, K, 82)
    sx, sw = inputs.scales(M, 83), inputs.scales(N, 84)
    assert_rel(run_linear(X, W, sx, sw, lb.LB_AUTO), oracle.linear_s8(X, W, sx, sw))


# The four-wave kernel's narrower tiles (256x192 and 192x256): an automatic
# choice of variant 6 takes them for the int8 GEMM and the linear layer when
# the 256x256 grid would fill less than one round of the CUs and the narrower
# grid still fits in one.  Ragged edges in both dimensions, K of one alignment
# unit, a K tail, several stages.
NARROW = [(512, 380, (256, 192)), (380, 512, (192, 256)), (500, 370, (256, 192)), (370, 500, (192, 256))]


def assert_plan(op, M, N, K, launches, tile, bands):
    plan = lb.lb_auto_plan(op, M, N, K)
    assert (plan["launches"], (plan["tile_m"], plan["tile_n"]), plan["k_bands"]) == (launches, tile, bands), plan


@pytest.mark.parametrize("M,N,tile", NARROW)
def test_narrow_four_wave_tiles_match_oracle(forced_auto_variant, M, N, tile):
    forced_auto_variant(6)
    for K in (16, 64, 1040, 4096):
        assert_plan(lb.LB_S8, M, N, K, 1, tile, 1)
        assert_plan(lb.LB_PLAN_LINEAR, M, N, K, 1, tile, 1)
        print(f"[parity] narrow tile {tile} {M}x{N}x{K}", flush=True)
        A, B = make("s8", M, N, K, 6100 + K)
        np.testing.assert_array_equal(run("s8", A, B, lb.LB_AUTO, K), ref("s8", A, B, K))
        sx, sw = inputs.scales(M, 6200 + K), inputs.scales(N, 6300 + K)
        assert_rel(run_linear(A, B, sx, sw, lb.LB_AUTO), oracle.linear_s8(A, B, sx, sw))


@pytest.mark.parametrize("M,N", [(512, 380), (380, 512), (500, 370), (370, 500)])
def test_narrow_four_wave_tile_int4_matches_oracle(forced_auto_variant, M, N):
    """int4 takes the 256x192 narrow tile in either orientation (its unpack
    schedule exists for six fragment columns, not six rows)."""
    forced_auto_variant(6)
    for K in (32, 64, 1056, 4096):
        assert_plan(lb.LB_S4, M, N, K, 1, (256, 192), 1)
        print(f"[parity] narrow tile int4 {M}x{N}x{K}", flush=True)
        A, B = make("s4", M, N, K, 6600 + K)
        np.testing.assert_array_equal(run("s4", A, B, lb.LB_AUTO, K), ref("s4", A, B, K))


def _narrow_random_cases(n=16, seed=6700):
    """Seeded partial-round shapes: M, N in 600..4000 (ragged), K a random
    multiple of 32 up to 3200 (1-bit: of 128 up to 12800); each case names its
    op and the narrow tile it must take on a 256-CU GPU."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        M, N = (int(v) for v in rng.integers(600, 4001, 2))
        K = 32 * int(rng.integers(1, 101))
        t256 = -(-M // 256) * -(-N // 256)
        wide, tall = -(-M // 256) * -(-N // 192), -(-M // 192) * -(-N // 256)
        if t256 >= 256 or 4 * t256 <= 256:      # a partial round, not few enough tiles for K bands
            continue
        op = ("s8", "s4", "linear", "b1")[len(cases) % 4]
        if op == "b1":
            K *= 4
        if wide <= 256 and (op in ("s4", "b1") or tall > 256 or wide <= tall):
            tile = (256, 192)
        elif tall <= 256 and op in ("s8", "linear"):
            tile = (192, 256)
        else:
            continue
        cases.append((op, M, N, K, tile))
    return cases


@pytest.mark.parametrize("op,M,N,K,tile", _narrow_random_cases())
def test_narrow_four_wave_tiles_random_shapes(forced_auto_variant, op, M, N, K, tile):
    forced_auto_variant(6)
    code = {"s8": lb.LB_S8, "s4": lb.LB_S4, "b1": lb.LB_B1, "linear": lb.LB_PLAN_LINEAR}[op]
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert_plan(code, M, N, K, 1, tile, 1)
    print(f"[parity] narrow random {op} {M}x{N}x{K} {tile}", flush=True)
    if op == "linear":
        X, W = inputs.s8_rows(M, K, 6800 + K), inputs.s8_rows(N, K, 6801 + K)
        sx, sw = inputs.scales(M, 6802), inputs.scales(N, 6803)
        assert_rel(run_linear(X, W, sx, sw, lb.LB_AUTO), oracle.linear_s8(X, W, sx, sw))
    else:
        A, B = make(op, M, N, K, 6900 + K)
        np.testing.assert_array_equal(run(op, A, B, lb.LB_AUTO, K), ref(op, A, B, K))


@pytest.mark.parametrize("M,N", [(512, 380), (380, 512), (500, 370)])
def test_narrow_four_wave_tile_b1_matches_oracle(forced_auto_variant, M, N):
    """The 1-bit GEMM (FP4 route) takes the 256x192 narrow tile in either
    orientation (its plane schedule exists for six fragment columns)."""
    forced_auto_variant(6)
    for K in (128, 1024, 8320, 16384):
        assert_plan(lb.LB_B1, M, N, K, 1, (256, 192), 1)
        print(f"[parity] narrow tile 1-bit {M}x{N}x{K}", flush=True)
        A, B = make("b1", M, N, K, 6650 + K)
        np.testing.assert_array_equal(run("b1", A, B, lb.LB_AUTO, K), ref("b1", A, B, K))


def test_narrow_four_wave_tile_b1_extreme_values(forced_auto_variant):
    """All ones at 2^20 bits through the 1-bit narrow tile give K; 0x55.. against
    0xAA.. gives 0."""
    forced_auto_variant(6)
    M, N, K = 2304, 2400, 1 << 20
    assert_plan(lb.LB_B1, M, N, K, 1, (256, 192), 1)
    print(f"[parity] narrow tile 1-bit extreme {M}x{N}x{K}", flush=True)
    ones = np.full((M, K // 32), 0xFFFFFFFF, np.uint32)
    assert (run("b1", ones, ones[:N], lb.LB_AUTO) == K).all()
    fives = np.full((M, K // 32), 0x55555555, np.uint32)
    aas = np.full((N, K // 32), 0xAAAAAAAA, np.uint32)
    assert (run("b1", fives, aas, lb.LB_AUTO) == 0).all()


@pytest.mark.parametrize("kind,M,N,K,narrow", [
    ("s4", 4096, 3072, 2048, True), ("s4", 5120, 2304, 2048, True), ("b1", 8192, 1536, 8192, True),
    ("b1", 2816, 4096, 16384, True), ("s4", 2048, 4096, 2048, False), ("b1", 2304, 2400, 8192, False),
])
def test_automatic_choice_takes_a_nearly_full_narrow_round(kind, M, N, K, narrow):
    """Without LB_AUTO_VARIANT: where a round of 256x192 tiles fills at least
    7/8 of the CUs the automatic path runs it (variant 6), whatever the
    selector chose; with fewer narrow tiles it keeps the selector's tile.  The
    result matches the oracle either way."""
    assert "LB_AUTO_VARIANT" not in os.environ
    code = {"s4": lb.LB_S4, "b1": lb.LB_B1}[kind]
    plan = lb.lb_auto_plan(code, M, N, K)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        if narrow:
            assert (plan["tile_m"], plan["tile_n"], plan["launches"]) == (256, 192, 1), plan
        else:
            info = lb.lb_variant_info(code, lb.lb_select_variant(code, M, N, K, 0)[0])
            assert (plan["tile_m"], plan["tile_n"]) == (info["tile_m"], info["tile_n"]), plan
    print(f"[parity] automatic narrow round {kind} {M}x{N}x{K}: {plan}", flush=True)
    A, B = make(kind, M, N, K, 7100)
    np.testing.assert_array_equal(run(kind, A, B, lb.LB_AUTO, K), ref(kind, A, B, K))


def test_narrow_four_wave_tiles_extreme_values(forced_auto_variant):
    """All -128 at the largest K through both narrow tiles: every sum is
    16384 K, 2^31 - 262144 (int8 GEMM), and the linear layer's outputs are that
    count times sx[m] sw[n]."""
    forced_auto_variant(6)
    K = 131056
    for M, N, tile in ((2304, 2400, (256, 192)), (2400, 2304, (192, 256))):
        assert_plan(lb.LB_S8, M, N, K, 1, tile, 1)
        print(f"[parity] narrow tile {tile} extreme {M}x{N}x{K}", flush=True)
        got = run("s8", np.full((M, K), -128, np.int8), np.full((N, K), -128, np.int8), lb.LB_AUTO)
        assert (got == 16384 * K).all()
    M, N, K4 = 2304, 2400, 131040
    assert_plan(lb.LB_S4, M, N, K4, 1, (256, 192), 1)
    print(f"[parity] narrow tile int4 extreme {M}x{N}x{K4}", flush=True)
    A4 = inputs.pack_s4(np.full((M, K4), -8, np.int8))
    got = run("s4", A4, inputs.pack_s4(np.full((N, K4), -8, np.int8)), lb.LB_AUTO)
    assert (got == 64 * K4).all()
    M, N = 300, 200
    assert_plan(lb.LB_PLAN_LINEAR, M, N, K, 1, (192, 256), 1)
    X = np.full((M, K), -128, np.int8)
    sx, sw = inputs.scales(M, 6401), inputs.scales(N, 6402)
    want = 16384.0 * K * np.outer(sx.astype(np.float64), sw.astype(np.float64))
    assert_rel(run_linear(X, np.full((N, K), -128, np.int8), sx, sw, lb.LB_AUTO), want)


@pytest.mark.parametrize("kind,M,N,tile", [("s8", 4096, 3072, (256, 192)), ("s8", 3072, 4096, (192, 256)),
                                            ("s4", 4096, 3072, (256, 192)), ("b1", 4096, 3072, (256, 192))])
def test_narrow_four_wave_tiles_full_size(forced_auto_variant, kind, M, N, tile):
    """One round of narrow tiles filling all 256 CUs (16 x 16 tiles), every
    element against the oracle."""
    forced_auto_variant(6)
    K = 8192 if kind == "b1" else 4096
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert_plan({"s8": lb.LB_S8, "s4": lb.LB_S4, "b1": lb.LB_B1}[kind], M, N, K, 1, tile, 1)
    print(f"[parity] narrow tile {kind} {tile} {M}x{N}x{K}", flush=True)
    A, B = make(kind, M, N, K, 6500)
    np.testing.assert_array_equal(run(kind, A, B, lb.LB_AUTO, K), ref(kind, A, B, K))


@pytest.mark.parametrize("kind,M,N,K", [("s8", 64, 64, 8192), ("s8", 4000, 4810, 4096), ("s8", 500, 370, 1040)])
def test_graph_capture_of_automatic_launches(forced_auto_variant, kind, M, N, K):
    """The automatic path's extra launches (the zeroing of C before K bands, or
    the second launch of a two-launch split) and its narrow four-wave tile,
    captured into a HIP graph: every replay, with eager work and a clobbered C
    in between, reproduces the oracle."""
    if (M, N) == (64, 64):
        assert k_bands(kind, M, N, K) >= 2
    elif (M, N) == (500, 370):
        forced_auto_variant(6)
        assert_plan(lb.LB_S8, M, N, K, 1, (256, 192), 1)
    else:
        forced_auto_variant(6)
        assert splits(lb.LB_S8, M, N, K, 6)
    A, B = make(kind, M, N, K, 5151)
    dA, dB = to_dev(A), to_dev(B)
    want = oracle.gemm_s8(A, B)
    C = torch.zeros(M, N, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lb.lb_gemm_s8(dA, dB, C, lb.LB_AUTO)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lb.lb_gemm_s8(dA, dB, C, lb.LB_AUTO)
    x = to_dev(inputs.s8_rows(256, 1024, 5152))
    other = torch.empty(256, 256, dtype=torch.int32, device="cuda")
    for r in range(3):
        C.fill_(12345)
        lb.lb_gemm_s8(x, x, other, lb.LB_AUTO)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(C.cpu().numpy(), want, err_msg=f"replay {r}")

