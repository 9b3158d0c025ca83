"""Pins of the CPU oracle against facts that do not come from the oracle itself.

The pages define the operation only as the exact product A x B = C over 1-, 4-
and 8-bit operands (digest of "Leveraging Large-Scale Data for Efficient Low-Bit
CUTLASS GEMM Optimization via Neural Networks", Research results item 1 and the
editor's summary).  They print no worked example, so each pin below is one of:
hand-worked fixtures (tests/golden), exhaustive tables built from Python
integers, closed forms, algebraic identities, an independent numpy formulation,
or a statistical property of the seeded inputs.  The convolution of the im2win
convolution summary (gist.science paper 2608.20725, method section) is pinned
the same way, plus two routes that do not go through its loops: a 1x1
convolution is a GEMM, and the page's own window-tensor route must agree with
the definition.  The final test plants plausible mistakes in a copy of the
oracle's C source and checks that some pin catches each one.
"""
import json
import os
import tempfile

import numpy as np
import pytest

import inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
GOLDEN_CONV = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_conv.json")


# --------------------------------------------------------------------------
# independent decoders (written differently from the oracle's C decoders)
# --------------------------------------------------------------------------

def unpack_s4_np(packed: np.ndarray) -> np.ndarray:
    """Vectorised nibble decode: sign-extend by shifting into the top of an int8."""
    p = packed.astype(np.uint8)
    lo = ((p << 4).astype(np.int8) >> 4).astype(np.int64)    # even k
    hi = (p.astype(np.int8) >> 4).astype(np.int64)           # odd k
    out = np.empty((p.shape[0], p.shape[1] * 2), np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def unpack_b1_np(words: np.ndarray) -> np.ndarray:
    by = np.ascontiguousarray(words.astype("<u4")).view(np.uint8)
    return np.unpackbits(by, axis=1, bitorder="little").astype(np.int64)


# --------------------------------------------------------------------------
# pins: each takes an oracle library handle and raises AssertionError on failure
# --------------------------------------------------------------------------

def pin_golden(h):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        kind = c["kind"]
        if kind == "s8":
            C = oracle.gemm_s8(np.array(c["A"], np.int8), np.array(c["B"], np.int8), handle=h)
            np.testing.assert_array_equal(C, np.array(c["C"], np.int32), err_msg=c["why"])
        elif kind == "s4":
            C = oracle.gemm_s4(np.array(c["A_bytes"], np.uint8), np.array(c["B_bytes"], np.uint8),
                               c["K"], handle=h)
            np.testing.assert_array_equal(C, np.array(c["C"], np.int32), err_msg=c["why"])
        elif kind == "b1":
            C = oracle.gemm_b1(np.array(c["A_words"], np.uint32), np.array(c["B_words"], np.uint32),
                               c["K"], handle=h)
            np.testing.assert_array_equal(C, np.array(c["C"], np.int32), err_msg=c["why"])
        elif kind == "linear":
            out = oracle.linear_s8(np.array(c["X"], np.int8), np.array(c["W"], np.int8),
                                   np.array(c["sx"], np.float32), np.array(c["sw"], np.float32),
                                   handle=h)
            np.testing.assert_array_equal(out, np.array(c["out"], np.float64), err_msg=c["why"])
        else:
            raise AssertionError(f"unknown fixture kind {kind}")


def pin_s8_multiplication_table(h):
    """K = 1 with every int8 value on both sides: C must be the 256 x 256 product table."""
    vals = np.arange(-128, 128, dtype=np.int64)
    A = vals.astype(np.int8).reshape(256, 1)
    C = oracle.gemm_s8(A, A.copy(), handle=h)
    table = [[int(a) * int(b) for b in vals] for a in vals]
    np.testing.assert_array_equal(C, np.array(table, np.int32))


def pin_s4_decode_table(h):
    """K = 2, all 16 nibble values at the even and at the odd position.

    Row r of A puts value v_r = r - 8 at k = 0 (low nibble) and 0 at k = 1; row
    16 + r puts it at k = 1 (high nibble).  B row s holds the value u_s = s - 8 in
    both nibbles.  So C[r, s] = v_r * u_s and C[16 + r, s] = v_r * u_s, with the
    nibble bit patterns written as literals (two's complement of v in 4 bits).
    """
    nib = {v: (v + 16) % 16 for v in range(-8, 8)}
    A = np.zeros((32, 1), np.uint8)
    for r, v in enumerate(range(-8, 8)):
        A[r, 0] = nib[v]             # low nibble (even k)
        A[16 + r, 0] = nib[v] * 16   # high nibble (odd k)
    B = np.array([[nib[u] * 17] for u in range(-8, 8)], np.uint8)
    C = oracle.gemm_s4(A, B, 2, handle=h)
    want = [[v * u for u in range(-8, 8)] for v in range(-8, 8)] * 2
    np.testing.assert_array_equal(C, np.array(want, np.int32))


def pin_b1_popcount_form(h):
    """1-bit GEMM equals the sum over words of popcount(a AND b) (Python ints)."""
    g = inputs.rng(7)
    for (M, N, K) in [(5, 7, 32), (3, 4, 96), (9, 2, 256)]:
        A = g.integers(0, 2**32, (M, K // 32), dtype=np.uint32)
        B = g.integers(0, 2**32, (N, K // 32), dtype=np.uint32)
        C = oracle.gemm_b1(A, B, K, handle=h)
        want = [[sum(bin(int(a) & int(b)).count("1") for a, b in zip(A[m], B[n]))
                 for n in range(N)] for m in range(M)]
        np.testing.assert_array_equal(C, np.array(want, np.int32))


def pin_small_random_python(h):
    """Random tiny shapes against pure-Python loops over independently decoded values."""
    g = inputs.rng(11)
    for _ in range(6):
        M, N = int(g.integers(1, 10)), int(g.integers(1, 10))
        # s8, K in 1..48
        K = int(g.integers(1, 49))
        A = g.integers(-128, 128, (M, K), dtype=np.int8)
        B = g.integers(-128, 128, (N, K), dtype=np.int8)
        want = [[sum(int(A[m, k]) * int(B[n, k]) for k in range(K)) for n in range(N)]
                for m in range(M)]
        np.testing.assert_array_equal(oracle.gemm_s8(A, B, handle=h), np.array(want, np.int32))
        # s4, K even in 2..96
        K = 2 * int(g.integers(1, 49))
        Av = g.integers(-8, 8, (M, K), dtype=np.int8)
        Bv = g.integers(-8, 8, (N, K), dtype=np.int8)
        want = [[sum(int(Av[m, k]) * int(Bv[n, k]) for k in range(K)) for n in range(N)]
                for m in range(M)]
        got = oracle.gemm_s4(inputs.pack_s4(Av), inputs.pack_s4(Bv), K, handle=h)
        np.testing.assert_array_equal(got, np.array(want, np.int32))
        # b1, K in 32..96
        K = 32 * int(g.integers(1, 4))
        Ab = g.integers(0, 2, (M, K), dtype=np.uint8)
        Bb = g.integers(0, 2, (N, K), dtype=np.uint8)
        want = [[sum(int(Ab[m, k]) * int(Bb[n, k]) for k in range(K)) for n in range(N)]
                for m in range(M)]
        got = oracle.gemm_b1(inputs.pack_b1(Ab), inputs.pack_b1(Bb), K, handle=h)
        np.testing.assert_array_equal(got, np.array(want, np.int32))


def pin_closed_forms(h):
    """Constant operands have closed-form products: C = K * a * b everywhere."""
    M, N = 3, 5
    for K in (16, 48, 1024):
        for a, b in [(1, 1), (-128, -128), (127, -128), (-1, 127)]:
            C = oracle.gemm_s8(np.full((M, K), a, np.int8), np.full((N, K), b, np.int8), handle=h)
            assert (C == K * a * b).all(), (K, a, b)
    for K in (32, 64, 4096):
        for a, b in [(-8, -8), (7, 7), (-8, 7), (1, -1)]:
            A = inputs.pack_s4(np.full((M, K), a, np.int8))
            B = inputs.pack_s4(np.full((N, K), b, np.int8))
            C = oracle.gemm_s4(A, B, K, handle=h)
            assert (C == K * a * b).all(), (K, a, b)
    for K in (32, 128, 8192):
        ones = np.full((M, K // 32), 0xFFFFFFFF, np.uint32)
        assert (oracle.gemm_b1(ones, ones[:1].repeat(N, 0), K, handle=h) == K).all()
        fives = np.full((M, K // 32), 0x55555555, np.uint32)
        aas = np.full((N, K // 32), 0xAAAAAAAA, np.uint32)
        assert (oracle.gemm_b1(fives, aas, K, handle=h) == 0).all()
        assert (oracle.gemm_b1(fives, fives[:1].repeat(N, 0), K, handle=h) == K // 2).all()


def pin_identity(h):
    """B = identity (K = N) returns A, for every bit width."""
    g = inputs.rng(13)
    K = 64
    A = g.integers(-128, 128, (7, K), dtype=np.int8)
    eye = np.eye(K, dtype=np.int8)
    np.testing.assert_array_equal(oracle.gemm_s8(A, eye, handle=h), A.astype(np.int32))
    Av = g.integers(-8, 8, (7, K), dtype=np.int8)
    got = oracle.gemm_s4(inputs.pack_s4(Av), inputs.pack_s4(eye), K, handle=h)
    np.testing.assert_array_equal(got, Av.astype(np.int32))
    Ab = g.integers(0, 2, (7, K), dtype=np.uint8)
    got = oracle.gemm_b1(inputs.pack_b1(Ab), inputs.pack_b1(eye.astype(np.uint8)), K, handle=h)
    np.testing.assert_array_equal(got, Ab.astype(np.int32))


def pin_transpose_identity(h):
    """Swapping the two operand buffers (and M, N) transposes C."""
    g = inputs.rng(17)
    M, N = 6, 11
    A = g.integers(-128, 128, (M, 80), dtype=np.int8)
    B = g.integers(-128, 128, (N, 80), dtype=np.int8)
    np.testing.assert_array_equal(oracle.gemm_s8(B, A, handle=h), oracle.gemm_s8(A, B, handle=h).T)
    A4, B4 = inputs.s4_rows(M, 96, 1), inputs.s4_rows(N, 96, 2)
    np.testing.assert_array_equal(oracle.gemm_s4(B4, A4, 96, handle=h),
                                  oracle.gemm_s4(A4, B4, 96, handle=h).T)
    A1, B1 = inputs.b1_rows(M, 128, 3), inputs.b1_rows(N, 128, 4)
    np.testing.assert_array_equal(oracle.gemm_b1(B1, A1, 128, handle=h),
                                  oracle.gemm_b1(A1, B1, 128, handle=h).T)


def pin_numpy_independent(h):
    """numpy int64 matmul over independently unpacked operands (non-square shapes)."""
    M, N = 37, 53
    A = inputs.s8_rows(M, 272, 21)
    B = inputs.s8_rows(N, 272, 22)
    want = A.astype(np.int64) @ B.astype(np.int64).T
    np.testing.assert_array_equal(oracle.gemm_s8(A, B, handle=h), want)
    K = 320
    A4, B4 = inputs.s4_rows(M, K, 23), inputs.s4_rows(N, K, 24)
    want = unpack_s4_np(A4) @ unpack_s4_np(B4).T
    np.testing.assert_array_equal(oracle.gemm_s4(A4, B4, K, handle=h), want)
    K = 384
    A1, B1 = inputs.b1_rows(M, K, 25), inputs.b1_rows(N, K, 26)
    want = unpack_b1_np(A1) @ unpack_b1_np(B1).T
    np.testing.assert_array_equal(oracle.gemm_b1(A1, B1, K, handle=h), want)


def pin_linear(h):
    """Linear layer against int64 matmul and fp64 scaling, plus exact closed forms."""
    M, N, K = 9, 14, 96
    X, W = inputs.s8_rows(M, K, 31), inputs.s8_rows(N, K, 32)
    sx, sw = inputs.scales(M, 33), inputs.scales(N, 34)
    acc = X.astype(np.int64) @ W.astype(np.int64).T
    want = acc.astype(np.float64) * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    got = oracle.linear_s8(X, W, sx, sw, handle=h)
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)
    # all -128 operands: acc = 16384 K; power-of-two scales keep the product exact
    X = np.full((2, K), -128, np.int8)
    W = np.full((3, K), -128, np.int8)
    sx = np.array([0.5, 0.25], np.float32)
    sw = np.array([2.0, 0.125, 1.0], np.float32)
    got = oracle.linear_s8(X, W, sx, sw, handle=h)
    want = np.array([[16384 * K * a * b for b in (2.0, 0.125, 1.0)] for a in (0.5, 0.25)])
    np.testing.assert_array_equal(got, want)


def pin_overflow_detected(h):
    """K = 131072 with all -128 gives 2^31, one past int32: the oracle must refuse."""
    K = 131072
    A = np.full((1, K), -128, np.int8)
    ok = oracle.gemm_s8(A[:, : K - 1].copy(), A[:, : K - 1].copy(), handle=h)
    assert ok[0, 0] == 16384 * (K - 1)
    try:
        oracle.gemm_s8(A, A.copy(), handle=h)
    except oracle.OracleOverflow:
        return
    raise AssertionError("overflow not reported")


def pin_b1_statistics(h):
    """Bernoulli(0.5) bits: an exact sum identity and the first two moments.

    Summing C over all (m, n) gives sum_k (ones in column k of A) * (ones in
    column k of B), exactly.  Each entry has mean K/4 and variance 3K/16;
    entries sharing a row or a column have covariance K/16, which sets the
    spread of the grand mean.
    """
    K, M, N = 8192, 64, 48
    A, B = inputs.b1_rows(M, K, 3001), inputs.b1_rows(N, K, 3002)
    C = oracle.gemm_b1(A, B, K, handle=h).astype(np.float64)
    colA = unpack_b1_np(A).sum(axis=0)
    colB = unpack_b1_np(B).sum(axis=0)
    assert C.sum() == float((colA * colB).sum())
    sd_mean = np.sqrt((1 / M + 1 / N) * K / 16 + 3 * K / (16 * M * N))
    assert abs(C.mean() - K / 4) < 6 * sd_mean
    assert 0.85 < C.std() / np.sqrt(3 * K / 16) < 1.15


# --------------------------------------------------------------------------
# convolution pins
# --------------------------------------------------------------------------

def conv_numpy(x, f, stride, pad):
    """Independent formulation: zero-pad, take every window with numpy strides,
    contract over (kh, kw, c) in int64.  x (N,H,W,C), f (Co,Kh,Kw,C) int64."""
    N, H, W, C = x.shape
    Co, Kh, Kw, _ = f.shape
    (sh, sw), (ph, pw) = stride, pad
    xp = np.pad(x, ((0, 0), (ph, ph), (pw, pw), (0, 0)))
    win = np.lib.stride_tricks.sliding_window_view(xp, (Kh, Kw), axis=(1, 2))  # N,Hp-Kh+1,Wp-Kw+1,C,Kh,Kw
    win = win[:, ::sh, ::sw]
    return np.einsum("nhwcij,oijc->nhwo", win.astype(np.int64), f.astype(np.int64))


def unpack_s4_last(packed):
    """(..., C/2) packed bytes -> (..., C) int64 values (even c in the low nibble)."""
    flat = packed.reshape(-1, packed.shape[-1])
    return unpack_s4_np(flat).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


def pin_conv_golden(h):
    with open(GOLDEN_CONV) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        if c["kind"] == "s8":
            y = oracle.conv2d_s8(np.array(c["x"], np.int8), np.array(c["f"], np.int8),
                                 c["stride"], c["pad"], handle=h)
        else:
            y = oracle.conv2d_s4(np.array(c["x_bytes"], np.uint8), np.array(c["f_bytes"], np.uint8),
                                 c["C"], c["stride"], c["pad"], handle=h)
        np.testing.assert_array_equal(y, np.array(c["y"], np.int32), err_msg=c["why"])


def pin_conv_1x1_is_gemm(h):
    """A 1x1 convolution with unit stride and no padding is the GEMM of the
    pixels (N*H*W rows of C) with the filters (Co rows of C)."""
    g = inputs.rng(41)
    x = g.integers(-128, 128, (2, 5, 7, 48), dtype=np.int8)
    f = g.integers(-128, 128, (9, 1, 1, 48), dtype=np.int8)
    y = oracle.conv2d_s8(x, f, handle=h)
    want = oracle.gemm_s8(x.reshape(-1, 48), f.reshape(9, 48), handle=h)
    np.testing.assert_array_equal(y.reshape(-1, 9), want)
    x4 = inputs.s4_rows(2 * 5 * 7, 64, 42).reshape(2, 5, 7, 32)
    f4 = inputs.s4_rows(6, 64, 43).reshape(6, 1, 1, 32)
    y4 = oracle.conv2d_s4(x4, f4, 64, handle=h)
    want4 = oracle.gemm_s4(x4.reshape(-1, 32), f4.reshape(6, 32), 64, handle=h)
    np.testing.assert_array_equal(y4.reshape(-1, 6), want4)


CONV_CASES = [  # (N, H, W, C, Co, Kh, Kw, stride, pad)
    (1, 6, 5, 3, 4, 3, 3, (1, 1), (1, 1)),
    (2, 7, 9, 4, 3, 3, 2, (2, 1), (0, 1)),
    (1, 9, 8, 2, 2, 5, 3, (2, 3), (2, 1)),
    (3, 4, 4, 6, 5, 1, 3, (1, 2), (0, 2)),
    (1, 3, 11, 8, 2, 3, 7, (1, 1), (1, 3)),
]


def pin_conv_numpy(h):
    """Random convolutions (strides, paddings, non-square filters) against numpy."""
    g = inputs.rng(44)
    for (N, H, W, C, Co, Kh, Kw, st, pd) in CONV_CASES:
        x = g.integers(-128, 128, (N, H, W, C), dtype=np.int8)
        f = g.integers(-128, 128, (Co, Kh, Kw, C), dtype=np.int8)
        np.testing.assert_array_equal(oracle.conv2d_s8(x, f, st, pd, handle=h), conv_numpy(x, f, st, pd))
        C4 = 2 * C
        x4 = inputs.s4_rows(N * H * W, C4, 45).reshape(N, H, W, C)
        f4 = inputs.s4_rows(Co * Kh * Kw, C4, 46).reshape(Co, Kh, Kw, C)
        want = conv_numpy(unpack_s4_last(x4), unpack_s4_last(f4), st, pd)
        np.testing.assert_array_equal(oracle.conv2d_s4(x4, f4, C4, st, pd, handle=h), want)


def pin_conv_closed_forms(h):
    """Constant image and filter: each output is a*b*C times the number of
    filter taps that land inside the image, counted per axis from the window
    origin (ho*sh - ph, wo*sw - pw)."""
    N, H, W, C, Co = 1, 7, 6, 5, 2
    for (Kh, Kw, st, pd) in [(3, 3, (1, 1), (1, 1)), (5, 2, (2, 3), (2, 1)), (4, 4, (3, 1), (3, 0))]:
        Ho, Wo = oracle.conv_out_dims(H, W, Kh, Kw, st, pd)
        rows = [min(H, ho * st[0] - pd[0] + Kh) - max(0, ho * st[0] - pd[0]) for ho in range(Ho)]
        cols = [min(W, wo * st[1] - pd[1] + Kw) - max(0, wo * st[1] - pd[1]) for wo in range(Wo)]
        taps = np.array([[r * c for c in cols] for r in rows], np.int64)
        for a, b in [(1, 1), (-128, -128), (127, -3)]:
            y = oracle.conv2d_s8(np.full((N, H, W, C), a, np.int8), np.full((Co, Kh, Kw, C), b, np.int8),
                                 st, pd, handle=h)
            assert (y == (a * b * C * taps)[None, :, :, None]).all(), (Kh, Kw, st, pd, a, b)
        C4 = 2 * C
        for a, b in [(-8, -8), (7, -8)]:
            x4 = inputs.pack_s4(np.full((N * H * W, C4), a, np.int8)).reshape(N, H, W, C)
            f4 = inputs.pack_s4(np.full((Co * Kh * Kw, C4), b, np.int8)).reshape(Co, Kh, Kw, C)
            y = oracle.conv2d_s4(x4, f4, C4, st, pd, handle=h)
            assert (y == (a * b * C4 * taps)[None, :, :, None]).all(), (Kh, Kw, st, pd, a, b)


def pin_conv_im2win_route(h):
    """The page's window-tensor route (transform, then one contiguous dot product
    per output) equals the definition, and the window tensor holds Kh/sh times
    the image rather than im2col's Kh*Kw/(sh*sw) copies."""
    g = inputs.rng(47)
    for (N, H, W, C, Co, Kh, Kw, st, pd) in CONV_CASES:
        x = g.integers(-128, 128, (N, H, W, C), dtype=np.int8)
        f = g.integers(-128, 128, (Co, Kh, Kw, C), dtype=np.int8)
        win = oracle.im2win_s8(x, Kh, Kw, st, pd, handle=h)
        Ho, _ = oracle.conv_out_dims(H, W, Kh, Kw, st, pd)
        assert win.shape == (N, Ho, W + 2 * pd[1], Kh, C)
        y = oracle.conv2d_im2win_s8(win, f, H, W, st, pd, handle=h)
        np.testing.assert_array_equal(y, oracle.conv2d_s8(x, f, st, pd, handle=h))
        np.testing.assert_array_equal(y, conv_numpy(x, f, st, pd))


PINS = [pin_golden, pin_s8_multiplication_table, pin_s4_decode_table, pin_b1_popcount_form,
        pin_small_random_python, pin_closed_forms, pin_identity, pin_transpose_identity,
        pin_numpy_independent, pin_linear, pin_overflow_detected, pin_b1_statistics,
        pin_conv_golden, pin_conv_1x1_is_gemm, pin_conv_numpy, pin_conv_closed_forms,
        pin_conv_im2win_route]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


# --------------------------------------------------------------------------
# input generators: formats and distributions (no GEMM arithmetic involved)
# --------------------------------------------------------------------------

def test_pack_s4_layout():
    v = np.array([[-8, 7, 1, -1]], np.int8)
    np.testing.assert_array_equal(inputs.pack_s4(v), np.array([[0x78, 0xF1]], np.uint8))
    with pytest.raises(ValueError):
        inputs.pack_s4(np.array([[8, 0]], np.int8))


def test_pack_b1_layout():
    bits = np.zeros((1, 64), np.uint8)
    bits[0, [0, 3, 31, 32]] = 1
    np.testing.assert_array_equal(inputs.pack_b1(bits), np.array([[0x80000009, 1]], np.uint32))


def test_generators_seeded_and_in_range():
    a = inputs.s8_rows(64, 256, 1001)
    assert a.dtype == np.int8 and a.min() == -128 and a.max() == 127
    np.testing.assert_array_equal(a, inputs.s8_rows(64, 256, 1001))
    v = inputs.s4_values(64, 256, 2001)
    assert v.min() == -8 and v.max() == 7
    w = inputs.b1_rows(4, 8192, 3001)
    assert w.dtype == np.uint32 and w.shape == (4, 256)
    s = inputs.scales(1000, 5003)
    assert s.dtype == np.float32 and s.min() >= 1e-3 and s.max() <= 1e-2


# --------------------------------------------------------------------------
# planted mistakes: each mutant of oracle.c must fail at least one pin
# --------------------------------------------------------------------------

MUTANTS = {
    "s8_drops_last_k": ("for (int64_t k = 0; k < K; ++k)\n                acc += (int64_t)s8_at(arow",
                        "for (int64_t k = 0; k < K - 1; ++k)\n                acc += (int64_t)s8_at(arow"),
    "s8_reads_unsigned": ("return (int)rowp[k];", "return (int)(uint8_t)rowp[k];"),
    "s4_no_sign_extension": ("? (int)nib - 16 : (int)nib", "? (int)nib : (int)nib"),
    "s4_wrong_byte": ("unsigned byte = rowp[k / 2];", "unsigned byte = rowp[k / 4];"),
    "s4_drops_last_k": ("for (int64_t k = 0; k < K; ++k)\n                acc += (int64_t)s4_at",
                        "for (int64_t k = 1; k < K; ++k)\n                acc += (int64_t)s4_at"),
    "b1_or_instead_of_and": ("(b1_at(arow, k) * b1_at(brow, k))", "(b1_at(arow, k) | b1_at(brow, k))"),
    "b1_wrong_bit": ("(rowp[k / 32] >> (k % 32))", "(rowp[k / 32] >> (k % 31))"),
    "c_transposed_store": ("C[m * N + n] = (int32_t)(uint32_t)(uint64_t)acc;\n        }\n    }\n    return bad;\n}\n\nint orc_gemm_s4",
                           "C[n * M + m] = (int32_t)(uint32_t)(uint64_t)acc;\n        }\n    }\n    return bad;\n}\n\nint orc_gemm_s4"),
    "b_row_stride_wrong": ("const int8_t *brow = B + n * K;\n            int64_t acc = 0;\n            for (int64_t k = 0; k < K; ++k)\n                acc += (int64_t)s8_at(arow",
                           "const int8_t *brow = B + n;\n            int64_t acc = 0;\n            for (int64_t k = 0; k < K; ++k)\n                acc += (int64_t)s8_at(arow"),
    "linear_drops_sw": ("* (double)sx[m] * (double)sw[n];", "* (double)sx[m];"),
    "linear_sx_by_column": ("* (double)sx[m] * (double)sw[n];", "* (double)sx[n % M] * (double)sw[n];"),
    "conv_pad_sign": ("x8_at(X, H, W, C, n, ho * sh + kh - ph, wo", "x8_at(X, H, W, C, n, ho * sh + kh + ph, wo"),
    "conv_width_stride_ignored": ("ho * sh + kh - ph, wo * sw + kw - pw, c) *\n                                   (int64_t)s8_at",
                                  "ho * sh + kh - ph, wo + kw - pw, c) *\n                                   (int64_t)s8_at"),
    "conv_filter_kh_kw_swapped": ("(int64_t)s8_at(F + ((co * Kh + kh) * Kw + kw) * C, c);",
                                  "(int64_t)s8_at(F + ((co * Kw + kw) * Kh + kh) * C, c);"),
    "conv_padding_reads_one": ("if (h < 0 || h >= H || w < 0 || w >= W) return 0;\n    return s8_at",
                               "if (h < 0 || h >= H || w < 0 || w >= W) return 1;\n    return s8_at"),
    "conv_s4_filter_nibbles_swapped": ("(int64_t)s4_at(F + ((co * Kh + kh) * Kw + kw) * (C / 2), c);",
                                       "(int64_t)s4_at(F + ((co * Kh + kh) * Kw + kw) * (C / 2), c ^ 1);"),
    "conv_output_nchw": ("Y[((n * Ho + ho) * Wo + wo) * Co + co] = (int32_t)(uint32_t)(uint64_t)acc;\n            }\n    }\n    return bad;\n}\n\nint orc_conv2d_s4",
                         "Y[((n * Co + co) * Ho + ho) * Wo + wo] = (int32_t)(uint32_t)(uint64_t)acc;\n            }\n    }\n    return bad;\n}\n\nint orc_conv2d_s4"),
    "im2win_window_ignores_stride": ("const int8_t *window = row + wo * sw * Kh * C;", "const int8_t *window = row + wo * Kh * C;"),
    "overflow_unchecked": ("static int fits_i32(int64_t v) { return v >= INT32_MIN && v <= INT32_MAX; }",
                           "static int fits_i32(int64_t v) { (void)v; return 1; }"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    with tempfile.TemporaryDirectory() as d:
        msrc = os.path.join(d, "mutant.c")
        with open(msrc, "w") as f:
            f.write(src.replace(old, new))
        lib_path = oracle.build(msrc, os.path.join(d, "libmutant.so"),
                                extra_flags=["-Wno-unused-function", "-Wno-unused-parameter"])
        h = oracle.load_library(lib_path)
        failures = []
        for pin in PINS:
            try:
                pin(h)
            except (AssertionError, oracle.OracleOverflow):
                failures.append(pin.__name__)
        assert failures, f"mutant {name} passed every pin"
