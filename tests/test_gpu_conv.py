"""GPU parity of the low-bit convolution against the CPU oracle.

The operation is the convolution of the im2win convolution summary
(gist.science paper 2608.20725, problem statement and method: NHWC images, the
whole batch at once) under the reading written in the oracle: zero padding,
strides, filters (Co, Kh, Kw, C), output NHWC int32.  Every result is an
integer sum and must match the oracle bit-exactly.

The small cases run every kernel variant and cover ragged output-pixel counts
and channel counts (not multiples of any tile), pixels of 16-48 and 80-112
bytes (a 64-byte K block then spans several filter taps), non-square filters, unequal
strides and paddings, padding as wide as the filter (outputs that see only
padding), a 1x1 filter with stride larger than one and a single-pixel image.
The layer-sized cases run in the configuration the benchmark times (automatic
variant choice) and are compared in full.  Outputs land in buffers with guard
bands that must come back untouched.
"""
import numpy as np
import pytest

import inputs
import oracle

torch = pytest.importorskip("torch")
import bit_integer_gemm_amd as lb  # noqa: E402

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINEL = 0x5A5A5A5A


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_conv(kind, x, f, stride, pad, variant):
    N, H, W = x.shape[:3]
    Co, Kh, Kw = f.shape[:3]
    Ho, Wo = lb.conv_out_dims(H, W, Kh, Kw, stride, pad)
    n = N * Ho * Wo * Co
    flat = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.int32, device="cuda")
    Y = flat[GUARD:GUARD + n].view(N, Ho, Wo, Co)
    if kind == "s8":
        lb.lb_conv2d_s8(to_dev(x), to_dev(f), Y, stride, pad, variant)
    else:
        lb.lb_conv2d_s4(to_dev(x), to_dev(f), Y, stride, pad, variant)
    torch.cuda.synchronize()
    head, tail = flat[:GUARD].cpu(), flat[-GUARD:].cpu()
    assert (head == SENTINEL).all() and (tail == SENTINEL).all(), "write outside Y"
    return Y.cpu().numpy()


def make(kind, N, H, W, C, Co, Kh, Kw, seed):
    if kind == "s8":
        return inputs.s8_nhwc(N, H, W, C, seed), inputs.s8_nhwc(Co, Kh, Kw, C, seed + 1)
    return inputs.s4_nhwc(N, H, W, C, seed), inputs.s4_nhwc(Co, Kh, Kw, C, seed + 1)


def ref(kind, x, f, C, stride, pad):
    if kind == "s8":
        return oracle.conv2d_s8(x, f, stride, pad)
    return oracle.conv2d_s4(x, f, C, stride, pad)


# (N, H, W, C, Co, Kh, Kw, stride, pad); C is in elements (64 or more bytes per pixel)
SMALL = [
    (2, 9, 7, 128, 40, 3, 3, (1, 1), (1, 1)),
    (1, 12, 10, 128, 72, 3, 2, (2, 1), (1, 0)),
    (3, 5, 6, 256, 33, 1, 1, (1, 1), (0, 0)),
    (1, 11, 13, 128, 17, 5, 5, (2, 2), (2, 2)),
    (2, 4, 5, 128, 9, 3, 3, (1, 1), (3, 3)),      # padding wider than the filter reach
    (1, 7, 9, 256, 24, 1, 1, (3, 2), (0, 0)),
    (1, 1, 1, 128, 5, 1, 1, (1, 1), (0, 0)),      # a single pixel
    (1, 6, 3, 128, 130, 1, 7, (1, 1), (0, 3)),    # 1 x 7 filter, Co over two medium tiles
]


def conv_c(kind, C):
    """Channel count for the dtype: int8 cases halve C where it stays a multiple of 64."""
    return C if kind == "s4" else max(64, C // 2)


@pytest.mark.parametrize("kind", ["s8", "s4"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_conv_small_all_variants(kind, case):
    N, H, W, C, Co, Kh, Kw, st, pd = SMALL[case]
    C = conv_c(kind, C)
    x, f = make(kind, N, H, W, C, Co, Kh, Kw, 600 + 10 * case)
    want = ref(kind, x, f, C, st, pd)
    for v in [lb.LB_AUTO] + list(range(lb.LB_NUM_VARIANTS)):
        got = run_conv(kind, x, f, st, pd, v)
        np.testing.assert_array_equal(got, want, err_msg=f"{kind} case {case} variant {v}")


# Fewer than 64 channel bytes per pixel, or not a multiple of 64: a 64-byte K
# block spans several filter taps, and each 16-byte piece is gathered from its
# own tap.  (N, H, W, Cb, Co, Kh, Kw, stride, pad) with Cb in bytes per pixel
# (int8: C = Cb; int4: C = 2*Cb).
SMALL_C = [
    (2, 9, 7, 16, 40, 3, 3, (1, 1), (1, 1)),
    (1, 12, 10, 32, 72, 3, 2, (2, 1), (1, 0)),
    (1, 11, 13, 48, 17, 5, 5, (2, 2), (2, 2)),
    (2, 4, 5, 80, 9, 3, 3, (1, 1), (3, 3)),       # padding wider than the filter reach
    (1, 6, 3, 16, 130, 1, 7, (1, 1), (0, 3)),     # 1 x 7: a block crosses a filter row
    (1, 9, 8, 16, 24, 5, 1, (1, 1), (2, 0)),      # 5 x 1: every tap is a new filter row
    (2, 32, 30, 16, 64, 7, 7, (2, 2), (3, 3)),    # a 7x7 stride-2 stem, RGB padded to 16
    (1, 5, 5, 112, 33, 2, 2, (1, 1), (0, 0)),
]


@pytest.mark.parametrize("kind", ["s8", "s4"])
@pytest.mark.parametrize("case", range(len(SMALL_C)))
def test_conv_few_channels_all_variants(kind, case):
    N, H, W, Cb, Co, Kh, Kw, st, pd = SMALL_C[case]
    C = Cb if kind == "s8" else 2 * Cb
    x, f = make(kind, N, H, W, C, Co, Kh, Kw, 900 + 10 * case)
    want = ref(kind, x, f, C, st, pd)
    for v in [lb.LB_AUTO] + list(range(lb.LB_NUM_VARIANTS)):
        got = run_conv(kind, x, f, st, pd, v)
        np.testing.assert_array_equal(got, want, err_msg=f"{kind} few-channel case {case} variant {v}")


def test_conv_rgb_padded_to_16_channels():
    """A 3-channel layer run with X and F zero-padded to 16 channels equals the
    oracle's 3-channel convolution."""
    N, H, W, Co, Kh, Kw, st, pd = 2, 20, 18, 24, 7, 7, (2, 2), (3, 3)
    x3 = inputs.s8_nhwc(N, H, W, 3, 950)
    f3 = inputs.s8_nhwc(Co, Kh, Kw, 3, 951)
    want = oracle.conv2d_s8(x3, f3, st, pd)
    x16 = np.zeros((N, H, W, 16), np.int8)
    x16[..., :3] = x3
    f16 = np.zeros((Co, Kh, Kw, 16), np.int8)
    f16[..., :3] = f3
    for v in (lb.LB_AUTO, 0, 6, 7):
        np.testing.assert_array_equal(run_conv("s8", x16, f16, st, pd, v), want, err_msg=f"variant {v}")


@pytest.mark.parametrize("kind", ["s8", "s4"])
def test_conv_1x1_matches_gemm_on_gpu(kind):
    """A 1x1, stride-1, unpadded convolution is the GEMM of pixels with filters."""
    N, H, W, C, Co = 2, 17, 15, 256, 96
    x, f = make(kind, N, H, W, C, Co, 1, 1, 700)
    y = run_conv(kind, x, f, (1, 1), (0, 0), lb.LB_AUTO)
    dA = to_dev(x.reshape(N * H * W, -1))
    dB = to_dev(f.reshape(Co, -1))
    Cm = torch.empty((N * H * W, Co), dtype=torch.int32, device="cuda")
    (lb.lb_gemm_s8 if kind == "s8" else lb.lb_gemm_s4)(dA, dB, Cm)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.reshape(-1, Co), Cm.cpu().numpy())


# Layer-sized shapes (synthetic; see the design notes for the recipe).
LAYERS = {
    "7x7_s2_112x112x16": (4, 112, 112, 16, 64, 7, 7, (2, 2), (3, 3)),   # stem, RGB padded to 16
    "3x3_s1_56x56x64": (8, 56, 56, 64, 64, 3, 3, (1, 1), (1, 1)),
    "3x3_s2_28x28x128": (8, 28, 28, 128, 256, 3, 3, (2, 2), (1, 1)),
    "1x1_14x14x256": (8, 14, 14, 256, 1024, 1, 1, (1, 1), (0, 0)),
    "5x5_s1_14x14x128": (4, 14, 14, 128, 128, 5, 5, (1, 1), (2, 2)),
}


@pytest.mark.parametrize("kind", ["s8", "s4"])
@pytest.mark.parametrize("name", sorted(LAYERS))
def test_conv_layer_full_compare(kind, name):
    N, H, W, C, Co, Kh, Kw, st, pd = LAYERS[name]
    if kind == "s4" and C % 128:
        C *= 2
    x, f = make(kind, N, H, W, C, Co, Kh, Kw, 800)
    want = ref(kind, x, f, C, st, pd)
    got = run_conv(kind, x, f, st, pd, lb.LB_AUTO)
    np.testing.assert_array_equal(got, want, err_msg=f"{kind} {name}")


def test_conv_graph_capture_replays_match_eager():
    """Automatic-choice convolutions (a few-channel layer, which takes the small
    tile, and a wider one) captured into a HIP graph: every replay, with eager
    work in between, reproduces the oracle's result."""
    cases = [("s8", (2, 11, 9, 16, 48, 3, 3, (1, 1), (1, 1))), ("s4", (1, 8, 7, 128, 96, 3, 3, (2, 1), (1, 1)))]
    outs, wants = [], []
    g = torch.cuda.CUDAGraph()
    ops = []
    for kind, (N, H, W, C, Co, Kh, Kw, st, pd) in cases:
        x, f = make(kind, N, H, W, C, Co, Kh, Kw, 990)
        wants.append(ref(kind, x, f, C, st, pd))
        Ho, Wo = lb.conv_out_dims(H, W, Kh, Kw, st, pd)
        Y = torch.zeros((N, Ho, Wo, Co), dtype=torch.int32, device="cuda")
        ops.append((kind, to_dev(x), to_dev(f), Y, st, pd))
        outs.append(Y)
    fn = {"s8": lb.lb_conv2d_s8, "s4": lb.lb_conv2d_s4}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for kind, X, F, Y, st, pd in ops:
            fn[kind](X, F, Y, st, pd, lb.LB_AUTO)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for kind, X, F, Y, st, pd in ops:
            fn[kind](X, F, Y, st, pd, lb.LB_AUTO)
    for r in range(3):
        for Y in outs:
            Y.fill_(-1)
        kind, X, F, Y, st, pd = ops[0]
        scratch = torch.empty_like(Y)
        fn[kind](X, F, scratch, st, pd, 3)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for Y, want in zip(outs, wants):
            np.testing.assert_array_equal(Y.cpu().numpy(), want, err_msg=f"replay {r}")


def test_conv_extreme_values():
    """All -128 operands with padding: every output is 16384*C times its in-image
    tap count (the automatic choice here is the 64x64 tile with 64-byte stages)."""
    N, H, W, C, Co, Kh, Kw, st, pd = 1, 6, 7, 64, 20, 3, 3, (1, 2), (1, 1)
    x = np.full((N, H, W, C), -128, np.int8)
    f = np.full((Co, Kh, Kw, C), -128, np.int8)
    want = oracle.conv2d_s8(x, f, st, pd)
    for v in [lb.LB_AUTO] + list(range(lb.LB_NUM_VARIANTS)):
        np.testing.assert_array_equal(run_conv("s8", x, f, st, pd, v), want)
