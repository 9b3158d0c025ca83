"""Exact low-bit integer GEMM for AMD MI355X (gfx950) -- Python binding.

A thin ctypes layer over ``liblbgemm.so`` whose C ABI is declared in
``include/lb_gemm.h``.  The functions keep the C names and only marshal
arguments: they read shapes from the tensors, check dtypes, devices and
contiguity, and pass raw device pointers and torch's current HIP stream to the
library.  Every step of the computation runs in the library's HIP kernels;
there is no CPU or PyTorch fallback, and importing fails loudly when the
library has not been built.

Operand conventions (see the header): A is (M, K) row-major, B is given as its
(N, K) row-major rows (a column-major K x N matrix), C is (M, N) int32.  int4
operands are (rows, K/2) uint8 with the even k in the low nibble; 1-bit
operands are (rows, K/32) 32-bit words (torch.int32 or torch.uint32 bit
patterns) with element k in bit k % 32 of word k // 32.  Convolutions take an
NHWC image X (N, H, W, C), filters F (Co, Kh, Kw, C) and write Y (N, Ho, Wo,
Co) int32; int4 tensors hold C/2 bytes in the last dimension.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblbgemm.so")

LB_OK, LB_ERR_NULL, LB_ERR_SHAPE, LB_ERR_ALIGN, LB_ERR_VARIANT, LB_ERR_OVERFLOW, LB_ERR_HIP = range(7)
LB_S8, LB_S4, LB_B1 = 0, 1, 2
LB_PLAN_LINEAR = 3   # lb_auto_plan's op code for the linear layer
LB_AUTO = -1
LB_NUM_VARIANTS = 9
LB_DEFAULT_VARIANT = 7
K_ALIGN = {LB_S8: 16, LB_S4: 32, LB_B1: 128}
K_MAX = {LB_S8: 131071, LB_S4: 131071, LB_B1: 134217600}
# Longest 1-bit K one kernel pass covers, per matrix-instruction route (FP4, the
# default, sums in fp32, exact to 2^24; the int8 route, LB_B1_ROUTE=int8, sums 64
# per pair in int32); longer K runs as K bands (see the header).
B1_PASS_K = {"fp4": 1 << 24, "int8": 33554304}
CONV_C_ALIGN = {LB_S8: 16, LB_S4: 32}

# Exported symbols of include/lb_gemm.h (checked by the CPU tests).
EXPORTS = ("lb_gemm_s8", "lb_gemm_s4", "lb_gemm_b1", "lb_gemm_s8_linear", "lb_conv2d_s8",
           "lb_conv2d_s4", "lb_select_variant", "lb_status_string", "lb_variant_info",
           "lb_build_id", "lb_auto_plan")


class LbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def load(path: str = LIB_PATH):
    """Load the library (once).  Raises if it has not been built, or if it was
    built from sources other than the ones in this tree (its lb_build_id()
    differs from the hash of csrc/ and include/)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m bit_integer_gemm_amd._build`")
    lib = ctypes.CDLL(path)
    lib.lb_build_id.argtypes = []
    lib.lb_build_id.restype = ctypes.c_char_p
    from . import _build
    built, want = lib.lb_build_id().decode(), _build.source_sha()
    if built != want:
        raise ImportError(f"{path} was built from sources {built}, the tree holds {want}: "
                          "rebuild with `python -m bit_integer_gemm_amd._build`")
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    for name in ("lb_gemm_s8", "lb_gemm_s4", "lb_gemm_b1"):
        f = getattr(lib, name)
        f.argtypes = [p, p, p, i64, i64, i64, i32, p]
        f.restype = i32
    lib.lb_gemm_s8_linear.argtypes = [p, p, p, p, p, i64, i64, i64, i32, p]
    lib.lb_gemm_s8_linear.restype = i32
    for name in ("lb_conv2d_s8", "lb_conv2d_s4"):
        f = getattr(lib, name)
        f.argtypes = [p, p, p] + [i64] * 11 + [i32, p]
        f.restype = i32
    ip = ctypes.POINTER(ctypes.c_int)
    lib.lb_select_variant.argtypes = [i32, i64, i64, i64, i32, ip, ip]
    lib.lb_select_variant.restype = i32
    lib.lb_status_string.argtypes = [i32]
    lib.lb_status_string.restype = ctypes.c_char_p
    lib.lb_variant_info.argtypes = [i32, i32, ip, ip, ip, ip]
    lib.lb_variant_info.restype = i32
    lib.lb_auto_plan.argtypes = [i32, i64, i64, i64, i32, ip, ip, ip, ip]
    lib.lb_auto_plan.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().lb_status_string(status).decode()


def build_id() -> str:
    """Source hash stamped into the loaded library."""
    return load().lb_build_id().decode()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _stream_handle(stream, device_index):
    import torch
    if stream is None:
        # torch's current stream on the operands' device (raw hipStream_t)
        return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(device_index))
    return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))


def _check(t, dtypes, shape, what):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be on a GPU (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{what}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{what}: shape {tuple(t.shape)} != {tuple(shape)}")


def _same_device(*ts):
    d = ts[0].get_device()
    for t in ts[1:]:
        if t.get_device() != d:
            raise ValueError("all operands must be on the same GPU")
    return d


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _raise(st, where):
    if st != LB_OK:
        raise LbError(st, where)


# ---------------------------------------------------------------------------
# the C ABI, one function each
# ---------------------------------------------------------------------------

def lb_gemm_s8(A, B, C, variant: int = LB_AUTO, stream=None) -> None:
    """C (M, N) int32 = A (M, K) int8 x B, B given as (N, K) int8 rows."""
    import torch
    M, K = A.shape
    N = B.shape[0]
    _check(A, (torch.int8,), (M, K), "A")
    _check(B, (torch.int8,), (N, K), "B")
    _check(C, (torch.int32,), (M, N), "C")
    _raise(load().lb_gemm_s8(_ptr(A), _ptr(B), _ptr(C), M, N, K, variant,
                             _stream_handle(stream, _same_device(A, B, C))), "lb_gemm_s8")


def lb_gemm_s4(A, B, C, variant: int = LB_AUTO, stream=None) -> None:
    """C (M, N) int32 = A x B for packed int4: A (M, K/2) uint8, B (N, K/2) uint8."""
    import torch
    M, Kh = A.shape
    N = B.shape[0]
    _check(A, (torch.uint8,), (M, Kh), "A")
    _check(B, (torch.uint8,), (N, Kh), "B")
    _check(C, (torch.int32,), (M, N), "C")
    _raise(load().lb_gemm_s4(_ptr(A), _ptr(B), _ptr(C), M, N, 2 * Kh, variant,
                             _stream_handle(stream, _same_device(A, B, C))), "lb_gemm_s4")


def lb_gemm_b1(A, B, C, variant: int = LB_AUTO, stream=None) -> None:
    """C (M, N) int32 = popcount(A AND B) over K bits: A (M, K/32), B (N, K/32) words."""
    import torch
    words = (torch.int32, torch.uint32)
    M, Kw = A.shape
    N = B.shape[0]
    _check(A, words, (M, Kw), "A")
    _check(B, words, (N, Kw), "B")
    _check(C, (torch.int32,), (M, N), "C")
    _raise(load().lb_gemm_b1(_ptr(A), _ptr(B), _ptr(C), M, N, 32 * Kw, variant,
                             _stream_handle(stream, _same_device(A, B, C))), "lb_gemm_b1")


def lb_gemm_s8_linear(X, W, sx, sw, out, variant: int = LB_AUTO, stream=None) -> None:
    """out (M, N) fp32 = (X (M, K) int8 x W (N, K) int8) * sx[m] * sw[n]."""
    import torch
    M, K = X.shape
    N = W.shape[0]
    _check(X, (torch.int8,), (M, K), "X")
    _check(W, (torch.int8,), (N, K), "W")
    _check(sx, (torch.float32,), (M,), "sx")
    _check(sw, (torch.float32,), (N,), "sw")
    _check(out, (torch.float32,), (M, N), "out")
    _raise(load().lb_gemm_s8_linear(_ptr(X), _ptr(W), _ptr(sx), _ptr(sw), _ptr(out), M, N, K, variant,
                                    _stream_handle(stream, _same_device(X, W, sx, sw, out))),
           "lb_gemm_s8_linear")


def conv_out_dims(H: int, W: int, Kh: int, Kw: int, stride=(1, 1), pad=(0, 0)):
    """(Ho, Wo) of a convolution (the formula in the header)."""
    return (H + 2 * pad[0] - Kh) // stride[0] + 1, (W + 2 * pad[1] - Kw) // stride[1] + 1


def _conv(name, dtype, X, F, Y, stride, pad, variant, stream, cdiv):
    N, H, W, cl = X.shape
    Co, Kh, Kw, cl2 = F.shape
    C = cl * cdiv
    Ho, Wo = conv_out_dims(H, W, Kh, Kw, stride, pad)
    _check(X, (dtype,), (N, H, W, cl), "X")
    _check(F, (dtype,), (Co, Kh, Kw, cl), "F")
    import torch
    _check(Y, (torch.int32,), (N, Ho, Wo, Co), "Y")
    fn = getattr(load(), name)
    _raise(fn(_ptr(X), _ptr(F), _ptr(Y), N, H, W, C, Co, Kh, Kw, stride[0], stride[1], pad[0], pad[1],
              variant, _stream_handle(stream, _same_device(X, F, Y))), name)


def lb_conv2d_s8(X, F, Y, stride=(1, 1), pad=(0, 0), variant: int = LB_AUTO, stream=None) -> None:
    """Y (N, Ho, Wo, Co) int32 = convolution of X (N, H, W, C) int8 with F (Co, Kh, Kw, C) int8."""
    import torch
    _conv("lb_conv2d_s8", torch.int8, X, F, Y, tuple(stride), tuple(pad), variant, stream, 1)


def lb_conv2d_s4(X, F, Y, stride=(1, 1), pad=(0, 0), variant: int = LB_AUTO, stream=None) -> None:
    """As lb_conv2d_s8 for packed int4: X (N, H, W, C/2) uint8, F (Co, Kh, Kw, C/2) uint8."""
    import torch
    _conv("lb_conv2d_s4", torch.uint8, X, F, Y, tuple(stride), tuple(pad), variant, stream, 2)


def lb_select_variant(dtype: int, M: int, N: int, K: int, cu_count: int = 0):
    """(best, second) variant indices for a shape; cu_count <= 0 asks the device."""
    best, second = ctypes.c_int(-1), ctypes.c_int(-1)
    _raise(load().lb_select_variant(dtype, M, N, K, cu_count, ctypes.byref(best), ctypes.byref(second)),
           "lb_select_variant")
    return best.value, second.value


def lb_variant_info(dtype: int, variant: int) -> dict:
    """Workgroup tile (rows, columns, K elements per stage) and stage count of a variant."""
    vals = [ctypes.c_int(0) for _ in range(4)]
    _raise(load().lb_variant_info(dtype, variant, *[ctypes.byref(v) for v in vals]), "lb_variant_info")
    return dict(zip(("tile_m", "tile_n", "tile_k", "stages"), (v.value for v in vals)))


def lb_auto_plan(op: int, M: int, N: int, K: int, cu_count: int = 0) -> dict:
    """What an LB_AUTO call makes for a shape: the number of launches, the first
    launch's workgroup tile and its K bands.  op: LB_S8, LB_S4, LB_B1 or
    LB_PLAN_LINEAR; cu_count <= 0 plans for the current device."""
    vals = [ctypes.c_int(0) for _ in range(4)]
    _raise(load().lb_auto_plan(op, M, N, K, cu_count, *[ctypes.byref(v) for v in vals]), "lb_auto_plan")
    return dict(zip(("launches", "tile_m", "tile_n", "k_bands"), (v.value for v in vals)))


def ops(dtype: int, M: int, N: int, K: int) -> int:
    """Operation count used for TOPS: 2*M*N*K (K in elements, or bits for 1-bit)."""
    return 2 * M * N * K
