"""CPU oracle for the low-bit integer GEMM and convolution -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
imports nothing from the GPU library: the two share only the seeded input
generators in ``inputs/``, which hold none of the GEMM's arithmetic.

The arithmetic lives in ``oracle.c`` (plain triple loops, see its header for
what is computed and which reading of the pages each part follows).  This module
only builds it with gcc and marshals numpy arrays into it.

Layouts (readings; the pages fix only the product A x B = C and the bit widths):
  A  : M x K row-major            (int8 / packed int4 bytes / packed 1-bit words)
  B  : K x N column-major, i.e. an (N, K) row-major array of the same kind
  C  : M x N row-major int32
Convolution (readings of the im2win convolution summary; see oracle.c):
  x  : N x H x W x C (NHWC), f : Co x Kh x Kw x C, y : N x Ho x Wo x Co int32
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
          "-Wall", "-Wextra", "-Werror"]


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *extra_flags, src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    i64 = ctypes.c_int64
    p = ctypes.c_void_p
    for name in ("orc_gemm_s8", "orc_gemm_s4", "orc_gemm_b1"):
        f = getattr(lib, name)
        f.argtypes = [p, p, p, i64, i64, i64]
        f.restype = ctypes.c_int
    lib.orc_linear_s8.argtypes = [p, p, p, p, p, i64, i64, i64]
    lib.orc_linear_s8.restype = ctypes.c_int
    conv_args = [p, p, p] + [i64] * 11
    for name in ("orc_conv2d_s8", "orc_conv2d_s4", "orc_conv2d_im2win_s8"):
        f = getattr(lib, name)
        f.argtypes = conv_args
        f.restype = ctypes.c_int
    lib.orc_im2win_s8.argtypes = [p, p] + [i64] * 10
    lib.orc_im2win_s8.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    return lib


def load_library(path: str):
    """Load an oracle shared library at ``path`` (used for planted-mistake builds)."""
    return _bind(ctypes.CDLL(path))


def lib():
    """The oracle library, built on first use if it is not there yet."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = load_library(_LIB)
    return _lib


class OracleOverflow(ArithmeticError):
    """An exact sum did not fit in int32."""


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_rows(a: np.ndarray, dtype, cols: int, what: str):
    if a.dtype != dtype or a.ndim != 2 or a.shape[1] != cols or not a.flags.c_contiguous:
        raise ValueError(f"{what}: need C-contiguous {np.dtype(dtype).name} array with "
                         f"{cols} columns, got {a.dtype} {a.shape}")


def _run(fn, A, B, C, M, N, K):
    rc = fn(_ptr(A), _ptr(B), _ptr(C), M, N, K)
    if rc != 0:
        raise OracleOverflow("a sum of products does not fit int32")
    return C


def gemm_s8(A: np.ndarray, B: np.ndarray, *, handle=None) -> np.ndarray:
    """C = A (M x K int8, row-major) times B (given as N x K int8 rows)."""
    L = handle or lib()
    M, K = A.shape
    N = B.shape[0]
    _check_rows(A, np.int8, K, "A")
    _check_rows(B, np.int8, K, "B")
    C = np.empty((M, N), np.int32)
    return _run(L.orc_gemm_s8, A, B, C, M, N, K)


def gemm_s4(A: np.ndarray, B: np.ndarray, K: int, *, handle=None) -> np.ndarray:
    """C = A x B for packed signed int4 rows (K/2 bytes each, low nibble = even k)."""
    L = handle or lib()
    if K <= 0 or K % 2:
        raise ValueError("K must be a positive multiple of 2")
    M, N = A.shape[0], B.shape[0]
    _check_rows(A, np.uint8, K // 2, "A")
    _check_rows(B, np.uint8, K // 2, "B")
    C = np.empty((M, N), np.int32)
    return _run(L.orc_gemm_s4, A, B, C, M, N, K)


def gemm_b1(A: np.ndarray, B: np.ndarray, K: int, *, handle=None) -> np.ndarray:
    """C = A x B for 1-bit rows packed 32 per uint32 (bit k%32 of word k/32)."""
    L = handle or lib()
    if K <= 0 or K % 32:
        raise ValueError("K must be a positive multiple of 32")
    M, N = A.shape[0], B.shape[0]
    _check_rows(A, np.uint32, K // 32, "A")
    _check_rows(B, np.uint32, K // 32, "B")
    C = np.empty((M, N), np.int32)
    return _run(L.orc_gemm_b1, A, B, C, M, N, K)


def linear_s8(X: np.ndarray, W: np.ndarray, sx: np.ndarray, sw: np.ndarray,
              *, handle=None) -> np.ndarray:
    """out[m, n] = (sum_k X[m,k] W[n,k]) * sx[m] * sw[n], evaluated in fp64."""
    L = handle or lib()
    M, K = X.shape
    N = W.shape[0]
    _check_rows(X, np.int8, K, "X")
    _check_rows(W, np.int8, K, "W")
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    if sx.shape != (M,) or sw.shape != (N,):
        raise ValueError("sx must have M entries and sw N entries")
    out = np.empty((M, N), np.float64)
    rc = L.orc_linear_s8(_ptr(X), _ptr(W), _ptr(sx), _ptr(sw), _ptr(out), M, N, K)
    if rc != 0:
        raise OracleOverflow("a sum of products does not fit int32")
    return out


def conv_out_dims(H, W, Kh, Kw, stride=(1, 1), pad=(0, 0)):
    """(Ho, Wo) of a convolution; ValueError for impossible geometry."""
    sh, sw = stride
    ph, pw = pad
    if sh <= 0 or sw <= 0 or ph < 0 or pw < 0 or H + 2 * ph < Kh or W + 2 * pw < Kw:
        raise ValueError("impossible convolution geometry")
    return (H + 2 * ph - Kh) // sh + 1, (W + 2 * pw - Kw) // sw + 1


def _conv_call(fn, X, F, C, stride, pad):
    N, H, W = X.shape[:3]
    Co, Kh, Kw = F.shape[:3]
    Ho, Wo = conv_out_dims(H, W, Kh, Kw, stride, pad)
    Y = np.empty((N, Ho, Wo, Co), np.int32)
    rc = fn(_ptr(X), _ptr(F), _ptr(Y), N, H, W, C, Co, Kh, Kw, stride[0], stride[1], pad[0], pad[1])
    if rc == 2:
        raise ValueError("impossible convolution geometry")
    if rc != 0:
        raise OracleOverflow("a sum of products does not fit int32")
    return Y


def _check_conv(X, F, dtype, last):
    for a, what in ((X, "X"), (F, "F")):
        if a.dtype != dtype or a.ndim != 4 or not a.flags.c_contiguous or a.shape[3] != last:
            raise ValueError(f"{what}: need a C-contiguous 4-D {np.dtype(dtype).name} array "
                             f"with last dimension {last}, got {a.dtype} {a.shape}")


def conv2d_s8(X: np.ndarray, F: np.ndarray, stride=(1, 1), pad=(0, 0), *, handle=None) -> np.ndarray:
    """y (N, Ho, Wo, Co) int32 = convolution of x (N, H, W, C) int8 with f (Co, Kh, Kw, C) int8."""
    L = handle or lib()
    _check_conv(X, F, np.int8, X.shape[3] if X.ndim == 4 else -1)
    return _conv_call(L.orc_conv2d_s8, X, F, X.shape[3], tuple(stride), tuple(pad))


def conv2d_s4(X: np.ndarray, F: np.ndarray, C: int, stride=(1, 1), pad=(0, 0), *, handle=None) -> np.ndarray:
    """Convolution of packed int4 x (N, H, W, C/2 bytes) with packed f (Co, Kh, Kw, C/2 bytes)."""
    L = handle or lib()
    if C <= 0 or C % 2:
        raise ValueError("C must be a positive multiple of 2")
    _check_conv(X, F, np.uint8, C // 2)
    return _conv_call(L.orc_conv2d_s4, X, F, C, tuple(stride), tuple(pad))


def im2win_s8(X: np.ndarray, Kh: int, Kw: int, stride=(1, 1), pad=(0, 0), *, handle=None) -> np.ndarray:
    """The window tensor (N, Ho, W + 2 pw, Kh, C) of the im2win transformation."""
    L = handle or lib()
    if X.dtype != np.int8 or X.ndim != 4 or not X.flags.c_contiguous:
        raise ValueError("X: need a C-contiguous 4-D int8 array")
    N, H, W, C = X.shape
    Ho, Wo = conv_out_dims(H, W, Kh, Kw, stride, pad)
    Win = np.empty((N, Ho, W + 2 * pad[1], Kh, C), np.int8)
    rc = L.orc_im2win_s8(_ptr(X), _ptr(Win), N, H, W, C, Kh, Kw, stride[0], stride[1], pad[0], pad[1])
    if rc:
        raise ValueError("impossible convolution geometry")
    return Win


def conv2d_im2win_s8(Win: np.ndarray, F: np.ndarray, H: int, W: int, stride=(1, 1), pad=(0, 0),
                     *, handle=None) -> np.ndarray:
    """Convolution taken from the window tensor, one contiguous window per output."""
    L = handle or lib()
    N, Ho, Wp, Kh, C = Win.shape
    Co, Kh2, Kw, C2 = F.shape
    if Win.dtype != np.int8 or F.dtype != np.int8 or Kh2 != Kh or C2 != C or Wp != W + 2 * pad[1]:
        raise ValueError("window tensor and filter do not match")
    if conv_out_dims(H, W, Kh, Kw, stride, pad)[0] != Ho:
        raise ValueError("window tensor does not match the geometry")
    Wo = conv_out_dims(H, W, Kh, Kw, stride, pad)[1]
    Y = np.empty((N, Ho, Wo, Co), np.int32)
    rc = L.orc_conv2d_im2win_s8(_ptr(np.ascontiguousarray(Win)), _ptr(np.ascontiguousarray(F)), _ptr(Y),
                                N, H, W, C, Co, Kh, Kw, stride[0], stride[1], pad[0], pad[1])
    if rc == 2:
        raise ValueError("impossible convolution geometry")
    if rc:
        raise OracleOverflow("a sum of products does not fit int32")
    return Y


def num_threads(*, handle=None) -> int:
    return (handle or lib()).orc_num_threads()
