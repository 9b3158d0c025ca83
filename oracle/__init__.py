"""CPU oracle for the low-bit integer GEMM -- TEST INFRASTRUCTURE ONLY.

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


def num_threads(*, handle=None) -> int:
    return (handle or lib()).orc_num_threads()
