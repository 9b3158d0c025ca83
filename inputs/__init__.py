"""Seeded synthetic operands for the low-bit GEMM (shared by tests and benchmark).

This module draws random operands and lays them out in the packed formats the
library and the oracle both accept.  It holds none of the GEMM's arithmetic: no
products, no sums, no decoding of packed values.  Every generator uses numpy's
PCG64 with an explicit seed, so the same call gives the same bytes everywhere.

Formats (readings; the pages name 1-, 4- and 8-bit operands but no storage):
  int8  : one signed byte per element.
  int4  : signed nibbles in [-8, 7], two per byte along K, even k in the low nibble.
  1-bit : 32 elements per uint32 along K, element k in bit (k % 32) of word k // 32.
Every operand is stored as rows of K elements: A as M rows, B as N rows (the
bytes of a K x N column-major matrix).  Convolution images are NHWC and filters
(Co, Kh, Kw, C): the same rows, reshaped, with C as the packed axis.

The distributions mirror the workloads the library is measured on: uniform int8
over [-128, 127], uniform int4 over [-8, 7], Bernoulli(0.5) bits and fp32 scales
uniform in [1e-3, 1e-2].  They stand in for the tuning dataset the pages describe,
which is not available here.
"""
from __future__ import annotations

import numpy as np

# Fixed seeds of the measured workloads (A, B, ...).
SEEDS = {
    "s8_256": (1001, 1002),
    "s4_4096": (2001, 2002),
    "b1_4096": (3001, 3002),
    "linear": (5001, 5002, 5003, 5004),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def s8_rows(rows: int, K: int, seed: int) -> np.ndarray:
    """(rows, K) int8, uniform over [-128, 127]."""
    return rng(seed).integers(-128, 128, size=(rows, K), dtype=np.int8)


def s4_values(rows: int, K: int, seed: int) -> np.ndarray:
    """(rows, K) int8 holding int4 values uniform over [-8, 7] (unpacked)."""
    return rng(seed).integers(-8, 8, size=(rows, K), dtype=np.int8)


def pack_s4(values: np.ndarray) -> np.ndarray:
    """Pack (rows, K) int4 values into (rows, K/2) bytes, even k in the low nibble."""
    v = np.asarray(values)
    if v.ndim != 2 or v.shape[1] % 2:
        raise ValueError("need a 2-D array with an even number of columns")
    if v.min(initial=0) < -8 or v.max(initial=0) > 7:
        raise ValueError("int4 values must lie in [-8, 7]")
    u = (v.astype(np.int16) & 0xF).astype(np.uint8)
    return np.ascontiguousarray(u[:, 0::2] | (u[:, 1::2] << 4))


def s4_rows(rows: int, K: int, seed: int) -> np.ndarray:
    """(rows, K/2) packed int4 bytes of uniform values over [-8, 7]."""
    return pack_s4(s4_values(rows, K, seed))


def pack_b1(bits: np.ndarray) -> np.ndarray:
    """Pack a (rows, K) array of 0/1 into (rows, K/32) uint32, bit k%32 of word k//32."""
    b = np.asarray(bits)
    if b.ndim != 2 or b.shape[1] % 32:
        raise ValueError("need a 2-D array whose column count is a multiple of 32")
    if b.size and (b.min() < 0 or b.max() > 1):
        raise ValueError("bits must be 0 or 1")
    by = np.packbits(b.astype(np.uint8), axis=1, bitorder="little")
    return np.ascontiguousarray(by).view("<u4").astype(np.uint32)


def b1_rows(rows: int, K: int, seed: int) -> np.ndarray:
    """(rows, K/32) uint32 words whose bits are independent Bernoulli(0.5)."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    return rng(seed).integers(0, 2**32, size=(rows, K // 32), dtype=np.uint32)


def s8_nhwc(N: int, H: int, W: int, C: int, seed: int) -> np.ndarray:
    """(N, H, W, C) int8 image batch (or (Co, Kh, Kw, C) filters), uniform over [-128, 127]."""
    return s8_rows(N * H * W, C, seed).reshape(N, H, W, C)


def s4_nhwc(N: int, H: int, W: int, C: int, seed: int) -> np.ndarray:
    """(N, H, W, C/2) packed int4 bytes along C, values uniform over [-8, 7]."""
    return s4_rows(N * H * W, C, seed).reshape(N, H, W, C // 2)


def scales(n: int, seed: int) -> np.ndarray:
    """(n,) fp32 dequantisation scales uniform in [1e-3, 1e-2]."""
    return rng(seed).uniform(1e-3, 1e-2, size=n).astype(np.float32)
