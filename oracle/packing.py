"""Packed code format and its dequantising consumers (test infrastructure only).

The pages stop at integer codes: the quantizer outputs an integer matrix
("GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding", arxivlens page, Abstract; the
mind-verse.de article, "GPTQ-2D: Eine Weiterentwicklung der adaptiven Rundung").
Storing them at `bits` bits each is the step after; the pages define no format, so
this is the plainest dense one:

  * a code z in [lo, hi] = [-2^(bits-1), 2^(bits-1)-1] is stored as the unsigned
    field u = z - lo in [0, 2^bits - 1];
  * row r is one little-endian bit string: code c occupies bits c*bits ..
    c*bits + bits - 1 of it, least significant bit first;
  * each row is held in ceil(n*bits / 32) uint32 words (bit i of the string is bit
    i % 32 of word i // 32); unused high bits of the last word are zero.

Dequantisation is Q = diag(s) Z; the consumer is y_b = Q x_b for a batch of vectors.
"""
from __future__ import annotations

import numpy as np


def words_per_row(n: int, bits: int) -> int:
    return (n * bits + 31) // 32


def pack_rows(Z: np.ndarray, bits: int) -> np.ndarray:
    """Bit-by-bit construction of the format above (plain loops over bit positions)."""
    Z = np.asarray(Z, dtype=np.int64)
    rows, n = Z.shape
    lo = -(1 << (bits - 1))
    U = Z - lo
    if U.size and (U.min() < 0 or U.max() >= (1 << bits)):
        raise ValueError("code out of range")
    out = np.zeros((rows, words_per_row(n, bits)), dtype=np.uint64)
    for c in range(n):
        for b in range(bits):
            pos = c * bits + b
            bit = (U[:, c] >> b) & 1
            out[:, pos // 32] |= bit.astype(np.uint64) << np.uint64(pos % 32)
    return out.astype(np.uint32)


def unpack_rows(P: np.ndarray, n: int, bits: int) -> np.ndarray:
    """Inverse of pack_rows: read each field back bit by bit."""
    P = np.asarray(P, dtype=np.uint64)
    rows = P.shape[0]
    lo = -(1 << (bits - 1))
    U = np.zeros((rows, n), dtype=np.int64)
    for c in range(n):
        for b in range(bits):
            pos = c * bits + b
            bit = (P[:, pos // 32] >> np.uint64(pos % 32)) & np.uint64(1)
            U[:, c] |= bit.astype(np.int64) << b
    return (U + lo).astype(np.int32)


def dequantize(P: np.ndarray, n: int, bits: int, scales: np.ndarray) -> np.ndarray:
    """Q = diag(s) Z from the packed rows (float64)."""
    return np.asarray(scales, dtype=np.float64)[:, None] * unpack_rows(P, n, bits)


def packed_gemv(P: np.ndarray, n: int, bits: int, scales: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Y[b] = Q X[b] for each row of X (batch x n), in float64."""
    Q = dequantize(P, n, bits, scales)
    return np.asarray(X, dtype=np.float64) @ Q.T
