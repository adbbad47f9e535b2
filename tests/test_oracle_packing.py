"""Pins of the packed code format oracle (oracle/packing.py).

Every check builds the expected words another way: a hand-worked example, byte and
nibble views of the same bits through numpy, and the two-factor oracle's Q.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import packing
from synthetic import make_random

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hand_worked_3bit_row():
    lines = [l for l in open(os.path.join(HERE, "golden", "pack_3bit_example.txt"))
             if not l.startswith("#")]
    z = np.array([[int(v) for v in lines[0].split()]])
    words = np.array([[int(v) for v in lines[1].split()]], dtype=np.uint32)
    assert np.array_equal(packing.pack_rows(z, 3), words)
    assert np.array_equal(packing.unpack_rows(words, z.shape[1], 3), z)


def test_8bit_fields_are_the_offset_bytes():
    rng = np.random.default_rng(1)
    z = rng.integers(-128, 128, size=(3, 13))
    P = packing.pack_rows(z, 8)
    b = np.zeros((3, 4 * P.shape[1]), dtype=np.uint8)
    b[:, :13] = (z + 128).astype(np.uint8)
    assert np.array_equal(P, b.view("<u4"))


def test_4bit_fields_are_nibbles_low_first():
    rng = np.random.default_rng(2)
    z = rng.integers(-8, 8, size=(4, 22))
    u = (z + 8).astype(np.uint8)
    u = np.concatenate([u, np.zeros((4, 2), np.uint8)], axis=1)   # 24 nibbles = 3 words
    by = u[:, 0::2] | (u[:, 1::2] << 4)
    assert np.array_equal(packing.pack_rows(z, 4), by.view("<u4"))


@pytest.mark.parametrize("bits", range(2, 9))
def test_roundtrip_and_padding_bits_are_zero(bits):
    rng = np.random.default_rng(bits)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    for n in (1, 31, 32, 33, 100):
        z = rng.integers(lo, hi + 1, size=(5, n))
        P = packing.pack_rows(z, bits)
        assert P.shape == (5, (n * bits + 31) // 32)
        assert np.array_equal(packing.unpack_rows(P, n, bits), z)
        used = n * bits - 32 * (P.shape[1] - 1)
        if used < 32:
            assert np.all(P[:, -1] >> np.uint32(used) == 0)


def test_out_of_range_code_rejected():
    with pytest.raises(ValueError):
        packing.pack_rows(np.array([[8]]), 4)


def test_dequantize_reproduces_the_quantizer_q_and_gemv():
    oracle.build_library(force=False)
    wl = make_random(9, 37, 3, seed=4)
    out = oracle.quantize(wl.W, wl.A, wl.B, wl.scales, wl.bits)
    P = packing.pack_rows(out["Z"], wl.bits)
    np.testing.assert_array_equal(packing.dequantize(P, 37, wl.bits, wl.scales), out["Q"])
    X = np.random.default_rng(5).standard_normal((3, 37))
    Y = packing.packed_gemv(P, 37, wl.bits, wl.scales, X)
    for b in range(3):      # each output written out as an explicit dot product
        for r in range(9):
            ref = sum(out["Q"][r, c] * X[b, c] for c in range(37))
            assert abs(Y[b, r] - ref) <= 1e-12 * (1 + np.abs(out["Q"][r]) @ np.abs(X[b]))
