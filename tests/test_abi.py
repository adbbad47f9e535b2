"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments
on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq2d.h")


@pytest.fixture(scope="module")
def lib():
    import two_sided_adaptive_amd as g2d
    if not os.path.exists(g2d.LIB_PATH):
        from two_sided_adaptive_amd import build
        build.build()
    return g2d.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(gptq2d_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("gptq2d_quantize", "gptq2d_factor", "gptq2d_quantize_factored",
                 "gptq2d_workspace_bytes", "gptq2d_strerror"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    import two_sided_adaptive_amd as g2d
    raw = ctypes.CDLL(g2d.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_invalid_arguments_rejected_on_host(lib):
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    # m <= 0 -> -1, n <= 0 -> -2, bits -> -3, dtype -> -4, null W -> -5 ...
    assert lib.gptq2d_quantize(0, 4, 4, 0, p, p, p, p, p, p, None, 0, None, None) == -1
    assert lib.gptq2d_quantize(4, 0, 4, 0, p, p, p, p, p, p, None, 0, None, None) == -2
    assert lib.gptq2d_quantize(4, 4, 1, 0, p, p, p, p, p, p, None, 0, None, None) == -3
    assert lib.gptq2d_quantize(4, 4, 9, 0, p, p, p, p, p, p, None, 0, None, None) == -3
    assert lib.gptq2d_quantize(4, 4, 4, 7, p, p, p, p, p, p, None, 0, None, None) == -4
    assert lib.gptq2d_quantize(4, 4, 4, 0, None, p, p, p, p, p, None, 0, None, None) == -5
    assert lib.gptq2d_quantize(4, 4, 4, 0, p, None, p, p, p, p, None, 0, None, None) == -6
    assert lib.gptq2d_quantize(4, 4, 4, 0, p, p, None, p, p, p, None, 0, None, None) == -7
    assert lib.gptq2d_quantize(4, 4, 4, 0, p, p, p, None, p, p, None, 0, None, None) == -8
    assert lib.gptq2d_quantize(4, 4, 4, 0, p, p, p, p, None, p, None, 0, None, None) == -9
    assert lib.gptq2d_quantize(4, 4, 4, 0, p, p, p, p, p, None, None, 0, None, None) == -10
    assert lib.gptq2d_quantize(4, 4, 4, 0, p, p, p, p, p, p, p, 8, None, None) == -12
    assert lib.gptq2d_quantize(4, 4, 4, 0, p, p, p, p, p, p, None, 8, None, None) == -12
    assert lib.gptq2d_quantize_factored(4, 4, 4, 1, p, p, None, p, p, p, None, 0, None,
                                        None) == -7
    assert lib.gptq2d_factor(-3, 0, p, p, None, 0, None, None) == -1
    assert lib.gptq2d_factor(8, 2, p, p, None, 0, None, None) == -2
    assert lib.gptq2d_factor(8, 0, None, p, None, 0, None, None) == -3
    assert lib.gptq2d_factor(8, 0, p, None, None, 0, None, None) == -4
    assert lib.gptq2d_factor(8, 0, p, p, p, 16, None, None) == -6


def test_workspace_sizes(lib):
    assert lib.gptq2d_workspace_bytes(0, 3, 0) == 0
    assert lib.gptq2d_workspace_bytes(3, 3, 5) == 0
    small = lib.gptq2d_workspace_bytes(32, 32, 1)
    assert small > 0 and small % 256 == 0
    assert lib.gptq2d_sweep_workspace_bytes(4096, 4096, 0) >= 4 * 4096 * 4096 * 4
    assert lib.gptq2d_workspace_bytes(4096, 4096, 1) > lib.gptq2d_workspace_bytes(4096, 4096, 0)


def test_strerror(lib):
    assert lib.gptq2d_strerror(0) == b"success"
    assert b"argument" in lib.gptq2d_strerror(-3)
    assert lib.gptq2d_strerror(12345)


def test_three_factor_arguments_rejected_on_host(lib):
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    q = lib.gptq2d_quantize3
    ok = [4, 5, 6, 4, 1, p, p, p, p, p, p, p, None, 0, None, None]
    assert q(*ok[:0], 0, *ok[1:]) == -1
    for i, bad in [(1, 0), (2, -1), (3, 1), (3, 9), (4, 3)]:
        args = list(ok)
        args[i] = bad
        assert q(*args) == -(i + 1), (i, bad)
    for i in range(5, 12):  # null W, A1, A2, A3, scales, codes, Q
        args = list(ok)
        args[i] = None
        assert q(*args) == -(i + 1), i
    args = list(ok)
    args[12], args[13] = p, 8
    assert q(*args) == -14
    args[12] = None
    assert q(*args) == -14
    assert lib.gptq2d_workspace3_bytes(0, 4, 4, 1) == 0
    assert lib.gptq2d_workspace3_bytes(4, 4, 4, 3) == 0
    w = lib.gptq2d_workspace3_bytes(16, 1024, 1024, 1)
    assert w % 256 == 0 and w >= 16 * 1024 * 1024 * 8 + 2 * 1024 * 1024 * 8


def test_packing_arguments_rejected_on_host(lib):
    p = ctypes.c_void_p(16)
    assert lib.gptq2d_packed_row_words(11, 3) == 2
    assert lib.gptq2d_packed_row_words(4096, 4) == 512
    assert lib.gptq2d_packed_row_words(0, 4) == 0 and lib.gptq2d_packed_row_words(8, 9) == 0
    assert lib.gptq2d_pack(0, 4, 4, p, p, None) == -1
    assert lib.gptq2d_pack(4, 0, 4, p, p, None) == -2
    assert lib.gptq2d_pack(4, 4, 1, p, p, None) == -3
    assert lib.gptq2d_pack(4, 4, 4, None, p, None) == -4
    assert lib.gptq2d_pack(4, 4, 4, p, None, None) == -5
    assert lib.gptq2d_unpack(4, 4, 4, 3, p, p, p, None) == -4
    assert lib.gptq2d_unpack(4, 4, 4, 1, p, None, p, None) == -6
    assert lib.gptq2d_unpack(4, 4, 4, 1, p, p, None, None) == -7
    assert lib.gptq2d_packed_gemv(4, 4, 4, 1, p, p, 0, p, p, None) == -7
    assert lib.gptq2d_packed_gemv(4, 4, 4, 1, p, p, 9, p, p, None) == -7
    assert lib.gptq2d_packed_gemv(4, 4, 4, 1, p, p, 2, None, p, None) == -8
    assert lib.gptq2d_packed_gemv(4, 4, 4, 1, p, p, 2, p, None, None) == -9


def test_gram_arguments_rejected_on_host(lib):
    p = ctypes.c_void_p(16)
    assert lib.gptq2d_gram_accumulate(0, 4, 1, p, 1.0, p, None) == -1
    assert lib.gptq2d_gram_accumulate(4, 0, 1, p, 1.0, p, None) == -2
    assert lib.gptq2d_gram_accumulate(4, 4, 2, p, 1.0, p, None) == -3
    assert lib.gptq2d_gram_accumulate(4, 4, 1, None, 1.0, p, None) == -4
    assert lib.gptq2d_gram_accumulate(4, 4, 1, p, float("nan"), p, None) == -5
    assert lib.gptq2d_gram_accumulate(4, 4, 1, p, float("inf"), p, None) == -5
    assert lib.gptq2d_gram_accumulate(4, 4, 1, p, 1.0, None, None) == -6
    P = (ctypes.c_int64 * 2)(4, 0)
    N = (ctypes.c_int64 * 2)(3, 3)
    X = (ctypes.c_void_p * 2)(16, 16)
    al = (ctypes.c_double * 2)(1.0, 1.0)
    assert lib.gptq2d_gram_accumulate_batched(0, P, N, 1, X, al, X, None) == -1
    assert lib.gptq2d_gram_accumulate_batched(2, P, N, 1, X, al, X, None) == -2   # p[1] = 0
    P[1] = 4
    assert lib.gptq2d_gram_accumulate_batched(2, P, N, 7, X, al, X, None) == -4
    assert lib.gptq2d_gram_accumulate_batched(2, P, N, 1, None, al, X, None) == -5


def test_noalloc_arguments_and_limit_checked_on_host(lib):
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    q = lib.gptq2d_quantize_noalloc
    ok = [4, 4, 4, 1, p, p, p, p, p, p, None, None]
    for i, bad in [(0, 0), (1, -2), (2, 1), (2, 9), (3, 2)]:
        args = list(ok)
        args[i] = bad
        assert q(*args) == -(i + 1), (i, bad)
    for i in range(4, 10):  # null W, A, B, scales, codes, Q
        args = list(ok)
        args[i] = None
        assert q(*args) == -(i + 1), i
    # a problem whose workspace exceeds the static buffer is refused before any HIP call
    limit = 64 << 20
    assert lib.gptq2d_workspace_bytes(896, 896, 1) <= limit
    assert lib.gptq2d_workspace_bytes(1024, 1024, 1) > limit
    assert q(1024, 1024, 4, 1, p, p, p, p, p, p, None, None) == 3
    assert q(2000, 64, 4, 0, p, p, p, p, p, p, None, None) == 3
    assert b"scratch" in lib.gptq2d_strerror(3)
