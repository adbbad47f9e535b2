"""Pins of the three-factor oracle (Hessian A1 (x) A2 (x) A3 over a 3-way tensor).

"GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding" (arxivlens page), Abstract: the
algorithm extends to Hessians with any number of Kronecker factors.  The result is
defined as one-dimensional GPTQ on vec(W) under the full Kronecker Gram; every check
below uses a construction independent of the nested slab sweep.
"""
import itertools

import numpy as np
import pytest

import oracle
from synthetic import make3, make_random, make_random3


@pytest.fixture(scope="module", autouse=True)
def _build():
    oracle.build_library(force=False)


def _q3(wl):
    return oracle.quantize3(wl.W, wl.A1, wl.A2, wl.A3, wl.scales, wl.bits)


@pytest.mark.parametrize("seed", range(5))
def test_matches_vectorized_definition(seed):
    rng = np.random.default_rng(900 + seed)
    for _ in range(4):
        m1, m2, m3 = (int(v) for v in rng.integers(1, 7, size=3))
        bits = int(rng.integers(2, 9))
        wl = make_random3(m1, m2, m3, bits, seed=100 * seed + 7 * m1 + 3 * m2 + m3)
        z = _q3(wl)["Z"]
        zv = oracle.gptq_vectorized3(wl.W, wl.A1, wl.A2, wl.A3, wl.scales, bits)
        assert np.array_equal(z, zv), (m1, m2, m3, bits)
    # the feedback matters: the result departs from round-to-nearest
    wl = make_random3(5, 6, 7, 3, seed=seed)
    rtn = np.clip(np.rint(wl.W / wl.scales[:, :, None]), -4, 3)
    assert np.count_nonzero(_q3(wl)["Z"] != rtn) > 10


def test_single_last_mode_is_the_two_factor_problem():
    # m3 = 1 with one scale per slab: the tensor is an m1 x m2 matrix under A1 (x) A2
    wl = make_random3(9, 11, 1, 3, seed=5)
    wl.scales[:] = wl.scales.max(axis=1, keepdims=True)
    z3 = _q3(wl)["Z"][:, :, 0]
    z2 = oracle.quantize(wl.W[:, :, 0], wl.A1, wl.A2, wl.scales[:, 0], wl.bits)["Z"]
    assert np.array_equal(z3, z2)


def test_single_slab_is_the_two_factor_problem():
    wl = make_random3(1, 13, 10, 4, seed=6)
    z3 = _q3(wl)["Z"][0]
    z2 = oracle.quantize(wl.W[0], wl.A2, wl.A3, wl.scales[0], wl.bits)["Z"]
    assert np.array_equal(z3, z2)


def test_identity_first_factor_gives_independent_slabs():
    wl = make_random3(4, 8, 9, 4, seed=7, kind="identity1")
    z3 = _q3(wl)["Z"]
    for k in range(4):
        zk = oracle.gptq_vectorized(wl.W[k], wl.A2, wl.A3, wl.scales[k], wl.bits)
        assert np.array_equal(z3[k], zk)


@pytest.mark.parametrize("perm", [p for p in itertools.permutations(range(3)) if p != (0, 1, 2)])
def test_mode_permutation_symmetry_with_global_scale(perm):
    # Feedback only flows along the product order (i1<=k1, i2<=k2, i3<=k3), so every
    # ordering of the modes visits a linear extension of it and rounds identically.
    wl = make_random3(4, 5, 6, 3, seed=8)
    wl.scales[:] = wl.scales.max()
    z = _q3(wl)["Z"]
    mats = (wl.A1, wl.A2, wl.A3)
    Wp = np.ascontiguousarray(np.transpose(wl.W, perm))
    sp = np.full(Wp.shape[:2], wl.scales.flat[0])
    zp = oracle.quantize3(Wp, *(mats[i] for i in perm), sp, wl.bits)["Z"]
    assert np.array_equal(zp, np.transpose(z, perm))


@pytest.mark.parametrize("name", ["K1"])
def test_certificate_on_three_factor_workload(name):
    wl = make3(name)
    out = _q3(wl)
    c = oracle.certificate3(wl.W, out["Q"], out["U1"], out["U2"], out["U3"], wl.scales, wl.bits)
    assert c["mismatch"] == 0
    assert c["max_interior_ratio"] <= 0.5 + 1e-9
    # a flipped code breaks it
    Q = out["Q"].copy()
    k = (1, 40, 33)
    Q[k] += wl.scales[k[:2]] * (1 if out["Z"][k] < (1 << (wl.bits - 1)) - 1 else -1)
    c2 = oracle.certificate3(wl.W, Q, out["U1"], out["U2"], out["U3"], wl.scales, wl.bits)
    assert c2["mismatch"] > 0 or c2["max_interior_ratio"] > 0.5 + 1e-9


def test_objective3_is_the_kronecker_quadratic_form():
    wl = make_random3(3, 4, 5, 4, seed=9)
    Q = wl.scales[:, :, None] * _q3(wl)["Z"]
    e = (wl.W - Q).reshape(-1)
    H = np.kron(wl.A1, np.kron(wl.A2, wl.A3))
    assert np.isclose(oracle.objective3(wl.W, Q, wl.A1, wl.A2, wl.A3), e @ H @ e, rtol=1e-12)


def test_adaptive_rounding_beats_rtn_in_three_factors():
    wl = make3("K1")
    Q = _q3(wl)["Q"]
    rtn = wl.scales[:, :, None] * np.clip(np.rint(wl.W / wl.scales[:, :, None]), -8, 7)
    f = lambda X: oracle.objective3(wl.W, X, wl.A1, wl.A2, wl.A3)  # noqa: E731
    assert f(Q) < 0.8 * f(rtn)


# --- planted mistakes in a copy of the nested loop must be caught -------------------------

def _nested(wl, mutation):
    U1, U2, U3 = (oracle.factor_unit_upper(a) for a in (wl.A1, wl.A2, wl.A3))
    m1 = wl.W.shape[0]
    Z = np.empty(wl.W.shape, dtype=np.int32)
    R1 = np.empty(wl.W.shape)
    for k in range(m1):
        g = wl.W[k].copy()
        for i in range(k):
            c = U1[k, i] if mutation == "transposed_u1" else U1[i, k]
            if mutation == "sign":
                c = -c
            g -= c * R1[i]
        out = oracle.sweep(g, U2, U3, wl.scales[k], wl.bits)
        Z[k] = out["Z"]
        R1[k] = (wl.W[k] if mutation == "residual_from_w" else g) - out["Q"]
        if mutation == "residual_is_step_error":
            R1[k] = oracle.sweep(g, U2, U3, wl.scales[k], wl.bits, return_delta=True)["Delta"]
    return Z


@pytest.mark.parametrize("mutation", [None, "transposed_u1", "sign", "residual_from_w",
                                      "residual_is_step_error"])
def test_planted_mistakes_in_the_slab_feedback_are_caught(mutation):
    cases = [make_random3(6, 8, 9, 3, seed=s) for s in (13, 14)]
    hit = False
    for wl in cases:
        zv = oracle.gptq_vectorized3(wl.W, wl.A1, wl.A2, wl.A3, wl.scales, wl.bits)
        agree = np.array_equal(_nested(wl, mutation), zv)
        if mutation is None:
            assert agree
        hit |= not agree
    assert hit == (mutation is not None)


def test_two_factor_generator_is_unchanged():
    # the added tensor builders leave the matrix builders' streams alone
    a = make_random(5, 6, 4, seed=3)
    b = make_random(5, 6, 4, seed=3)
    assert np.array_equal(a.W, b.W)
