"""Planted mistakes in (a copy of) the oracle must be caught by the pins.

Each test plants one plausible mistake -- a transposed operand, a wrong sign, a
dropped term, an off-by-one in the feedback range -- into the oracle on the CPU
and checks that the brute-force pins (Babai on the Kronecker lattice, quartic
vectorised GPTQ) disagree with the mutated result.  This shows the pins are
sensitive to the kinds of error they are meant to catch.
"""
import numpy as np
import pytest

import oracle
from synthetic import make_random


def _nested_sweep_py(W, Ua, Ub, s, bits, mutation=None):
    """Pure-numpy copy of the oracle's nested sweep with an optional planted mistake."""
    m, n = W.shape
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    Z = np.zeros((m, n), dtype=np.int64)
    R = np.zeros((m, n))
    for k in range(m):
        top = k - 1 if mutation == "vertical_skips_last" else k
        g = W[k].copy()
        for i in range(max(top, 0)):
            coef = Ua[k, i] if mutation == "transpose_ua" else Ua[i, k]
            if mutation == "vertical_sign":
                coef = -coef
            g -= coef * R[i]
        t = g.copy()
        for l in range(n):
            z = min(max(np.rint(t[l] / s[k]), lo), hi)
            q = s[k] * z
            d = t[l] - q
            Z[k, l] = z
            if mutation != "drop_horizontal":
                t[l + 1:] -= d * Ub[l, l + 1:]
        R[k] = (t if mutation == "residual_from_target" else g) - s[k] * Z[k]
    return Z


@pytest.fixture(scope="module")
def case():
    wl = make_random(9, 10, 3, seed=21)
    Ua, Ub = oracle.factor_unit_upper(wl.A), oracle.factor_unit_upper(wl.B)
    zb = oracle.babai_nearest_plane(wl.W, wl.A, wl.B, wl.scales, 3)
    return wl, Ua, Ub, zb


def test_unmutated_copy_agrees(case):
    wl, Ua, Ub, zb = case
    assert np.array_equal(_nested_sweep_py(wl.W, Ua, Ub, wl.scales, 3), zb)


@pytest.mark.parametrize("mutation", ["transpose_ua", "vertical_sign", "drop_horizontal",
                                      "vertical_skips_last", "residual_from_target"])
def test_mutation_is_caught(case, mutation):
    wl, Ua, Ub, zb = case
    z = _nested_sweep_py(wl.W, Ua, Ub, wl.scales, 3, mutation=mutation)
    assert not np.array_equal(z, zb), mutation


@pytest.mark.parametrize("planted", ["transpose_factor", "unnormalised_factor", "swap_sides"])
def test_factor_mistakes_are_caught(case, planted):
    wl, Ua, Ub, zb = case
    if planted == "transpose_factor":
        Ua2, Ub2 = Ua.T.copy(), Ub
        Ua2 = np.triu(Ua2) + np.eye(wl.m) - np.diag(np.diag(Ua2))  # keep it upper, unit
    elif planted == "unnormalised_factor":
        u = np.linalg.cholesky(np.linalg.inv(wl.A)).T
        Ua2, Ub2 = u, Ub
    else:
        Ua2, Ub2 = oracle.factor_unit_upper(wl.B)[: wl.m, : wl.m], Ub
    z = oracle.sweep(wl.W, Ua2, Ub2, wl.scales, 3)["Z"]
    assert not np.array_equal(z, zb), planted
