"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these compare the oracle with itself: every check uses an independent
construction (brute-force Babai on the Kronecker lattice, the quartic vectorised
GPTQ with an explicit mn x mn Gram, one-sided textbook GPTQ, RTN, closed-form
certificate, exact invariances of the problem).
"""
import numpy as np
import pytest
import scipy.linalg as sla

import oracle
from synthetic import make, make_random


@pytest.fixture(scope="module", autouse=True)
def _build():
    oracle.build_library(force=False)


def _q(wl, **kw):
    return oracle.quantize(wl.W, wl.A, wl.B, wl.scales, wl.bits, **kw)


# --- T1: brute-force Babai nearest plane on the mn-dimensional lattice ---------

def test_c1_matches_babai_1024_dim_lattice():
    wl = make("C1")
    out = _q(wl)
    zb = oracle.babai_nearest_plane(wl.W, wl.A, wl.B, wl.scales, wl.bits)
    assert np.array_equal(out["Z"], zb)
    # the problem is non-trivial: adaptive rounding departs from RTN on many entries
    assert np.count_nonzero(out["Z"] != oracle.rtn(wl.W, wl.scales, wl.bits)) > 20


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_match_babai_and_vectorized(seed):
    rng = np.random.default_rng(seed)
    for _ in range(4):
        m, n = (int(v) for v in rng.integers(1, 17, size=2))
        bits = int(rng.integers(2, 9))
        wl = make_random(m, n, bits, seed=1000 * seed + m * 31 + n)
        out = _q(wl)
        zb = oracle.babai_nearest_plane(wl.W, wl.A, wl.B, wl.scales, bits)
        zv = oracle.gptq_vectorized(wl.W, wl.A, wl.B, wl.scales, bits)
        assert np.array_equal(out["Z"], zb), (m, n, bits)
        assert np.array_equal(out["Z"], zv), (m, n, bits)


def test_no_clamp_regime_bits16_matches_unclamped_babai():
    # with 16 bits and scales 1/100 of the range no decision is ever clamped
    wl = make_random(9, 13, 16, seed=7)
    wl.scales[:] = np.max(np.abs(wl.W), axis=1) / 100.0
    out = _q(wl)
    zb = oracle.babai_nearest_plane(wl.W, wl.A, wl.B, wl.scales, 16, clamp=False)
    assert np.array_equal(out["Z"], zb)
    assert np.abs(out["Z"]).max() < (1 << 15) - 1


def test_vectorized_gptq_up_to_48x48():
    wl = make_random(48, 40, 3, seed=3)
    out = _q(wl)
    zv = oracle.gptq_vectorized(wl.W, wl.A, wl.B, wl.scales, 3)
    assert np.array_equal(out["Z"], zv)


# --- the Babai routine itself: Gram-Schmidt box characterisation ---------------

def test_babai_residual_lies_in_gram_schmidt_box():
    """Babai's output is the lattice point whose residual has every Gram-Schmidt
    coordinate in [-1/2, 1/2] (unclamped case).  Checked with a Cholesky-based
    Gram-Schmidt of the basis in Babai's order (independent of the QR routine)."""
    wl = make_random(5, 6, 8, seed=11)
    z = oracle.babai_nearest_plane(wl.W, wl.A, wl.B, wl.scales, 8, clamp=False).reshape(-1)
    n = wl.n
    H = np.kron(wl.A, wl.B)
    svec = np.repeat(wl.scales, n)
    G = (H * svec[None, :]) * svec[:, None]            # Gram of basis b_i = C s_i e_i
    x = wl.W.reshape(-1) / svec                        # target in basis coordinates
    # Babai visits coordinate 0 first: orthogonalise in reverse order of the columns
    J = np.arange(len(x))[::-1]
    L = np.linalg.cholesky(G[np.ix_(J, J)])            # G_rev = L L^T
    # Gram-Schmidt coordinates of the residual (L^T plays the role of R in a QR)
    gs = (L.T @ (x - z)[J]) / np.diag(L)
    assert np.max(np.abs(gs)) <= 0.5 + 1e-9


# --- T3: special cases reduce to textbook routines -----------------------------

def test_identity_a_is_rowwise_one_sided_gptq():
    wl = make_random(10, 23, 3, seed=5, kind="identity_a")
    out = _q(wl)
    assert np.array_equal(out["Z"], oracle.gptq_1d(wl.W, wl.B, wl.scales, 3))


def test_identity_b_is_columnwise_one_sided_gptq():
    wl = make_random(21, 9, 4, seed=6, kind="identity_b")
    out = _q(wl)
    ref = np.stack([oracle.gptq_1d_coords(wl.W[:, l], wl.scales, wl.A, 4)
                    for l in range(wl.n)], axis=1)
    assert np.array_equal(out["Z"], ref)


def test_diagonal_metrics_reduce_to_rtn():
    wl = make_random(17, 19, 4, seed=8, kind="diagonal")
    out = _q(wl)
    assert np.array_equal(out["Z"], oracle.rtn(wl.W, wl.scales, 4))


@pytest.mark.parametrize("shape", [(1, 29), (29, 1)])
def test_single_row_or_column_is_one_sided(shape):
    m, n = shape
    wl = make_random(m, n, 3, seed=9)
    out = _q(wl)
    if m == 1:
        ref = oracle.gptq_1d(wl.W, wl.B, wl.scales, 3)
    else:
        ref = oracle.gptq_1d_coords(wl.W[:, 0], wl.scales, wl.A, 3)[:, None]
    assert np.array_equal(out["Z"], ref)


# --- T4: certificate -------------------------------------------------------------

@pytest.mark.parametrize("name", ["C1", "C2"])
def test_certificate_on_configs(name):
    wl = make(name)
    out = _q(wl)
    cert = oracle.certificate(wl.W, out["Q"], out["Ua"], out["Ub"], wl.scales, wl.bits)
    assert cert["mismatch"] == 0
    assert cert["max_interior_ratio"] <= 0.5 + 1e-9
    assert cert["min_margin"] > 1e-9


def test_certificate_detects_a_flipped_code():
    wl = make_random(12, 14, 4, seed=12)
    out = _q(wl)
    Q = out["Q"].copy()
    Z = out["Z"]
    k, l = 6, 7
    step = 1 if Z[k, l] < wl.hi else -1
    Q[k, l] += step * wl.scales[k]
    cert = oracle.certificate(wl.W, Q, out["Ua"], out["Ub"], wl.scales, wl.bits)
    assert cert["mismatch"] > 0 or cert["max_interior_ratio"] > 0.5


def test_delta_identity_w_minus_q():
    """W - Q = Ua'^T Delta Ub' along the trajectory (the separable feedback)."""
    wl = make_random(15, 11, 3, seed=13)
    Ua, Ub = oracle.factor_unit_upper(wl.A), oracle.factor_unit_upper(wl.B)
    out = oracle.sweep(wl.W, Ua, Ub, wl.scales, 3, return_delta=True)
    np.testing.assert_allclose(wl.W - out["Q"], Ua.T @ out["Delta"] @ Ub, atol=1e-13)
    # R is the error each row hands down: R = Delta Ub'
    np.testing.assert_allclose(out["R"], out["Delta"] @ Ub, atol=1e-13)


# --- T5: invariances ----------------------------------------------------------------

def test_transpose_symmetry_with_global_scale():
    wl = make_random(13, 8, 4, seed=14, global_scale=True)
    out = _q(wl)
    outT = oracle.quantize(wl.W.T.copy(), wl.B, wl.A, np.full(wl.n, wl.scales[0]), 4)
    assert np.array_equal(outT["Z"], out["Z"].T)


def test_power_of_two_metric_scaling_is_exact():
    wl = make_random(11, 12, 4, seed=15)
    out = _q(wl)
    out2 = oracle.quantize(wl.W, 4.0 * wl.A, 0.25 * wl.B, wl.scales, 4)
    assert np.array_equal(out2["Z"], out["Z"])
    assert np.array_equal(out2["Q"], out["Q"])


def test_factor_route_independence():
    """Reversed Cholesky (A = V V^T, V upper) then triangular inverse gives the same
    unit factor as GPTQ's inverse-then-Cholesky route, and the same codes."""
    wl = make("C2")
    J = np.arange(wl.m)[::-1]
    L = np.linalg.cholesky(wl.A[np.ix_(J, J)])
    Linv = sla.solve_triangular(L, np.eye(wl.m), lower=True)
    Ua_alt = Linv[np.ix_(J, J)]
    Ua_alt = Ua_alt / np.diag(Ua_alt)[:, None]
    Ua = oracle.factor_unit_upper(wl.A)
    np.testing.assert_allclose(Ua_alt, Ua, rtol=0, atol=1e-9)
    Ub = oracle.factor_unit_upper(wl.B)
    a = oracle.sweep(wl.W, Ua, Ub, wl.scales, 4)["Z"]
    b = oracle.sweep(wl.W, Ua_alt, Ub, wl.scales, 4)["Z"]
    assert np.array_equal(a, b)


def test_factor_diagonalises_by_congruence():
    """U' unit upper with U' A U'^T diagonal: the defining property of the factor."""
    wl = make_random(40, 3, 4, seed=16)
    U = oracle.factor_unit_upper(wl.A)
    assert np.allclose(np.diag(U), 1.0) and np.allclose(np.tril(U, -1), 0.0)
    M = U @ wl.A @ U.T
    off = M - np.diag(np.diag(M))
    assert np.max(np.abs(off)) < 1e-12 * np.max(np.abs(np.diag(M)))


def test_factor_rejects_non_spd():
    a = np.eye(4)
    a[2, 2] = -1.0
    with pytest.raises(np.linalg.LinAlgError):
        oracle.factor_unit_upper(a)


# --- T6: determinism of the OpenMP split -----------------------------------------------

def test_threads_are_bit_identical():
    wl = make("C2")
    Ua, Ub = oracle.factor_unit_upper(wl.A), oracle.factor_unit_upper(wl.B)
    a = oracle.sweep(wl.W, Ua, Ub, wl.scales, 4, nthreads=1)
    b = oracle.sweep(wl.W, Ua, Ub, wl.scales, 4, nthreads=4)
    assert np.array_equal(a["Z"], b["Z"]) and np.array_equal(a["Q"], b["Q"])
    assert np.array_equal(a["R"], b["R"])


# --- prefixes: the bases of the large-size parity checks --------------------------------

def test_row_and_column_prefixes_are_exact_subproblems():
    wl = make_random(23, 19, 3, seed=17)
    Ua, Ub = oracle.factor_unit_upper(wl.A), oracle.factor_unit_upper(wl.B)
    full = oracle.sweep(wl.W, Ua, Ub, wl.scales, 3)
    r, c = 9, 7
    top = oracle.sweep(wl.W[:r], Ua[:r, :r], Ub, wl.scales[:r], 3)
    left = oracle.sweep(wl.W[:, :c], Ua, Ub[:c, :c], wl.scales, 3)
    assert np.array_equal(top["Z"], full["Z"][:r])
    assert np.array_equal(left["Z"], full["Z"][:, :c])


# --- objective ------------------------------------------------------------------------------

def test_objective_is_the_kronecker_quadratic_form():
    wl = make_random(6, 5, 4, seed=18)
    Q = wl.scales[:, None] * oracle.rtn(wl.W, wl.scales, 4)
    e = (wl.W - Q).reshape(-1)
    ref = float(e @ np.kron(wl.A, wl.B) @ e)
    assert abs(oracle.objective(wl.W, Q, wl.A, wl.B) - ref) <= 1e-13 * abs(ref)


def test_adaptive_rounding_beats_rtn_on_c2():
    wl = make("C2")
    out = _q(wl)
    f_rtn = oracle.objective(wl.W, wl.scales[:, None] * oracle.rtn(wl.W, wl.scales, 4),
                             wl.A, wl.B)
    f = oracle.objective(wl.W, out["Q"], wl.A, wl.B)
    assert f < 0.8 * f_rtn


def test_golden_c1_codes_reproduce():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "c1_codes.txt")
    gold = np.loadtxt(path, dtype=np.int64, comments="#")
    wl = make("C1")
    assert np.array_equal(_q(wl)["Z"], gold)
