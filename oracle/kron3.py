"""Oracle for three Kronecker factors (test infrastructure only; see the package docstring).

Source: "GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding" (arxivlens page), Abstract:
the algorithm extends to Hessians with any number of Kronecker factors.  The page
gives no further detail, so the readings are the two-factor ones carried over:

  * W is a 3-way tensor (m1 x m2 x m3) and the Gram of vec(W) (row-major, last index
    fastest) is A1 (x) A2 (x) A3;
  * the result is *defined* as one-dimensional GPTQ on vec(W) in that natural order
    (``gptq_vectorized3`` writes the definition out, quartic work, tiny inputs only);
  * one grid step per fibre along the last mode, scales of shape (m1, m2) (for m1 = 1
    these are the two-factor per-row scales).

``quantize3`` reaches the same trajectory with the structure: the unit factor of the
Kronecker Gram is U1' (x) U2' (x) U3', so the feedback into slab i1 from earlier slabs
is separable, sum_{i < i1} U1'[i, i1] R1[i], with R1[i] = g[i] - Q[i] the slab's
target after that feedback minus its rounded values; each slab is then a two-factor
problem (A2, A3) solved by the two-factor oracle sweep.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .gptq2d import _f64, _gptq_coords, factor_unit_upper, sweep


def quantize3_factored(W, U1, U2, U3, scales, bits) -> Dict[str, np.ndarray]:
    """Nested sweep over slabs in float64 given the three unit factors.

    Outer one-dimensional GPTQ over the first index with U1'; the slab "rounding" is
    the two-factor sweep with (U2', U3').  Mode-1 feedback is accumulated for each
    slab as one axpy per earlier slab, in ascending slab order, product then
    subtraction (no fused multiply-add).
    """
    W = _f64(W)
    m1, m2, m3 = W.shape
    U1 = _f64(U1)
    s = _f64(scales)
    if U1.shape != (m1, m1) or s.shape != (m1, m2):
        raise ValueError("shape mismatch")
    Z = np.empty((m1, m2, m3), dtype=np.int32)
    Q = np.empty((m1, m2, m3), dtype=np.float64)
    R1 = np.empty((m1, m2, m3), dtype=np.float64)
    for k in range(m1):
        g = W[k].copy()
        for i in range(k):
            g -= U1[i, k] * R1[i]
        out = sweep(g, U2, U3, s[k], bits)
        Z[k], Q[k] = out["Z"], out["Q"]
        R1[k] = g - Q[k]
    return {"Z": Z, "Q": Q, "R1": R1}


def quantize3(W, A1, A2, A3, scales, bits) -> Dict[str, np.ndarray]:
    """Factor the three metrics (GPTQ's route, LAPACK), then the nested sweep."""
    U1, U2, U3 = (factor_unit_upper(a) for a in (A1, A2, A3))
    out = quantize3_factored(W, U1, U2, U3, scales, bits)
    out["U1"], out["U2"], out["U3"] = U1, U2, U3
    return out


def gptq_vectorized3(W, A1, A2, A3, scales, bits) -> np.ndarray:
    """The definition: GPTQ on vec(W) with the explicit Gram kron(A1, kron(A2, A3)).

    Textbook factor (upper Cholesky of the inverse of the full Gram), no structure.
    """
    W = _f64(W)
    m1, m2, m3 = W.shape
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    H = np.kron(_f64(A1), np.kron(_f64(A2), _f64(A3)))
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    svec = np.repeat(_f64(scales).reshape(-1), m3)
    return _gptq_coords(W.reshape(-1), svec, U, lo, hi).reshape(m1, m2, m3)


def objective3(W, Q, A1, A2, A3) -> float:
    """vec(E)^T (A1 (x) A2 (x) A3) vec(E) with E = W - Q, applied mode by mode."""
    E = _f64(W) - _f64(Q)
    F = np.einsum("ai,ijk->ajk", _f64(A1), E)
    F = np.einsum("bj,ajk->abk", _f64(A2), F)
    F = np.einsum("abk,kc->abc", F, _f64(A3))
    return float(np.sum(E * F))


def certificate3(W, Q, U1, U2, U3, scales, bits) -> Dict[str, float]:
    """Closed-form check that Q is the trajectory's output for W under (U1', U2', U3').

    Along the trajectory vec(W - Q) = (U1' (x) U2' (x) U3')^T vec(Delta), Delta the
    per-entry step error.  Solving the three transposed triangular systems mode by
    mode recovers Delta*; Q is the output iff every code equals
    clamp(rint((Q + Delta*)/s)) and |Delta*| <= s/2 where no clamp was active.
    """
    from scipy.linalg import solve_triangular

    W, Q = _f64(W), _f64(Q)
    m1, m2, m3 = W.shape
    s = _f64(scales)[:, :, None]
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    X = (W - Q).reshape(m1, m2 * m3)
    X = solve_triangular(_f64(U1), X, trans="T", lower=False).reshape(m1, m2, m3)
    X = np.moveaxis(X, 1, 0).reshape(m2, m1 * m3)
    X = solve_triangular(_f64(U2), X, trans="T", lower=False).reshape(m2, m1, m3)
    X = np.moveaxis(X, 0, 1).reshape(m1 * m2, m3)
    D = solve_triangular(_f64(U3), X.T, trans="T", lower=False).T.reshape(m1, m2, m3)
    T = (Q + D) / s
    Zq = np.rint(Q / s)
    mismatch = int(np.count_nonzero(np.clip(np.rint(T), lo, hi) != Zq))
    interior = (Zq > lo) & (Zq < hi)
    excess = float(np.max((np.abs(D) / s)[interior])) if np.any(interior) else 0.0
    return {"mismatch": mismatch, "max_interior_ratio": excess, "entries": int(W.size)}
