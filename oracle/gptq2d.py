"""Oracle for GPTQ-2D (test infrastructure only; see the package docstring).

Sources, cited by page title and section:
  [arXiv]   "GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding" (arxivlens page):
            Abstract, Results, Limitations, Methodology, Technical contributions.
  [article] "Neue Ansaetze zur Effizienzsteigerung von Large Language Models durch
            GPTQ-2D" (mind-verse.de): sections "GPTQ-2D: Eine Weiterentwicklung der
            adaptiven Rundung", "Die algorithmische Neuerung und ihre Auswirkungen",
            "Geometrische Grundlagen und der Bezug zu Babai's Nearest Plane
            Algorithmus".

Problem (both pages): W (m x n) real, A (m x m) and B (n x n) fixed SPD; find
Q = diag(s) Z with Z integer in [lo, hi] by adaptive rounding under
tr(A (W-Q) B (W-Q)^T).  The result is *defined* as the trajectory of the naive
vectorised sweep, i.e. one-dimensional GPTQ on vec(W) with Gram A (x) B
([article] "Die algorithmische Neuerung", "Geometrische Grundlagen"; [arXiv]
Results).  ``gptq_vectorized`` is that definition written out (quartic work);
``sweep`` reaches the same trajectory in cubic work through the separable
rank-one structure of the feedback ([arXiv] Results, Technical contributions).

Readings where the pages are silent (all documented in the design notes):
  * natural coordinate order (row 0 / column 0 first), no reordering;
  * the triangular feedback factor is GPTQ's: the upper Cholesky factor of the
    inverse Gram, scaled to a unit diagonal;
  * rounding is IEEE round-half-to-even of the IEEE quotient t/s, then clamp;
  * symmetric signed grid lo = -2^(bits-1) .. hi = 2^(bits-1)-1 with fixed per-row
    scales.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Tuple

import numpy as np
import scipy.linalg as sla
from scipy.linalg import lapack

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nested_sweep.c")
_LIB = os.path.join(_HERE, "_nested_sweep.so")
_lib_handle = None


# ---------------------------------------------------------------------------
# build / load the plain-C sweep
# ---------------------------------------------------------------------------

def build_library(force: bool = True) -> str:
    """Compile nested_sweep.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_library(force=True)
        lib = ctypes.CDLL(_LIB)
        f = lib.oracle_gptq2d_sweep
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 4 + \
                     [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int]
        _lib_handle = lib
    return _lib_handle


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x: np.ndarray) -> int:
    return x.ctypes.data


# ---------------------------------------------------------------------------
# the method
# ---------------------------------------------------------------------------

def factor_unit_upper(A: np.ndarray) -> np.ndarray:
    """Unit-diagonal triangular feedback factor of an SPD matrix.

    [article] "GPTQ-2D: Eine Weiterentwicklung": errors propagate through a
    triangular feedback matrix; [arXiv] Limitations: fixed bases need their
    factorisations.  Reading: GPTQ's route, A^-1 = U^T U with U upper (Cholesky of
    the inverse), then U' = diag(U)^-1 U.  Computed with LAPACK in float64:
    potrf(A) -> potri (inverse) -> potrf of the inverse (upper).
    """
    a = _f64(A)
    if a.ndim != 2 or a.shape[0] != a.shape[1]:
        raise ValueError("A must be square")
    c, info = lapack.dpotrf(a, lower=1, clean=1)
    if info != 0:
        raise np.linalg.LinAlgError(f"matrix not SPD (potrf info={info})")
    inv, info = lapack.dpotri(c, lower=1)
    if info != 0:
        raise np.linalg.LinAlgError(f"potri info={info}")
    inv = np.tril(inv) + np.tril(inv, -1).T
    u, info = lapack.dpotrf(inv, lower=0, clean=1)
    if info != 0:
        raise np.linalg.LinAlgError(f"inverse not SPD (potrf info={info})")
    u = np.triu(u)
    return np.ascontiguousarray(u / np.diag(u)[:, None])


def sweep(W: np.ndarray, Ua: np.ndarray, Ub: np.ndarray, scales: np.ndarray, bits: int,
          nthreads: int = 0, return_delta: bool = False) -> Dict[str, np.ndarray]:
    """Cubic nested sweep in float64 (plain C), given the unit factors.

    Returns dict(Z=int32 codes, Q=float64 dequantised values, R=vertical residual,
    [Delta=step errors], threads=OpenMP threads used).  [arXiv] Results: same
    rounding as the one-dimensional trajectory with cubic work.
    """
    W = _f64(W)
    m, n = W.shape
    Ua, Ub, s = _f64(Ua), _f64(Ub), _f64(scales)
    if Ua.shape != (m, m) or Ub.shape != (n, n) or s.shape != (m,):
        raise ValueError("shape mismatch")
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    Z = np.empty((m, n), dtype=np.int32)
    Q = np.empty((m, n), dtype=np.float64)
    R = np.empty((m, n), dtype=np.float64)
    D = np.empty((m, n), dtype=np.float64) if return_delta else None
    used = _lib().oracle_gptq2d_sweep(m, n, _ptr(W), _ptr(Ua), _ptr(Ub), _ptr(s), lo, hi,
                                      _ptr(Z), _ptr(Q), _ptr(R),
                                      _ptr(D) if D is not None else None, int(nthreads))
    if used < 0:
        raise RuntimeError("oracle sweep failed")
    out = {"Z": Z, "Q": Q, "R": R, "threads": used}
    if D is not None:
        out["Delta"] = D
    return out


def quantize(W, A, B, scales, bits, nthreads: int = 0) -> Dict[str, np.ndarray]:
    """Factor both sides, then sweep.  Returns the sweep dict plus Ua, Ub."""
    Ua = factor_unit_upper(A)
    Ub = factor_unit_upper(B)
    out = sweep(W, Ua, Ub, scales, bits, nthreads=nthreads)
    out["Ua"], out["Ub"] = Ua, Ub
    return out


def objective(W, Q, A, B) -> float:
    """tr(A E B E^T), E = W - Q ([arXiv] Methodology: Kronecker-structured metric)."""
    E = _f64(W) - _f64(Q)
    return float(np.sum((_f64(A) @ E) * (E @ _f64(B))))


def rtn(W, scales, bits) -> np.ndarray:
    """Round-to-nearest codes clamp(rint(W/s)) (the baseline named by the article)."""
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    return np.clip(np.rint(_f64(W) / _f64(scales)[:, None]), lo, hi).astype(np.int32)


def _gptq_coords(x: np.ndarray, svec: np.ndarray, U: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Textbook GPTQ over the coordinates of x (U = upper Cholesky of the inverse Hessian)."""
    x = x.copy()
    z = np.empty(x.shape[0], dtype=np.int32)
    for c in range(x.shape[0]):
        zc = min(max(np.rint(x[c] / svec[c]), lo), hi)
        z[c] = int(zc)
        err = (x[c] - svec[c] * zc) / U[c, c]
        x[c + 1:] -= err * U[c, c + 1:]
    return z


def gptq_1d_coords(x, svec, H, bits) -> np.ndarray:
    """One-sided GPTQ of one vector x with Hessian H and per-coordinate scales svec."""
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    U = np.linalg.cholesky(np.linalg.inv(_f64(H))).T
    return _gptq_coords(_f64(x), _f64(svec), U, lo, hi)


def gptq_1d(W, H, scales, bits) -> np.ndarray:
    """One-sided GPTQ of each row of W with column Hessian H (GPTQ, cited by the article).

    Factor by the same textbook route: U = upper Cholesky of inv(H), no unit scaling.
    """
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    W = _f64(W)
    U = np.linalg.cholesky(np.linalg.inv(_f64(H))).T
    out = np.empty(W.shape, dtype=np.int32)
    for k in range(W.shape[0]):
        out[k] = _gptq_coords(W[k], np.full(W.shape[1], float(scales[k])), U, lo, hi)
    return out


def gptq_vectorized(W, A, B, scales, bits) -> np.ndarray:
    """The definition: GPTQ on vec_r(W) with the explicit mn x mn Gram kron(A, B).

    [article] "Geometrische Grundlagen": vectorising turns the two-sided problem into
    one quadratic form whose Gram matrix is a Kronecker product; "Die algorithmische
    Neuerung": the method follows the naive vectorised sweep exactly.  Quartic work:
    only for tiny inputs.  Uses no Kronecker structure in its factorisation.
    """
    W = _f64(W)
    m, n = W.shape
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    H = np.kron(_f64(A), _f64(B))
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    svec = np.repeat(_f64(scales), n)
    return _gptq_coords(W.reshape(-1), svec, U, lo, hi).reshape(m, n)


def babai_nearest_plane(W, A, B, scales, bits, clamp: bool = True) -> np.ndarray:
    """Babai's nearest-plane algorithm on the mn-dimensional Kronecker lattice.

    [article] "Geometrische Grundlagen": rounding under a quadratic metric is a
    closest-lattice-point problem, GPTQ is Babai's algorithm, and vectorisation gives
    the Gram A (x) B.  Lattice basis: columns of C diag(s) with C the symmetric
    square root of A (x) B, target C vec(W).  Babai's back substitution visits the
    last basis vector first, so the basis is reversed to visit coordinate 0 first
    (GPTQ's order).  With clamp=True each integer coordinate is clamped to [lo, hi]
    as it is decided (box-constrained variant).
    """
    W = _f64(W)
    m, n = W.shape
    N = m * n
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    H = np.kron(_f64(A), _f64(B))
    evals, evecs = np.linalg.eigh(H)
    C = (evecs * np.sqrt(evals)[None, :]) @ evecs.T
    svec = np.repeat(_f64(scales), n)
    M = (C * svec[None, :])[:, ::-1]          # column c <-> coordinate N-1-c
    Qm, Rm = np.linalg.qr(M)
    y = Qm.T @ (C @ W.reshape(-1))
    zr = np.zeros(N)
    for c in range(N - 1, -1, -1):
        v = np.rint((y[c] - Rm[c, c + 1:] @ zr[c + 1:]) / Rm[c, c])
        zr[c] = min(max(v, lo), hi) if clamp else v
    return zr[::-1].reshape(m, n).astype(np.int64)


def certificate(W, Q, Ua, Ub, scales, bits) -> Dict[str, float]:
    """Closed-form check that Q is the GPTQ-2D output for W under (Ua', Ub').

    Along the trajectory W - Q = Ua'^T Delta Ub', with Delta the per-entry step error
    (target minus rounded value).  So Delta* = Ua'^-T (W-Q) Ub'^-1 (two triangular
    solves) must satisfy Z = clamp(rint((Q + Delta*)/s)) everywhere and
    |Delta*| <= s/2 where no clamp was active; by induction over the dominance order
    this pins Q uniquely in exact arithmetic.  Returns counts and the smallest
    distance of (Q+Delta*)/s from a rounding boundary among entries where the
    decision is not clamped away.
    """
    W, Q, Ua, Ub = _f64(W), _f64(Q), _f64(Ua), _f64(Ub)
    s = _f64(scales)[:, None]
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    X = sla.solve_triangular(Ua, W - Q, trans="T", lower=False)
    D = sla.solve_triangular(Ub, X.T, trans="T", lower=False).T
    T = (Q + D) / s
    Zq = np.rint(Q / s)
    Zc = np.clip(np.rint(T), lo, hi)
    mismatch = int(np.count_nonzero(Zc != Zq))
    interior = (Zq > lo) & (Zq < hi)
    ratio = np.abs(D) / s
    excess = float(np.max(ratio[interior])) if np.any(interior) else 0.0
    frac = np.abs(T - np.floor(T) - 0.5)
    live = (T > lo - 0.5) & (T < hi + 0.5)
    margin = float(np.min(frac[live])) if np.any(live) else 0.5
    return {"mismatch": mismatch, "max_interior_ratio": excess, "min_margin": margin,
            "entries": int(W.size)}
