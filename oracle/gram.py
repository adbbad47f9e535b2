"""Kronecker factor accumulation (test infrastructure only).

The quantizer takes the factors A and B of a Kronecker-factored Hessian as given
("GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding", arxivlens page, Abstract).  The pages
do not say how they are estimated; the plain reading used here is the second-moment (Gram)
matrix of the activations, accumulated over blocks of samples: A <- A + alpha X^T X for a
block X of N samples (rows) of dimension p.  Written out with a library matrix product in
float64.
"""
from __future__ import annotations

import numpy as np


def gram_accumulate(A: np.ndarray, X: np.ndarray, alpha: float) -> np.ndarray:
    X = np.asarray(X, dtype=np.float64)
    return np.asarray(A, dtype=np.float64) + alpha * (X.T @ X)


def gram_entry(X: np.ndarray, i: int, j: int) -> float:
    """One entry of X^T X as an explicit sum over the samples (for sampled checks)."""
    X = np.asarray(X, dtype=np.float64)
    return float(sum(X[n, i] * X[n, j] for n in range(X.shape[0])))
