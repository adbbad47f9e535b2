"""Seeded generators for the layer shapes the GPTQ-2D pages talk about.

The pages ("GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding", Abstract) quantize
the linear layers of Llama-3.1-70B-Instruct under a Kronecker-factored Hessian.
Neither the weights nor the calibration data exist here, so these seeded,
synthetic layers stand in for them with 8B/70B-class projection shapes.

Every array is produced in float64 with numpy's PCG64 generator and then rounded
through the workload's native dtype, so the float32 and float64 runs of one
workload solve exactly the same problem.  The recipes (seed, distributions,
outliers, spectrum, damping) are documented next to each builder below.

Only inputs are produced here: W (m x n), the SPD matrices A (m x m, acting on
rows) and B (n x n, acting on columns), and the per-row grid scales
``s_k = max_l |W_kl| / hi`` with hi = 2**(bits-1) - 1.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Callable, Dict, Optional

import numpy as np

CONFIG_NAMES = ("C1", "C2", "C3", "C4", "C4T", "C5")


@dataclasses.dataclass
class Workload:
    name: str
    W: np.ndarray        # (m, n) float64, values representable in `dtype`
    A: np.ndarray        # (m, m) float64, symmetric
    B: np.ndarray        # (n, n) float64, symmetric
    scales: np.ndarray   # (m,) float64, representable in `dtype`
    bits: int
    dtype: str           # native dtype: "f32" or "f64"
    recipe: str

    @property
    def m(self) -> int:
        return self.W.shape[0]

    @property
    def n(self) -> int:
        return self.W.shape[1]

    @property
    def lo(self) -> int:
        return -(1 << (self.bits - 1))

    @property
    def hi(self) -> int:
        return (1 << (self.bits - 1)) - 1

    def cast(self, dtype: str):
        """Return (W, A, B, scales) as contiguous arrays of `dtype` ("f32"/"f64")."""
        np_dt = np.float32 if dtype == "f32" else np.float64
        return tuple(np.ascontiguousarray(x, dtype=np_dt)
                     for x in (self.W, self.A, self.B, self.scales))


# --------------------------------------------------------------------------
# building blocks (input generation only)
# --------------------------------------------------------------------------

def _round_through(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _sym(x: np.ndarray) -> np.ndarray:
    return 0.5 * (x + x.T)


def _haar(rng: np.random.Generator, p: int) -> np.ndarray:
    """Haar-random orthogonal matrix: QR of a Gaussian with the sign of diag(R) fixed."""
    g = rng.standard_normal((p, p))
    q, r = np.linalg.qr(g)
    q *= np.sign(np.diag(r))[None, :]
    return q


def _exact_gram(x: np.ndarray, frac_bits: int) -> np.ndarray:
    """X^T X of the samples rounded to multiples of 2^-frac_bits, computed exactly.

    The rounded samples are integers times 2^-frac_bits; while N * max|X|^2 * 4^frac_bits
    stays below 2^53 every product and partial sum of the integer Gram is exact in float64,
    so the result does not depend on the BLAS summation order, the thread count or the
    CPU.  Only a sample lying within rounding error of a grid midpoint could round
    differently on another machine, which the fine grid makes rare.  The rounding moves a
    sample by at most 2^-(frac_bits+1), far below the damping that is added afterwards.
    """
    xi = np.rint(np.ldexp(x, frac_bits))
    big = float(np.max(np.abs(xi))) if xi.size else 0.0
    if big * big * x.shape[0] >= 2.0 ** 53:
        raise ValueError("samples too large for an exact Gram at this grid")
    g = xi.T @ xi
    return np.ldexp(g, -2 * frac_bits)


def _spectral(rng: np.random.Generator, p: int, power: float, damp: float) -> np.ndarray:
    """U diag(k^-power) U^T + damp * I with U Haar (config C2)."""
    u = _haar(rng, p)
    lam = np.arange(1, p + 1, dtype=np.float64) ** (-power)
    return _sym((u * lam[None, :]) @ u.T) + damp * np.eye(p)


def _wishart_ar1(rng: np.random.Generator, p: int, samples: int, rho: float) -> np.ndarray:
    """X^T X / N from N samples of an AR(1) feature process, plus 1 % mean-diagonal damping."""
    z = rng.standard_normal((samples, p))
    x = np.empty_like(z)
    x[:, 0] = z[:, 0]
    c = np.sqrt(1.0 - rho * rho)
    for j in range(1, p):
        x[:, j] = rho * x[:, j - 1] + c * z[:, j]
    a = _exact_gram(x, 16) / samples
    return a + 0.01 * np.mean(np.diag(a)) * np.eye(p)


def _wishart_powerlaw(rng: np.random.Generator, p: int, samples: int, power: float,
                      damp: float = 0.01) -> np.ndarray:
    """X^T X / N with X = Z diag(sqrt(k^-power)) U^T (U Haar), plus damp (1 %) mean-diagonal
    damping."""
    u = _haar(rng, p)
    lam = np.arange(1, p + 1, dtype=np.float64) ** (-power)
    z = rng.standard_normal((samples, p))
    x = (z * np.sqrt(lam)[None, :]) @ u.T
    del z, u
    a = _exact_gram(x, 15) / samples
    return a + damp * np.mean(np.diag(a)) * np.eye(p)


def _wishart_iid(rng: np.random.Generator, p: int, samples: int, ridge: float) -> np.ndarray:
    """X^T X / N + ridge * I with X i.i.d. N(0, 1) (config C1 and random small cases)."""
    x = rng.standard_normal((samples, p))
    return _sym(x.T @ x) / samples + ridge * np.eye(p)


def _row_scales(w: np.ndarray, hi: int) -> np.ndarray:
    return np.max(np.abs(w), axis=1) / float(hi)


def _finish(name, w, a, b, bits, dtype, recipe) -> Workload:
    w = _round_through(w, dtype)
    a = _round_through(_sym(a), dtype)
    b = _round_through(_sym(b), dtype)
    hi = (1 << (bits - 1)) - 1
    s = _round_through(_row_scales(w, hi), dtype)
    return Workload(name, np.ascontiguousarray(w), np.ascontiguousarray(a),
                    np.ascontiguousarray(b), np.ascontiguousarray(s), bits, dtype, recipe)


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(4)]


# --------------------------------------------------------------------------
# the five layer recipes
# --------------------------------------------------------------------------

def _c1() -> Workload:
    gw, ga, gb, _ = _streams(101)
    w = 0.02 * gw.standard_normal((32, 32))
    a = _wishart_iid(ga, 32, 256, 0.01)
    b = _wishart_iid(gb, 32, 256, 0.01)
    return _finish("C1", w, a, b, 4, "f64",
                   "32x32 fp64; W~N(0,0.02^2); A,B = X^T X/256 + 0.01 I, X 256x32 N(0,1); 4-bit")


def _c2() -> Workload:
    gw, ga, gb, go = _streams(202)
    m = n = 512
    w = 0.02 * gw.standard_normal((m, n))
    cols = go.choice(n, size=int(round(0.005 * n)), replace=False)
    w[:, cols] *= 10.0
    a = _spectral(ga, m, 1.5, 1e-3)
    b = _spectral(gb, n, 1.5, 1e-3)
    return _finish("C2", w, a, b, 4, "f32",
                   "512x512 fp32; W~N(0,0.02^2), 3 outlier columns x10; "
                   "A,B = U diag(k^-1.5) U^T + 1e-3 I (Haar U); 4-bit")


def _c3() -> Workload:
    gw, ga, gb, _ = _streams(303)
    m = n = 4096
    w = 0.015 * gw.standard_normal((m, n))
    a = _wishart_ar1(ga, m, 2048, 0.3)
    b = _wishart_ar1(gb, n, 2048, 0.3)
    return _finish("C3", w, a, b, 4, "f32",
                   "4096x4096 fp32; W~N(0,0.015^2); A,B Wishart of 2048 AR(1) samples rho=0.3 "
                   "+ 1% mean-diagonal damping; 4-bit")


def _c4() -> Workload:
    gw, ga, gb, _ = _streams(404)
    m, n = 14336, 4096
    w = gw.standard_t(5.0, size=(m, n)) * (0.01 / np.sqrt(5.0 / 3.0))
    a = _wishart_powerlaw(ga, m, 4096, 1.0)
    b = _wishart_powerlaw(gb, n, 4096, 1.0)
    return _finish("C4", w, a, b, 4, "f32",
                   "14336x4096 fp32; W Student-t(5) std 0.01; A,B Wishart of 4096 samples with "
                   "k^-1 spectrum (Haar U) + 1% damping; 4-bit")


def _c4t() -> Workload:
    base = make("C4")
    w = np.ascontiguousarray(base.W.T)
    return _finish("C4T", w, base.B, base.A, 4, "f32",
                   "transpose of C4: W'=W^T, A'=B, B'=A, scales recomputed per row")


def _c5() -> Workload:
    gw, ga, gb, go = _streams(505)
    m = n = 8192
    w = 0.01 * gw.standard_normal((m, n))
    k = int(round(0.001 * m * n))
    idx = go.choice(m * n, size=k, replace=False)
    w.reshape(-1)[idx] *= 20.0
    a = _wishart_powerlaw(ga, m, 8192, 1.2)
    b = _wishart_powerlaw(gb, n, 8192, 1.2)
    return _finish("C5", w, a, b, 3, "f32",
                   "8192x8192 fp32; W~N(0,0.01^2), 0.1% entries x20; A,B Wishart of 8192 samples "
                   "with k^-1.2 spectrum (Haar U) + 1% damping; 3-bit")


_BUILDERS: Dict[str, Callable[[], Workload]] = {
    "C1": _c1, "C2": _c2, "C3": _c3, "C4": _c4, "C4T": _c4t, "C5": _c5,
}

SHAPES = {"C1": (32, 32, 4), "C2": (512, 512, 4), "C3": (4096, 4096, 4),
          "C4": (14336, 4096, 4), "C4T": (4096, 14336, 4), "C5": (8192, 8192, 3)}


# The most recently built large workloads, kept in memory: the transposed 14336-wide layer
# is built from the untransposed one, and a test process asks for each several times.
_MEMO: Dict[str, Workload] = {}
_MEMO_KEEP = 4


def _memo_put(name: str, wl: Workload) -> None:
    if wl.W.size < (1 << 22):
        return
    for x in (wl.W, wl.A, wl.B, wl.scales):
        x.flags.writeable = False  # shared by every caller: modify copies only
    _MEMO[name] = wl
    while len(_MEMO) > _MEMO_KEEP:
        _MEMO.pop(next(iter(_MEMO)))


def make(name: str, cache_dir: Optional[str] = None) -> Workload:
    """Build workload `name` (deterministic).  With `cache_dir`, reuse an .npz cache."""
    if name not in _BUILDERS:
        raise KeyError(f"unknown workload {name!r}; known: {CONFIG_NAMES}")
    path = None
    if cache_dir:
        os.makedirs(cache_dir, exist_ok=True)
        path = os.path.join(cache_dir, f"workload_{name}.npz")
        if os.path.exists(path):
            z = np.load(path)
            return Workload(name, z["W"], z["A"], z["B"], z["scales"], int(z["bits"]),
                            str(z["dtype"]), str(z["recipe"]))
    if name in _MEMO:
        return _MEMO[name]
    wl = _BUILDERS[name]()
    _memo_put(name, wl)
    if path:
        tmp = path + ".tmp.npz"
        np.savez(tmp, W=wl.W, A=wl.A, B=wl.B, scales=wl.scales, bits=wl.bits,
                 dtype=wl.dtype, recipe=wl.recipe)
        os.replace(tmp, path)
    return wl


def make_random(m: int, n: int, bits: int = 4, seed: int = 0, dtype: str = "f64",
                kind: str = "wishart", samples: Optional[int] = None,
                global_scale: bool = False) -> Workload:
    """Small random problem for parity and pin tests.

    kind = "wishart": A, B = X^T X / N + 0.05 I with N = max(p, 8) samples, which gives
    dense, strongly coupled metrics (every feedback term matters);
    kind = "identity_a" / "identity_b" / "diagonal": A and/or B replaced by the identity
    or a random positive diagonal (reductions to one-sided GPTQ and to RTN).
    global_scale=True uses one scale for all rows (needed by the transpose symmetry).
    """
    gw, ga, gb, _ = _streams(10_000 + seed)
    w = 0.02 * gw.standard_normal((m, n))
    na = samples or max(m, 8)
    nb = samples or max(n, 8)
    a = _wishart_iid(ga, m, na, 0.05)
    b = _wishart_iid(gb, n, nb, 0.05)
    if kind in ("identity_a", "diagonal"):
        a = np.eye(m) if kind == "identity_a" else np.diag(ga.uniform(0.5, 2.0, m))
    if kind in ("identity_b", "diagonal"):
        b = np.eye(n) if kind == "identity_b" else np.diag(gb.uniform(0.5, 2.0, n))
    wl = _finish(f"rand{m}x{n}b{bits}s{seed}{kind}", w, a, b, bits, dtype, f"random {kind}")
    if global_scale:
        wl.scales[:] = _round_through(np.array([np.max(np.abs(wl.W)) / wl.hi]), dtype)[0]
    return wl


# --------------------------------------------------------------------------
# three-factor (tensor) workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload3:
    """A 3-way weight tensor W (m1 x m2 x m3) under the Gram A1 (x) A2 (x) A3.

    scales has shape (m1, m2): one grid step per fibre along the last mode (for
    m1 = 1 this is the per-row scale of the two-factor problem).
    """
    name: str
    W: np.ndarray
    A1: np.ndarray
    A2: np.ndarray
    A3: np.ndarray
    scales: np.ndarray
    bits: int
    dtype: str
    recipe: str

    @property
    def shape(self):
        return self.W.shape


def _finish3(name, w, a1, a2, a3, bits, dtype, recipe) -> Workload3:
    w = _round_through(w, dtype)
    hi = (1 << (bits - 1)) - 1
    s = _round_through(np.max(np.abs(w), axis=2) / float(hi), dtype)
    mats = [np.ascontiguousarray(_round_through(_sym(a), dtype)) for a in (a1, a2, a3)]
    return Workload3(name, np.ascontiguousarray(w), *mats, np.ascontiguousarray(s), bits,
                     dtype, recipe)


SHAPES3 = {"K1": (4, 96, 80, 4), "K2": (16, 1024, 1024, 4)}


def make3(name: str) -> Workload3:
    """Three-factor workloads: K1 a small parity case, K2 the measured size.

    K2 stands for a stack of 16 square 1024-wide blocks (heads or experts) whose
    Hessian factors over stack index, rows and columns; each factor is a Wishart
    matrix of AR(1) samples as in the 4096-wide layer, the stack factor with a
    stronger correlation (rho = 0.5) so that the mode-1 feedback matters.
    """
    if name not in SHAPES3:
        raise KeyError(f"unknown workload {name!r}; known: {tuple(SHAPES3)}")
    m1, m2, m3, bits = SHAPES3[name]
    gw, g1, g2, g3 = _streams(707 if name == "K1" else 808)
    w = 0.015 * gw.standard_normal((m1, m2, m3))
    a1 = _wishart_ar1(g1, m1, 4 * m1, 0.5)
    a2 = _wishart_ar1(g2, m2, 2 * m2, 0.3)
    a3 = _wishart_ar1(g3, m3, 2 * m3, 0.3)
    return _finish3(name, w, a1, a2, a3, bits, "f64",
                    f"{m1}x{m2}x{m3} fp64; W~N(0,0.015^2); A1 Wishart of {4 * m1} AR(1) "
                    f"samples rho=0.5, A2/A3 of 2p samples rho=0.3, + 1% damping; {bits}-bit")


def make_random3(m1: int, m2: int, m3: int, bits: int = 4, seed: int = 0,
                 dtype: str = "f64", kind: str = "wishart") -> Workload3:
    """Small random tensor problem; kind "identity1" makes A1 the identity."""
    gw, g1, g2, g3 = _streams(20_000 + seed)
    w = 0.02 * gw.standard_normal((m1, m2, m3))
    a1 = np.eye(m1) if kind == "identity1" else _wishart_iid(g1, m1, max(m1, 8), 0.05)
    a2 = _wishart_iid(g2, m2, max(m2, 8), 0.05)
    a3 = _wishart_iid(g3, m3, max(m3, 8), 0.05)
    return _finish3(f"rand3_{m1}x{m2}x{m3}b{bits}s{seed}{kind}", w, a1, a2, a3, bits, dtype,
                    f"random3 {kind}")


def make_conditioned(p: int, damp: float, bits: int = 4, seed: int = 0) -> Workload:
    """Square p x p layer whose metrics A, B = U diag(k^-1.5) U^T + damp * I (Haar U, as in
    the 512-wide layer) have condition number about 1/damp: the precision study's inputs."""
    gw, ga, gb, _ = _streams(30_000 + seed)
    w = 0.02 * gw.standard_normal((p, p))
    a = _spectral(ga, p, 1.5, damp)
    b = _spectral(gb, p, 1.5, damp)
    return _finish(f"cond{p}d{damp:g}", w, a, b, bits, "f32",
                   f"{p}x{p}; W~N(0,0.02^2); A,B = U diag(k^-1.5) U^T + {damp:g} I (Haar U); "
                   f"{bits}-bit")


def make_powerlaw(p: int, power: float, damp: float, bits: int = 4, seed: int = 0) -> Workload:
    """Square p x p layer with the metrics of the 14336- and 8192-wide layers scaled down: A, B
    Wishart of p samples with a k^-power spectrum (Haar U) plus damp mean-diagonal damping,
    W i.i.d. N(0, 0.01^2); the precision study's second family."""
    gw, ga, gb, _ = _streams(40_000 + seed)
    w = 0.01 * gw.standard_normal((p, p))
    a = _wishart_powerlaw(ga, p, p, power, damp)
    b = _wishart_powerlaw(gb, p, p, power, damp)
    return _finish(f"pow{p}k{power:g}d{damp:g}", w, a, b, bits, "f32",
                   f"{p}x{p}; W~N(0,0.01^2); A,B Wishart of {p} samples, spectrum k^-{power:g} "
                   f"(Haar U) + {damp:g} mean-diagonal damping; {bits}-bit")
