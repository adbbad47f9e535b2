"""Write tests/golden/large_configs.json: oracle results for the full-size layers.

Only oracle/ and synthetic/ are used.  For each of the 4096x4096, 14336x4096 (and its
transpose) and 8192x8192 layers the script builds the seeded inputs, runs the oracle
(LAPACK factors, plain-C nested sweep in float64) on them and stores
  * SHA-256 digests of the float32 inputs (W, A, B, scales), so that a test can tell
    whether its own generator run produced the same problem;
  * the SHA-256 of the oracle's int8 code matrix (row-major) and of each block of 256
    rows, so that a test can check a full code matrix without the oracle's minutes of
    CPU time, and name the first block that differs;
  * the objective tr(A E B E^T) of the oracle's result and of round-to-nearest;
  * the distances |frac(t/s) - 1/2| of the oracle's own rounding targets from a
    rounding boundary: their minimum, how many fall below each threshold, and how many
    entries lie in the dependency cones (rows at or below and columns at or right of
    the entry) of the entries below each threshold.  An arithmetic whose error in t/s
    can reach a threshold may decide those entries differently, and every entry in
    their cones may then follow another trajectory.
Run:  python tests/golden/make_large_digests.py [names...]   (minutes of CPU per layer)
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synthetic import make  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "large_configs.json")
NAMES = ("C3", "C4", "C4T", "C5")
BLOCK_ROWS = 256
THRESHOLDS = (1e-3, 1e-4, 1e-5, 1e-6, 1e-7, 1e-8, 1e-9, 1e-10)


def sha(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()


def cone_size(mask: np.ndarray) -> int:
    """Entries (i, j) with some flagged (k, l), k <= i and l <= j."""
    m, n = mask.shape
    first = np.where(mask.any(axis=1), mask.argmax(axis=1), n)
    reach = np.minimum.accumulate(first)
    return int(np.sum(n - reach))


def run(name: str) -> dict:
    t0 = time.perf_counter()
    wl = make(name)
    W, A, B, s = wl.cast("f32")
    t1 = time.perf_counter()
    W64, A64, B64, s64 = (np.asarray(x, dtype=np.float64) for x in (W, A, B, s))
    Ua = oracle.factor_unit_upper(A64)
    Ub = oracle.factor_unit_upper(B64)
    t2 = time.perf_counter()
    out = oracle.sweep(W64, Ua, Ub, s64, wl.bits, return_delta=True)
    t3 = time.perf_counter()
    Z = out["Z"].astype(np.int8)
    lo, hi = wl.lo, wl.hi
    T = (out["Q"] + out["Delta"]) / s64[:, None]
    live = (T > lo - 0.5) & (T < hi + 0.5)
    frac = np.where(live, np.abs(T - np.floor(T) - 0.5), 0.5)
    del T
    margins = {}
    for thr in THRESHOLDS:
        mask = frac < thr
        cnt = int(np.count_nonzero(mask))
        entry = None
        if cnt:
            flat = int(np.argmax(mask.reshape(-1)))
            entry = [flat // wl.n, flat % wl.n]
        margins[f"{thr:g}"] = {"count": cnt, "first_row_major": entry,
                               "cone_entries": cone_size(mask) if cnt else 0}
    obj = oracle.objective(W64, out["Q"], A64, B64)
    zr = oracle.rtn(W64, s64, wl.bits)
    obj_rtn = oracle.objective(W64, s64[:, None] * zr, A64, B64)
    rec = {
        "shape": [wl.m, wl.n], "bits": wl.bits, "recipe": wl.recipe,
        "input_sha256": {"W": sha(W), "A": sha(A), "B": sha(B), "scales": sha(s)},
        "codes_sha256": sha(Z),
        "block_rows": BLOCK_ROWS,
        "codes_block_sha256": [sha(Z[r:r + BLOCK_ROWS]) for r in range(0, wl.m, BLOCK_ROWS)],
        "objective": obj, "objective_rtn": obj_rtn,
        "min_margin": float(np.min(frac)),
        "margins": margins,
        "oracle_threads": out["threads"],
        "oracle_seconds": {"generate": t1 - t0, "factor": t2 - t1, "sweep": t3 - t2},
    }
    print(f"{name}: factor {t2 - t1:.1f} s, sweep {t3 - t2:.1f} s, min margin "
          f"{rec['min_margin']:.3g}", flush=True)
    return rec


def main():
    names = sys.argv[1:] or list(NAMES)
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for name in names:
        data[name] = run(name)
        with open(OUT + ".tmp", "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
        os.replace(OUT + ".tmp", OUT)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
