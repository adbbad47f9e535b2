"""Input generators: deterministic, well-formed, and shaped as documented."""
import numpy as np
import pytest

from synthetic import make, make_random
from synthetic.configs import SHAPES


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_small_configs_are_deterministic_and_well_formed(name):
    a, b = make(name), make(name)
    assert np.array_equal(a.W, b.W) and np.array_equal(a.A, b.A) and np.array_equal(a.B, b.B)
    m, n, bits = SHAPES[name]
    assert a.W.shape == (m, n) and a.A.shape == (m, m) and a.B.shape == (n, n)
    assert a.bits == bits
    assert np.array_equal(a.A, a.A.T) and np.array_equal(a.B, a.B.T)
    assert np.min(np.linalg.eigvalsh(a.A)) > 0 and np.min(np.linalg.eigvalsh(a.B)) > 0
    assert np.all(a.scales > 0)
    # the largest entry of every row sits exactly on the grid's top level
    np.testing.assert_allclose(np.max(np.abs(a.W), axis=1) / a.scales, a.hi, rtol=1e-6)
    if a.dtype == "f32":
        for x in (a.W, a.A, a.B, a.scales):
            assert np.array_equal(x.astype(np.float32).astype(np.float64), x)


def test_c2_outlier_columns():
    wl = make("C2")
    col_rms = np.sqrt(np.mean(wl.W ** 2, axis=0))
    assert np.sum(col_rms > 0.1) == 3


def test_random_kinds():
    wl = make_random(6, 7, 3, seed=1, kind="identity_a")
    assert np.array_equal(wl.A, np.eye(6))
    wl = make_random(6, 7, 3, seed=1, kind="diagonal")
    assert np.count_nonzero(wl.A - np.diag(np.diag(wl.A))) == 0
    wl = make_random(6, 7, 3, seed=1, global_scale=True)
    assert np.all(wl.scales == wl.scales[0])
