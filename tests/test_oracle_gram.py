"""Pins of the Gram accumulation oracle (oracle/gram.py) by independent constructions."""
import numpy as np

from oracle import gram


def test_is_the_sum_of_outer_products():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((7, 5))
    A0 = rng.standard_normal((5, 5))
    A0 = A0 + A0.T
    want = A0.copy()
    for x in X:
        want += 0.25 * np.outer(x, x)
    np.testing.assert_allclose(gram.gram_accumulate(A0, X, 0.25), want, rtol=1e-13, atol=1e-13)
    assert np.isclose(gram.gram_entry(X, 1, 3), np.dot(X[:, 1], X[:, 3]))


def test_integer_samples_are_exact_and_blocks_add_up():
    rng = np.random.default_rng(2)
    X = rng.integers(-8, 9, size=(40, 6)).astype(np.float64)
    full = gram.gram_accumulate(np.zeros((6, 6)), X, 1.0)
    two = gram.gram_accumulate(gram.gram_accumulate(np.zeros((6, 6)), X[:17], 1.0), X[17:], 1.0)
    assert np.array_equal(full, two)
    ref = np.zeros((6, 6), dtype=np.int64)
    Xi = X.astype(np.int64)
    for i in range(6):
        for j in range(6):
            ref[i, j] = int(np.sum(Xi[:, i] * Xi[:, j]))
    assert np.array_equal(full, ref.astype(np.float64))


def test_symmetric_positive_semidefinite():
    X = np.random.default_rng(3).standard_normal((4, 9))   # rank 4 < 9
    G = gram.gram_accumulate(np.zeros((9, 9)), X, 1.0)
    assert np.array_equal(G, G.T)
    ev = np.linalg.eigvalsh(G)
    assert ev.min() > -1e-12 * ev.max()
    assert np.sum(ev > 1e-9 * ev.max()) == 4
