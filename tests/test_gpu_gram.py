"""Kronecker factor accumulation on the GPU (gptq2d_gram_accumulate through the C ABI)
against the oracle: bit-exact where every product and partial sum is an integer the dtype
holds exactly (any summation order then gives the same result), and within the dot-product
rounding bound otherwise."""
import numpy as np
import pytest

from oracle import gram

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda:0"


@pytest.fixture(scope="module")
def g2d():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_sided_adaptive_amd as m
    m.load_library()
    return m


def _sym_int(rng, p):
    a = rng.integers(-50, 51, size=(p, p)).astype(np.float64)
    return np.tril(a) + np.tril(a, -1).T


@pytest.mark.parametrize("shape", [(1, 1), (5, 3), (64, 64), (65, 130), (200, 333),
                                   (130, 4100)])
@pytest.mark.parametrize("dt", [torch.float64, torch.float32])
def test_integer_samples_exact(g2d, shape, dt):
    p, N = shape
    print(f"case gram int p={p} N={N} {dt}", flush=True)
    rng = np.random.default_rng(p * 7 + N)
    X = rng.integers(-8, 9, size=(N, p)).astype(np.float64)
    A0 = _sym_int(rng, p)
    A = torch.from_numpy(A0).to(DEV, dt)
    g2d.gram_accumulate(A, torch.from_numpy(X).to(DEV, dt), 2.0)
    torch.cuda.synchronize()
    want = gram.gram_accumulate(A0, X, 2.0)
    assert np.array_equal(A.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("dt", [torch.float64, torch.float32])
def test_random_samples_within_rounding_bound(g2d, dt):
    p, N = 300, 1000
    rng = np.random.default_rng(5)
    np_dt = np.float32 if dt == torch.float32 else np.float64
    X = rng.standard_normal((N, p)).astype(np_dt).astype(np.float64)
    A0 = np.eye(p)
    A = torch.from_numpy(A0).to(DEV, dt)
    g2d.gram_accumulate(A, torch.from_numpy(X).to(DEV, dt), 1.0 / N)
    got = A.cpu().numpy().astype(np.float64)
    want = gram.gram_accumulate(A0, X, 1.0 / N)
    u = 2.0 ** -24 if dt == torch.float32 else 2.0 ** -53
    k = N + 3  # N products and sums, the scaling by alpha and the final addition
    bound = k * u / (1 - k * u) * (np.abs(A0) + (np.abs(X).T @ np.abs(X)) / N)
    assert np.all(np.abs(got - want) <= bound)
    assert np.array_equal(got, got.T)


def test_batched_layers(g2d):
    rng = np.random.default_rng(6)
    shapes = [(96, 40), (33, 7), (128, 256)]
    Xs = [rng.integers(-4, 5, size=(N, p)).astype(np.float64) for p, N in shapes]
    A0s = [_sym_int(rng, p) for p, _ in shapes]
    As = [torch.from_numpy(a).to(DEV) for a in A0s]
    g2d.gram_accumulate_batched(As, [torch.from_numpy(x).to(DEV) for x in Xs], [1.0, 0.5, 3.0])
    torch.cuda.synchronize()
    for A, A0, X, al in zip(As, A0s, Xs, [1.0, 0.5, 3.0]):
        assert np.array_equal(A.cpu().numpy(), gram.gram_accumulate(A0, X, al))


def test_full_size_sampled_entries(g2d):
    # the 4096-wide factor from 8192 samples, the size the measured layer's metrics have
    p, N = 4096, 8192
    gen = torch.Generator(device=DEV).manual_seed(7)
    X = torch.randn((N, p), dtype=torch.float64, device=DEV, generator=gen)
    A = torch.zeros((p, p), dtype=torch.float64, device=DEV)
    g2d.gram_accumulate(A, X, 1.0 / N)
    Xc, Ac = X.cpu().numpy(), A.cpu().numpy()
    assert np.array_equal(Ac, Ac.T)
    rng = np.random.default_rng(8)
    idx = [(int(i), int(j)) for i, j in rng.integers(0, p, size=(40, 2))] + [(0, 0), (p - 1, p - 1),
                                                                             (p - 1, 0), (63, 64)]
    u = 2.0 ** -53
    for i, j in idx:
        want = gram.gram_entry(Xc, i, j) / N
        bound = (N + 3) * u * float(np.abs(Xc[:, i]) @ np.abs(Xc[:, j])) / N * 1.01
        assert abs(Ac[i, j] - want) <= bound, (i, j)
