"""Packed codes on the GPU (gptq2d_pack / gptq2d_unpack / gptq2d_packed_gemv through the C
ABI) against the oracle: packed words and Q bit-exact, the GEMV within the dot-product
rounding bound of its dtype."""
import numpy as np
import pytest

from oracle import packing

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


def _codes(rows, n, bits, seed):
    rng = np.random.default_rng(seed)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    z = rng.integers(lo, hi + 1, size=(rows, n))
    z[0, 0], z[-1, -1] = lo, hi          # both ends of the range
    return z.astype(np.int8)


SHAPES = [(1, 1), (3, 31), (5, 33), (7, 100), (65, 1000), (130, 4099), (9, 4096)]


@pytest.mark.parametrize("bits", range(2, 9))
@pytest.mark.parametrize("shape", SHAPES)
def test_pack_and_unpack_exact(g2d, bits, shape):
    rows, n = shape
    print(f"case pack bits={bits} shape={shape}", flush=True)
    z = _codes(rows, n, bits, seed=bits * 1000 + rows + n)
    P = g2d.pack(torch.from_numpy(z).to(DEV), bits)
    torch.cuda.synchronize()
    ref = packing.pack_rows(z, bits)
    assert np.array_equal(P.cpu().numpy().view(np.uint32), ref)
    s = np.random.default_rng(bits).uniform(0.001, 0.01, rows)
    for dt in (torch.float64, torch.float32):
        Q = g2d.unpack(P, n, bits, torch.from_numpy(s).to(DEV, dt)).cpu().numpy()
        s_in = s.astype(np.float32).astype(np.float64) if dt == torch.float32 else s
        want = s_in[:, None] * z.astype(np.float64)   # exact in float64
        if dt == torch.float32:
            want = want.astype(np.float32)             # one rounding, as the kernel's product
        assert np.array_equal(Q, want)


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("batch", [1, 3, 8])
@pytest.mark.parametrize("dt", [torch.float64, torch.float32])
@pytest.mark.parametrize("n", [2053, 2048])
def test_packed_gemv_within_rounding_bound(g2d, bits, batch, dt, n):
    rows = 257
    print(f"case gemv bits={bits} batch={batch} {dt}", flush=True)
    z = _codes(rows, n, bits, seed=bits + 10 * batch)
    rng = np.random.default_rng(batch)
    s = rng.uniform(0.001, 0.01, rows)
    X = rng.standard_normal((batch, n))
    np_dt = np.float32 if dt == torch.float32 else np.float64
    s, X = s.astype(np_dt).astype(np.float64), X.astype(np_dt).astype(np.float64)
    P = g2d.pack(torch.from_numpy(z).to(DEV), bits)
    Y = g2d.packed_gemv(P, n, bits, torch.from_numpy(s).to(DEV, dt),
                        torch.from_numpy(X).to(DEV, dt)).cpu().numpy().astype(np.float64)
    ref = packing.packed_gemv(packing.pack_rows(z, bits), n, bits, s, X)
    # |error| <= gamma_(n+1) * s * sum |z x| with gamma_k = k u / (1 - k u), u the unit roundoff
    u = 2.0 ** -24 if dt == torch.float32 else 2.0 ** -53
    k = n + 2
    bound = k * u / (1 - k * u) * (np.abs(X) @ np.abs(z.astype(np.float64)).T) * s[None, :]
    assert np.all(np.abs(Y - ref) <= bound + 1e-300)


def test_full_size_pack_of_quantizer_codes(g2d):
    # the 4096 x 4096 4-bit layer's shape, with codes from the quantizer on a seeded layer
    from synthetic import make
    wl = make("C3")
    W, A, B, s = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
                  for x in (wl.W, wl.A, wl.B, wl.scales))
    codes, Q = g2d.quantize(W, A, B, 4, s)
    P = g2d.pack(codes, 4)
    Q2 = g2d.unpack(P, 4096, 4, s)
    torch.cuda.synchronize()
    assert torch.equal(Q, Q2)
    z = codes.cpu().numpy()
    rows = np.array([0, 1, 777, 2048, 4095])
    Pc = P.cpu().numpy().view(np.uint32)
    assert np.array_equal(Pc[rows], packing.pack_rows(z[rows], 4))
