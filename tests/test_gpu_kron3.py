"""Parity of the three-factor path (gptq2d_quantize3, through the C ABI) with the CPU
oracle: bit-identical codes and Q in fp64, agreement and objective in fp32."""
import numpy as np
import pytest

import oracle
from synthetic import make3, make_random3

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def g2d():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_sided_adaptive_amd as m
    m.load_library()
    oracle.build_library(force=False)
    return m


def _run(g2d, wl, dtype="f64"):
    np_dt = np.float32 if dtype == "f32" else np.float64
    xs = [np.ascontiguousarray(x, dtype=np_dt) for x in (wl.W, wl.A1, wl.A2, wl.A3, wl.scales)]
    print(f"case {wl.name} {dtype} shape={wl.W.shape} bits={wl.bits}", flush=True)
    t = [torch.from_numpy(x).to(DEV) for x in xs]
    codes, Q = g2d.quantize3(t[0], t[1], t[2], t[3], wl.bits, t[4])
    torch.cuda.synchronize()
    return xs, codes.cpu().numpy().astype(np.int32), Q.cpu().numpy()


def test_k1_fp64_exact(g2d):
    wl = make3("K1")
    xs, z, Q = _run(g2d, wl)
    ref = oracle.quantize3(*xs, wl.bits)
    assert np.array_equal(z, ref["Z"]), f"{int(np.sum(z != ref['Z']))} mismatches"
    np.testing.assert_array_equal(Q, ref["Q"])


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 65, 63), (5, 1, 70), (20, 70, 1),
                                   (17, 33, 40), (37, 20, 24), (3, 130, 66),
                                   (37, 640, 24), (32, 1024, 40)])
def test_ragged_shapes_fp64_exact(g2d, shape):
    # Up to m1 m2 = 23170 rows (fp64) the call sweeps the stacked (m1 m2) x m3 matrix under
    # U1' (x) U2'; the last two shapes are above that and take the slab-by-slab route, where
    # m1 = 37 leaves a ragged block of the lazy slab feedback (16 slabs a block).
    bits = 2 + sum(shape) % 7
    wl = make_random3(*shape, bits, seed=shape[0] * 10007 + shape[1] * 101 + shape[2])
    xs, z, Q = _run(g2d, wl)
    ref = oracle.quantize3(*xs, bits)
    assert np.array_equal(z, ref["Z"]), f"{int(np.sum(z != ref['Z']))} mismatches"
    np.testing.assert_array_equal(Q, ref["Q"])


def test_k1_fp32_agreement_and_objective(g2d):
    wl = make3("K1")
    xs, z, Q = _run(g2d, wl, "f32")
    x64 = [np.asarray(x, dtype=np.float64) for x in xs]
    ref = oracle.quantize3(*x64, wl.bits)
    agree = float(np.mean(z == ref["Z"]))
    assert agree >= 0.999, agree
    f = lambda X: oracle.objective3(x64[0], X, *x64[1:4])  # noqa: E731
    assert abs(f(Q.astype(np.float64)) - f(ref["Q"])) <= 1e-3 * f(ref["Q"])


@pytest.mark.parametrize("which,code", [(1, 5), (3, 7)])
def test_non_spd_factor_reported(g2d, which, code):
    wl = make_random3(6, 20, 24, 4, seed=3)
    mats = [wl.A1, wl.A2, wl.A3]
    bad = mats[which - 1].copy()
    bad[2, 2] = -1.0
    mats[which - 1] = bad
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (wl.W, *mats, wl.scales)]
    with pytest.raises(g2d.GPTQ2DError, match=f"A{which} is not positive definite"):
        g2d.quantize3(t[0], t[1], t[2], t[3], wl.bits, t[4])
    torch.cuda.synchronize()
    del code


def test_k2_full_size_fp64_exact(g2d):
    # the measured tensor: 16 slabs of 1024 x 1024, the oracle takes some seconds per slab
    wl = make3("K2")
    xs, z, Q = _run(g2d, wl)
    ref = oracle.quantize3(*xs, wl.bits)
    assert np.array_equal(z, ref["Z"]), f"{int(np.sum(z != ref['Z']))} mismatches"
    np.testing.assert_array_equal(Q, ref["Q"])


@pytest.mark.parametrize("shape", [(6, 130, 40), (37, 640, 24)])
def test_workspace_contents_do_not_matter(g2d, shape):
    # a caller's workspace may hold anything, NaN included (the stacked route leaves the
    # tiles of U1' (x) U2' below its diagonal unwritten; the slab route keeps its slab
    # buffer there): the codes must still equal the oracle's
    bits = 4
    wl = make_random3(*shape, bits, seed=sum(shape))
    xs = [np.ascontiguousarray(x, dtype=np.float64) for x in (wl.W, wl.A1, wl.A2, wl.A3,
                                                                wl.scales)]
    t = [torch.from_numpy(x).to(DEV) for x in xs]
    ref = oracle.quantize3(*xs, bits)["Z"]
    need = g2d.load_library().gptq2d_workspace3_bytes(*shape, 1)
    for fill in (float("nan"), float("inf")):
        print(f"case workspace fill {fill} shape={shape}", flush=True)
        ws = torch.full((need // 8 + 1,), fill, dtype=torch.float64, device=DEV)
        codes, _ = g2d.quantize3(t[0], t[1], t[2], t[3], bits, t[4],
                                 workspace=ws.view(torch.uint8)[:need])
        z = codes.cpu().numpy().astype(np.int32)
        assert np.array_equal(z, ref), f"fill {fill}: {int(np.sum(z != ref))} mismatches"


@pytest.mark.parametrize("shape", [(6, 130, 40), (37, 640, 24)])
def test_bad_scale_reported_by_fibre(g2d, shape):
    # both routes name the fibre W[k][i][:] by k m2 + i + 1
    wl = make_random3(*shape, 4, seed=5)
    sc = wl.scales.copy()
    sc[2, 5] = 0.0
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
         for x in (wl.W, wl.A1, wl.A2, wl.A3, sc)]
    print(f"case bad scale shape={shape}", flush=True)
    with pytest.raises(g2d.GPTQ2DError, match=f"scale of row {2 * shape[1] + 6} "):
        g2d.quantize3(t[0], t[1], t[2], t[3], 4, t[4])
    torch.cuda.synchronize()
