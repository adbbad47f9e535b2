"""Parity of the HIP path (through the C ABI) with the CPU oracle.

fp64 mode: codes must be bit-identical to the oracle.  fp32 mode: >= 99.99 % of codes
agree and tr(A E B E^T) is within 1e-3 relative of the oracle's.
"""
import numpy as np
import pytest

import oracle
from synthetic import make, make_random

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def g2d():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_sided_adaptive_amd as m
    m.load_library()
    return m


DEV = "cuda:0"


def _dev(*xs):
    return [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in xs]


def _run(g2d, wl, dtype):
    W, A, B, s = wl.cast(dtype)
    print(f"case {wl.name} {dtype} m={wl.m} n={wl.n} bits={wl.bits}", flush=True)
    tW, tA, tB, ts = _dev(W, A, B, s)
    codes, Q = g2d.quantize(tW, tA, tB, wl.bits, ts)
    torch.cuda.synchronize()
    return (W, A, B, s), codes.cpu().numpy().astype(np.int32), Q.cpu().numpy()


def test_c1_fp64_matches_golden_and_oracle(g2d):
    import os
    wl = make("C1")
    _, z, Q = _run(g2d, wl, "f64")
    gold = np.loadtxt(os.path.join(os.path.dirname(__file__), "golden", "c1_codes.txt"),
                      dtype=np.int64, comments="#")
    assert np.array_equal(z, gold)
    np.testing.assert_array_equal(Q, wl.scales[:, None] * z)


@pytest.mark.parametrize("shape", [(1, 1), (1, 70), (70, 1), (65, 63), (63, 65), (130, 200),
                                   (200, 130), (257, 129), (64, 64), (128, 320)])
def test_odd_shapes_fp64_exact(g2d, shape):
    m, n = shape
    bits = 2 + (m * 7 + n) % 7
    wl = make_random(m, n, bits, seed=m * 1000 + n)
    (W, A, B, s), z, Q = _run(g2d, wl, "f64")
    ref = oracle.quantize(W, A, B, s, bits)
    assert np.array_equal(z, ref["Z"]), f"{int(np.sum(z != ref['Z']))} mismatches"
    np.testing.assert_array_equal(Q, ref["Q"])


@pytest.mark.parametrize("p", [1, 5, 64, 65, 200, 512, 1100])
def test_factor_matches_oracle(g2d, p):
    wl = make_random(p, 2, 4, seed=p)
    for dtype, tol in (("f64", 1e-10), ("f32", 1e-5)):
        A = wl.cast(dtype)[1]
        U = g2d.factor(_dev(A)[0]).cpu().numpy().astype(np.float64)
        ref = oracle.factor_unit_upper(A)
        err = np.max(np.abs(U - ref)) / max(1.0, np.max(np.abs(ref)))
        assert err < tol, (dtype, err)
        assert np.all(np.tril(U, -1) == 0)


def test_pair_with_long_inverse_rows_fp64_exact(g2d):
    # 10 and 17 row tiles of 64: the factors' inverse rows take up to three chunks, and the
    # two matrices' task groups interleave with different lengths
    m, n = 600, 1030
    wl = make_random(m, n, 3, seed=606)
    (W, A, B, s), z, Q = _run(g2d, wl, "f64")
    ref = oracle.quantize(W, A, B, s, 3)
    assert np.array_equal(z, ref["Z"]), f"{int(np.sum(z != ref['Z']))} mismatches"
    np.testing.assert_array_equal(Q, ref["Q"])


def test_c2_fp64_exact(g2d):
    wl = make("C2")
    (W, A, B, s), z, Q = _run(g2d, wl, "f64")
    ref = oracle.quantize(W, A, B, s, wl.bits)
    assert np.array_equal(z, ref["Z"]), f"{int(np.sum(z != ref['Z']))} mismatches"


def test_c2_fp32_agreement_and_objective(g2d):
    wl = make("C2")
    (W, A, B, s), z, Q = _run(g2d, wl, "f32")
    ref = oracle.quantize(W, A, B, s, wl.bits)
    agree = float(np.mean(z == ref["Z"]))
    print(f"C2 fp32 agreement {agree:.6f}", flush=True)
    assert agree >= 0.9999
    f_gpu = oracle.objective(W, Q.astype(np.float64), A, B)
    f_ref = oracle.objective(W, ref["Q"], A, B)
    assert abs(f_gpu - f_ref) <= 1e-3 * abs(f_ref)


def test_quantize_factored_with_oracle_factors(g2d):
    wl = make_random(150, 170, 4, seed=77)
    W, A, B, s = wl.cast("f64")
    Ua, Ub = oracle.factor_unit_upper(A), oracle.factor_unit_upper(B)
    tW, tUa, tUb, ts = _dev(W, Ua, Ub, s)
    codes, Q = g2d.quantize_factored(tW, tUa, tUb, 4, ts)
    ref = oracle.sweep(W, Ua, Ub, s, 4)
    assert np.array_equal(codes.cpu().numpy().astype(np.int32), ref["Z"])


def test_repeat_is_bitwise_deterministic(g2d):
    wl = make_random(300, 260, 4, seed=3)
    for dtype in ("f32", "f64"):
        _, z1, q1 = _run(g2d, wl, dtype)
        _, z2, q2 = _run(g2d, wl, dtype)
        assert np.array_equal(z1, z2) and np.array_equal(q1, q2)


@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_scheduling_knobs_do_not_change_results(g2d, dtype, monkeypatch):
    # The sweep's run-time plan (band workers per XCD and consecutive bands per XCD, the
    # share of update workgroups taking near tasks) decides which workgroup does what and
    # when, never the order of any sum: codes and Q are bitwise those of the default plan.
    wl = make_random(700, 650, 4, seed=21)
    _, z0, q0 = _run(g2d, wl, dtype)
    if dtype == "f64":
        W, A, B, s = wl.cast(dtype)
        assert np.array_equal(z0, oracle.quantize(W, A, B, s, 4)["Z"])
    for bands, near in (("1,1", None), ("2,4", None), ("3,2", "1"), (None, "3"),
                        (None, "1000"), ("6,1", "14")):
        for var, val in (("GPTQ2D_SWEEP_BANDS", bands), ("GPTQ2D_SWEEP_NEAR", near)):
            if val is None:
                monkeypatch.delenv(var, raising=False)
            else:
                monkeypatch.setenv(var, val)
        print(f"case plan bands={bands} near={near} {dtype}", flush=True)
        _, z, q = _run(g2d, wl, dtype)
        assert np.array_equal(z, z0), f"bands={bands} near={near}: codes differ"
        assert np.array_equal(q.view(np.uint8), q0.view(np.uint8)), f"bands={bands} near={near}: Q"


def test_numerical_failures_reported(g2d):
    wl = make_random(40, 30, 4, seed=4)
    W, A, B, s = wl.cast("f64")
    bad = A.copy()
    bad[7, 7] = -1.0
    with pytest.raises(g2d.GPTQ2DError, match="A is not positive definite"):
        g2d.quantize(*_dev(W, bad, B), 4, _dev(s)[0])
    badb = B.copy()
    badb[3, 3] = -5.0
    with pytest.raises(g2d.GPTQ2DError, match="B is not positive definite"):
        g2d.quantize(*_dev(W, A, badb), 4, _dev(s)[0])
    s2 = s.copy()
    s2[11] = 0.0
    with pytest.raises(g2d.GPTQ2DError, match="scale of row 12"):
        g2d.quantize(*_dev(W, A, B), 4, _dev(s2)[0])
    # the library still works afterwards
    (W, A, B, s), z, _ = _run(g2d, wl, "f64")
    assert np.array_equal(z, oracle.quantize(W, A, B, s, 4)["Z"])


@pytest.mark.parametrize("shape", [(130, 200), (200, 130), (257, 129), (65, 63)])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_workspace_contents_do_not_matter(g2d, shape, dtype):
    # a caller's workspace may hold anything, NaN included: the codes must not depend on it
    # (fp64: equal to the oracle; fp32: bitwise equal to a run on a zeroed workspace)
    m, n = shape
    bits = 2 + (m * 7 + n) % 7
    wl = make_random(m, n, bits, seed=m * 1000 + n, dtype=dtype)
    W, A, B, s = wl.cast(dtype)
    tW, tA, tB, ts = _dev(W, A, B, s)
    tdt = torch.float64 if dtype == "f64" else torch.float32
    need = g2d.workspace_bytes(m, n, tdt)
    if dtype == "f64":
        ref = oracle.quantize(W, A, B, s, bits)["Z"]
    else:
        ws0 = torch.zeros((need,), dtype=torch.uint8, device=DEV)
        ref = g2d.quantize(tW, tA, tB, bits, ts, workspace=ws0)[0].cpu().numpy().astype(np.int32)
    for fill in (float("nan"), float("inf"), 0.0):
        print(f"case workspace fill {fill} {dtype} m={m} n={n}", flush=True)
        ws = torch.full((need // 8 + 1,), fill, dtype=torch.float64, device=DEV)
        codes, Q = g2d.quantize(tW, tA, tB, bits, ts, workspace=ws.view(torch.uint8)[:need])
        z = codes.cpu().numpy().astype(np.int32)
        assert np.array_equal(z, ref), f"fill {fill}: {int(np.sum(z != ref))} mismatches"
