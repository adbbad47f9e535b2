"""Full-size parity for the benchmarked layer shapes.

At these sizes the whole oracle sweep takes minutes, so each case checks, on the GPU
result produced in the same configuration bench.py times:
  * the certificate on EVERY entry: Delta* = U'a^-T (W - Q) U'b^-1 from the oracle's
    float64 factors must reproduce the codes (Z = clamp(rint((Q + Delta*)/s))), which
    characterises the GPTQ-2D output uniquely in exact arithmetic;
  * exact sub-problems computed by the oracle one by one: the first rows (they depend
    only on rows above) and the first columns (they depend only on columns left).
fp64 mode must be bit-exact on the sampled rows/columns and certificate-clean; fp32 mode
must agree on >= 99.99 % of sampled codes and flag <= 0.01 % of entries.
"""
import os

import numpy as np
import pytest

import oracle
from synthetic import make

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

CACHE = os.environ.get("GPTQ2D_CACHE")
SAMPLE = 192


@pytest.fixture(scope="module")
def g2d():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import two_sided_adaptive_amd as m
    m.load_library()
    return m


def _check_large(g2d, name, dtype):
    wl = make(name, cache_dir=CACHE)
    W, A, B, s = wl.cast(dtype)
    print(f"case {name} {dtype} {wl.m}x{wl.n} bits={wl.bits}", flush=True)
    t = [torch.from_numpy(x).to("cuda:0") for x in (W, A, B, s)]
    codes, Q = g2d.quantize(t[0], t[1], t[2], wl.bits, t[3])
    torch.cuda.synchronize()
    z = codes.cpu().numpy().astype(np.int32)
    q_run = Q.cpu().numpy()
    # Q is the scale times the code, rounded once in the run dtype
    np.testing.assert_array_equal(q_run, s[:, None] * z.astype(s.dtype))
    q = q_run.astype(np.float64)
    W64, A64, B64, s64 = (x.astype(np.float64) for x in (W, A, B, s))
    Ua, Ub = oracle.factor_unit_upper(A64), oracle.factor_unit_upper(B64)
    cert = oracle.certificate(W64, q, Ua, Ub, s64, wl.bits)
    print(f"  certificate {cert}", flush=True)
    top = oracle.sweep(W64[:SAMPLE], Ua[:SAMPLE, :SAMPLE], Ub, s64[:SAMPLE], wl.bits)["Z"]
    left = oracle.sweep(W64[:, :SAMPLE], Ua, Ub[:SAMPLE, :SAMPLE], s64, wl.bits)["Z"]
    a_top = float(np.mean(top == z[:SAMPLE]))
    a_left = float(np.mean(left == z[:, :SAMPLE]))
    print(f"  sampled agreement rows {a_top:.6f} cols {a_left:.6f}", flush=True)
    if dtype == "f64":
        assert cert["mismatch"] == 0
        assert np.array_equal(top, z[:SAMPLE]) and np.array_equal(left, z[:, :SAMPLE])
    else:
        assert cert["mismatch"] <= 1e-4 * z.size
        assert a_top >= 0.9999 and a_left >= 0.9999


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_c3_full_size(g2d, dtype):
    _check_large(g2d, "C3", dtype)
