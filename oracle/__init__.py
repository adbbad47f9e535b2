"""CPU float64 oracle for GPTQ-2D two-sided adaptive rounding.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, build or call anything in this
package.  The GPU library never touches it, and the two share no code: the
oracle factors with LAPACK along GPTQ's inverse-then-Cholesky route and sweeps in
plain C (``nested_sweep.c``); the GPU library has its own kernels.

Parity status of each function (what pins it, see tests/test_oracle_pins.py):
  factor_unit_upper      pinned: reconstruction of A^-1, route independence
  sweep / quantize       pinned: brute-force Babai nearest plane, quartic
                         vectorised GPTQ, one-sided GPTQ (A=I, B=I), RTN (diagonal
                         A and B), certificate, transpose and scaling invariances
  gptq_1d                pinned: against Babai for m=1, against RTN for B=I
  babai_nearest_plane    pinned: exhaustive closest-vector search on tiny
                         lattices (bits=16, no clamp: Babai's error bound)
  certificate            pinned: detects planted code flips
  objective              pinned: explicit Kronecker quadratic form
  quantize3 (three       pinned: quartic vectorised GPTQ with the explicit
    Kronecker factors)   three-factor Gram, reduction to the two-factor sweep
                         (m3 = 1 and m1 = 1), independent slabs (A1 = I),
                         three-mode certificate, mode-permutation symmetry
  objective3             pinned: explicit Kronecker quadratic form
  packing.pack_rows /    pinned: hand-worked 3-bit row (tests/golden), byte and
    unpack_rows          nibble views for 8 and 4 bits, round trip, zero padding
  packing.dequantize /   pinned: equals the quantizer's Q; explicit dot products
    packed_gemv
  gram.gram_accumulate   pinned: sum of outer products, exact integer case,
                         symmetry and positive semi-definiteness
"""
from .gptq2d import (  # noqa: F401
    babai_nearest_plane,
    build_library,
    certificate,
    factor_unit_upper,
    gptq_1d,
    gptq_1d_coords,
    gptq_vectorized,
    objective,
    quantize,
    rtn,
    sweep,
)
from .kron3 import (  # noqa: F401
    certificate3,
    gptq_vectorized3,
    objective3,
    quantize3,
    quantize3_factored,
)
from . import packing  # noqa: F401,E402
from . import gram  # noqa: F401,E402
