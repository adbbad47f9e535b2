// Opt-in measurement hook: brackets library kernel launches with HIP events on the
// launch stream and accounts them to kernel classes together with the algorithmic
// flops and HBM bytes of each launch.  Off by default; when off every call below is
// a branch on one flag.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g2d {

enum KernelClass : int {
  KC_ROUND = 0,     // anti-diagonal rounding of one block diagonal
  KC_BAND = 1,      // near band feedback GEMMs of one block diagonal
  KC_POTRF = 2,     // one Cholesky step: diagonal block + inverse, panel, trailing
  KC_PANEL = 3,     // panel solve GEMM
  KC_TRAILING = 4,  // trailing-update GEMM of the Cholesky
  KC_TRTRI = 5,     // triangular-inverse doubling GEMMs
  KC_OTHER = 6,     // reverse/finalize/init/check kernels
  KC_FAR = 7,       // far band feedback GEMMs (second stream)
  KC_COUNT = 8
};

bool prof_on();
void prof_begin(int cls, hipStream_t s);
void prof_end(int cls, hipStream_t s, double flops, double bytes);

}  // namespace g2d
