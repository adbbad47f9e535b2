// Opt-in measurement hook: brackets library kernel launches with HIP events on the
// launch stream and accounts them to kernel classes together with the algorithmic
// flops and HBM bytes of each launch.  Off by default; when off every call below is
// a branch on one flag.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g2d {

enum KernelClass : int {
  KC_SWEEP = 0,      // the persistent sweep kernel: rounding, band updates, outputs
  KC_BAND_GEMM = 1,  // band-update tasks inside the sweep (busy time of the workgroups
                     // that ran them, in CU-milliseconds; one "launch" per task)
  KC_FACTOR = 2,     // the persistent Cholesky + inverse kernel of the factor stage
  KC_OTHER = 3,      // setup, init and check kernels
  KC_SLAB = 4,       // mode-1 feedback between the slabs of a three-factor tensor
  KC_PACK = 5,       // packing of codes, unpacking to Q, and the packed-code GEMV
  KC_GRAM = 6,       // Kronecker factor accumulation A += alpha X^T X (and its mirror pass)
  KC_COUNT = 7
};

bool prof_on();
void prof_begin(int cls, hipStream_t s);
void prof_end(int cls, hipStream_t s, double flops, double bytes);

// Device counters of the band-update tasks, accumulated by the sweep kernel while the
// hook is on (nullptr otherwise), per task class c (near, next, far):
// [3c] busy wall-clock ticks (100 MHz) summed over tasks, [3c + 1] task flops, [3c + 2] tasks.
constexpr int kTaskClasses = 3;
unsigned long long* band_stats_device();
// Reads the counters of each task class (arrays of kTaskClasses) and clears them
// (synchronous).
hipError_t band_stats_collect(double* cu_ms, double* flops, int64_t* tasks);

}  // namespace g2d
