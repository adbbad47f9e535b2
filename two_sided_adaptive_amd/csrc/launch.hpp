// Internal host-side interface between the C ABI (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace g2d {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Library-owned per-device resources: a second stream (default priority) and a pool
// of timing-disabled events.  Callers must hold lib_mutex() from the first use of
// the events until the last wait that names them has been enqueued.
std::recursive_mutex& lib_mutex();
hipError_t aux_resources(size_t nevents, hipStream_t* aux, hipEvent_t** events);
// events of the pool: 0, 1 join the caller's stream and the second stream around the
// factors (api.hip), 2, 3 order the factor stage's launches across the two streams
constexpr size_t kAuxEvents = 4;

// Factor stage (factor.hip): U' (dtype) of one SPD matrix A (dtype), fp64 inside.
size_t factor_workspace(int64_t p);
hipError_t factor_enqueue(int64_t p, int dtype, const void* A, void* U, void* ws, int* info,
                          int side_code, hipStream_t s);
// Both factors at once: A (m x m) on stream sa and B (n x n) on stream sb, with their
// launches interleaved on the host; info codes 1 for A and 2 for B.
hipError_t factor_pair_enqueue(int64_t m, const void* A, void* Ua, void* ws_a, hipStream_t sa,
                               int64_t n, const void* B, void* Ub, void* ws_b, hipStream_t sb,
                               int dtype, int* info);

// Sweep stage (sweep.hip): codes/Q from W, U'_a, U'_b, scales (all dtype).
size_t sweep_workspace(int64_t m, int64_t n, int dtype);
hipError_t sweep_enqueue(int64_t m, int64_t n, int bits, int dtype, const void* W,
                         const void* Ua, const void* Ub, const void* scales, int8_t* codes,
                         void* Q, void* ws, int* info, hipStream_t s);

}  // namespace g2d
