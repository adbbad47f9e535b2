// Three Kronecker factors ("GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding", arxivlens
// page, Abstract: the method extends to Hessians with any number of Kronecker factors).
//
// W is an m1 x m2 x m3 tensor under A1 (x) A2 (x) A3.  The unit feedback factor of the
// Kronecker Gram is U1' (x) U2' (x) U3', so the rounding splits into slabs W[k] (m2 x m3):
// slab k's target is W[k] - sum_{j<k} U1'[j,k] R1[j], where R1[j] = (slab j's target) -
// Q[j], and each target is then rounded as a two-factor problem (A2, A3) by the sweep
// kernel.  The mode-1 feedback is lazy in blocks of kSlabBlock slabs, as GPTQ's own
// blocking: a slab pulls the terms of the earlier slabs of its block just before its
// sweep, and a finished block pushes its terms to every later slab in one pass.
//
// When the stacked factor fits (the "tall" route below), the slabs are not swept one after
// another: with rows ordered (k, i) the tensor is an (m1 m2) x m3 matrix whose row Gram is
// A1 (x) A2, whose unit feedback factor is U1' (x) U2' (the Cholesky factor of a Kronecker
// product is the Kronecker product of the factors, and so are their unit scalings), and
// whose per-row scales are the per-fibre scales.  One two-factor sweep of that matrix
// follows the same trajectory (the order (k, i, l) is the row-major order of the tall
// matrix), with the slabs' band pipelines running together instead of one after another.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"
#include "prof.hpp"

namespace g2d {
namespace {

constexpr int kSlabBlock = 16;

// Wg[r] -= U1[j, r] * (Wg[j] - Q[j]) for every row r in [r0, r1) and j = j0 .. j1-1
// (j1 - j0 <= kSlabBlock, all j < r0), one thread per slab entry.  The terms are applied
// one by one in ascending j, each as a rounded product then a rounded subtraction (no
// fused multiply-add), so every entry sees exactly the sequence of operations of the
// plain one-axpy-per-slab definition whatever the blocking.
template <typename T>
__global__ __launch_bounds__(256) void k_slab_feedback(T* __restrict__ Wg,
                                                       const T* __restrict__ Q,
                                                       const T* __restrict__ U1, int64_t m1,
                                                       int64_t slab, int r0, int r1, int j0,
                                                       int j1) {
#pragma clang fp contract(off)
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= slab) return;
  const int nj = j1 - j0;
  T res[kSlabBlock];
#pragma unroll
  for (int t = 0; t < kSlabBlock; ++t)
    res[t] = t < nj ? Wg[(int64_t)(j0 + t) * slab + c] - Q[(int64_t)(j0 + t) * slab + c] : T(0);
  for (int r = r0 + (int)blockIdx.y; r < r1; r += (int)gridDim.y) {
    T g = Wg[(int64_t)r * slab + c];
#pragma unroll
    for (int t = 0; t < kSlabBlock; ++t) {
      if (t < nj) {
        const T prod = U1[(int64_t)(j0 + t) * m1 + r] * res[t];
        g = g - prod;
      }
    }
    Wg[(int64_t)r * slab + c] = g;
  }
}

template <typename T>
hipError_t slab_feedback(T* Wg, const T* Q, const T* U1, int64_t m1, int64_t slab, int r0,
                         int r1, int j0, int j1, hipStream_t s) {
  if (r1 <= r0 || j1 <= j0) return hipSuccess;
  if (j1 - j0 > kSlabBlock || j1 > r0) return hipErrorInvalidValue;
  const int64_t gx = cdiv(slab, 256);
  if (gx > 0x7FFFFFFF) return hipErrorInvalidValue;
  int64_t gy = cdiv(2048, gx);  // enough workgroups for small slabs
  if (gy > r1 - r0) gy = r1 - r0;
  if (gy > 65535) gy = 65535;
  const double es = (double)sizeof(T);
  prof_begin(KC_SLAB, s);
  k_slab_feedback<T><<<dim3((unsigned)gx, (unsigned)gy), 256, 0, s>>>(Wg, Q, U1, m1, slab, r0,
                                                                       r1, j0, j1);
  prof_end(KC_SLAB, s, 2.0 * (double)(j1 - j0) * (double)(r1 - r0) * (double)slab,
           es * (double)slab * (2.0 * (double)(j1 - j0) * (double)gy + 2.0 * (double)(r1 - r0)));
  return hipGetLastError();
}

// The stacked factor U1' (x) U2' is formed when it takes at most this many bytes.
constexpr int64_t kTallMaxBytes = (int64_t)4 << 30;
bool use_tall(int64_t m1, int64_t m2, int dtype) {
  const int64_t es = dtype == 0 ? 4 : 8, N = m1 * m2;
  return m1 > 1 && N <= 262140 && N * N <= kTallMaxBytes / es;
}

// Ut[x][y] = U1'[k][k'] U2'[i][i'] for x = k m2 + i, y = k' m2 + i' (zero below the
// diagonal because both factors are upper triangular with zero lower parts), one product
// per entry.  Only the 64 x 64 tiles on and above the diagonal are written: the sweep reads
// U'a tiles (rows of a band, columns of the same or a later band) and nothing else.
template <typename T>
__global__ __launch_bounds__(256) void k_kron_unit(const T* __restrict__ U1,
                                                   const T* __restrict__ U2, T* __restrict__ Ut,
                                                   int m1, int m2) {
  const int N = m1 * m2;  // (at most 262140: 32-bit index arithmetic)
  for (int x = blockIdx.y; x < N; x += gridDim.y) {
    const int y = (x & ~63) + (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (y >= N) continue;
    const int k = x / m2, i = x - k * m2, k1 = y / m2, i1 = y - k1 * m2;
    Ut[(int64_t)x * N + y] = U1[(int64_t)k * m1 + k1] * U2[(int64_t)i * m2 + i1];
  }
}

// Every fibre scale positive and finite, checked before the slab loop so that a bad one is
// reported by its fibre index k m2 + i + 1, as the stacked route's sweep reports it.
template <typename T>
__global__ __launch_bounds__(256) void k_check_fibre_scales(int64_t count,
                                                            const T* __restrict__ s, int* info) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= count) return;
  const T v = s[f];
  if (!(v > T(0)) || !isfinite(v)) record_info(info, 3, (int)(f + 1));
}

struct Kron3Ws {
  void *U1, *U2, *U3, *Wg, *scratch, *scratch3;
};

Kron3Ws carve3(int64_t m1, int64_t m2, int64_t m3, int dtype, void* ws) {
  const size_t es = dtype == 0 ? sizeof(float) : sizeof(double);
  char* c = (char*)ws;
  Kron3Ws w;
  w.U1 = c;
  c += align_up((size_t)m1 * m1 * es);
  w.U2 = c;
  c += align_up((size_t)m2 * m2 * es);
  w.U3 = c;
  c += align_up((size_t)m3 * m3 * es);
  w.Wg = c;
  c += align_up(use_tall(m1, m2, dtype) ? (size_t)(m1 * m2) * (size_t)(m1 * m2) * es
                                        : (size_t)m1 * m2 * m3 * es);
  w.scratch = c;
  w.scratch3 = c + factor_workspace(m2);
  return w;
}

// Tall route: factors, the stacked factor U1' (x) U2' (in the space the slab buffer Wg
// takes in the slab route, which holds it), then one sweep of the (m1 m2) x m3 matrix.
template <typename T>
hipError_t kron3_tall(int64_t m1, int64_t m2, int64_t m3, int bits, int dtype, const T* W,
                      const T* A1, const T* A2, const T* A3, const T* scales, int8_t* codes,
                      T* Q, void* ws, int* info, hipStream_t s) {
  const Kron3Ws w = carve3(m1, m2, m3, dtype, ws);
  const int64_t N = m1 * m2;
  T* Ut = (T*)w.Wg;
  hipError_t e = factor_pair_enqueue(m2, A2, w.U2, w.scratch, m3, A3, w.U3, w.scratch3, dtype,
                                     info, s, kInfoA2, kInfoA3);
  if (e == hipSuccess) e = factor_enqueue(m1, dtype, A1, w.U1, w.scratch, info, kInfoA1, s);
  if (e != hipSuccess) return e;
  const int64_t gx = cdiv(N, 256), gy = N < 65535 ? N : 65535;
  prof_begin(KC_OTHER, s);
  k_kron_unit<T><<<dim3((unsigned)gx, (unsigned)gy), 256, 0, s>>>((const T*)w.U1, (const T*)w.U2,
                                                                   Ut, (int)m1, (int)m2);
  // (about half of the N^2 entries: the tiles on and above the diagonal)
  prof_end(KC_OTHER, s, 0.5 * (double)N * (double)N,
           0.5 * (double)sizeof(T) * (double)N * (double)N);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return sweep_enqueue(N, m3, bits, dtype, W, Ut, w.U3, scales, codes, Q, w.scratch, info, s);
}

template <typename T>
hipError_t kron3_typed(int64_t m1, int64_t m2, int64_t m3, int bits, int dtype, const T* W,
                       const T* A1, const T* A2, const T* A3, const T* scales, int8_t* codes,
                       T* Q, void* ws, int* info, hipStream_t s) {
  if (use_tall(m1, m2, dtype))
    return kron3_tall<T>(m1, m2, m3, bits, dtype, W, A1, A2, A3, scales, codes, Q, ws, info, s);
  const Kron3Ws w = carve3(m1, m2, m3, dtype, ws);
  const int64_t slab = m2 * m3;
  T* Wg = (T*)w.Wg;
  const T* U1 = (const T*)w.U1;
  hipError_t e = factor_pair_enqueue(m2, A2, w.U2, w.scratch, m3, A3, w.U3, w.scratch3, dtype,
                                     info, s, kInfoA2, kInfoA3);
  if (e == hipSuccess) e = factor_enqueue(m1, dtype, A1, w.U1, w.scratch, info, kInfoA1, s);
  if (e == hipSuccess) {
    k_check_fibre_scales<T><<<(unsigned)cdiv(m1 * m2, 256), 256, 0, s>>>(m1 * m2, scales, info);
    e = hipGetLastError();
  }
  if (e == hipSuccess)
    e = hipMemcpyAsync(Wg, W, (size_t)m1 * slab * sizeof(T), hipMemcpyDeviceToDevice, s);
  for (int64_t b = 0; e == hipSuccess && b < m1; b += kSlabBlock) {
    const int64_t end = b + kSlabBlock < m1 ? b + kSlabBlock : m1;
    for (int64_t k = b; e == hipSuccess && k < end; ++k) {
      e = slab_feedback<T>(Wg, Q, U1, m1, slab, (int)k, (int)k + 1, (int)b, (int)k, s);
      if (e == hipSuccess)
        e = sweep_enqueue(m2, m3, bits, dtype, Wg + k * slab, w.U2, w.U3, scales + k * m2,
                          codes + k * slab, Q + k * slab, w.scratch, info, s);
    }
    if (e == hipSuccess)
      e = slab_feedback<T>(Wg, Q, U1, m1, slab, (int)end, (int)m1, (int)b, (int)end, s);
  }
  return e;
}

}  // namespace

size_t kron3_workspace(int64_t m1, int64_t m2, int64_t m3, int dtype) {
  const size_t es = dtype == 0 ? sizeof(float) : sizeof(double);
  size_t scratch = factor_workspace(m2) + factor_workspace(m3);
  if (factor_workspace(m1) > scratch) scratch = factor_workspace(m1);
  const bool tall = use_tall(m1, m2, dtype);
  // the tall route sweeps the stacked matrix and keeps U1' (x) U2' where the slab route
  // keeps its slab buffer
  const size_t sw = tall ? sweep_workspace(m1 * m2, m3, dtype) : sweep_workspace(m2, m3, dtype);
  if (sw > scratch) scratch = sw;
  const size_t mid = tall ? (size_t)(m1 * m2) * (size_t)(m1 * m2) * es : (size_t)m1 * m2 * m3 * es;
  return align_up((size_t)m1 * m1 * es) + align_up((size_t)m2 * m2 * es) +
         align_up((size_t)m3 * m3 * es) + align_up(mid) + scratch;
}

hipError_t kron3_enqueue(int64_t m1, int64_t m2, int64_t m3, int bits, int dtype, const void* W,
                         const void* A1, const void* A2, const void* A3, const void* scales,
                         int8_t* codes, void* Q, void* ws, int* info, hipStream_t s) {
  if (dtype == 0)
    return kron3_typed<float>(m1, m2, m3, bits, dtype, (const float*)W, (const float*)A1,
                              (const float*)A2, (const float*)A3, (const float*)scales, codes,
                              (float*)Q, ws, info, s);
  return kron3_typed<double>(m1, m2, m3, bits, dtype, (const double*)W, (const double*)A1,
                             (const double*)A2, (const double*)A3, (const double*)scales, codes,
                             (double*)Q, ws, info, s);
}

}  // namespace g2d
