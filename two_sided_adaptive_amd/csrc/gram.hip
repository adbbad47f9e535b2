// Kronecker factor accumulation: A += alpha * X^T X for a block of N samples (rows of the
// N x p activation matrix X).  The pages use Kronecker-factored Hessians without stating
// how the factors are estimated ("GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding",
// arxivlens page, Abstract: two-sided rounding under a Kronecker-factored Hessian); the
// plain second-moment (Gram) accumulation is the step before the quantizer.
//
// One workgroup per 64x64 tile of the lower triangle runs the MFMA tile GEMM over the
// samples (a "TN" product: both operands are column blocks of X, read k-major), adding into
// A; a second pass copies the lower triangle onto the upper through LDS, so A leaves
// symmetric.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"
#include "prof.hpp"

namespace g2d {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void k_gram(const T* __restrict__ X, T* __restrict__ A,
                                              int64_t p, int64_t N, int64_t kchunk, T alpha) {
  __shared__ TileSmem<T> sm;
  // blockIdx.x enumerates the lower tiles row by row: t = ti (ti + 1) / 2 + tj, tj <= ti
  const int64_t t = blockIdx.x;
  int64_t ti = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (ti * (ti + 1) / 2 > t) --ti;
  while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
  const int64_t tj = t - ti * (ti + 1) / 2;
  const int64_t i0 = ti * kTile, j0 = tj * kTile;
  const int M = (int)(p - i0 < kTile ? p - i0 : kTile);
  const int Nn = (int)(p - j0 < kTile ? p - j0 : kTile);
  for (int64_t k0 = 0; k0 < N; k0 += kchunk) {
    const int kc = (int)(N - k0 < kchunk ? N - k0 : kchunk);
    tile_gemm<T, true, false>(X + k0 * p + i0, p, X + k0 * p + j0, p, A + i0 * p + j0, p, M, Nn,
                              0, kc, alpha, T(1), sm);
    __syncthreads();
  }
}

// Upper tile (I, J), J >= I, becomes the transpose of lower tile (J, I); on a diagonal tile
// only the entries above the diagonal are written.
template <typename T>
__global__ __launch_bounds__(256) void k_mirror(T* __restrict__ A, int64_t p) {
  __shared__ T tile[kTile][kTile + 1];
  const int64_t t = blockIdx.x;
  int64_t tj = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (tj * (tj + 1) / 2 > t) --tj;
  while ((tj + 1) * (tj + 2) / 2 <= t) ++tj;
  const int64_t ti = t - tj * (tj + 1) / 2;  // ti <= tj: source tile (tj, ti) is lower
  const int64_t r0 = tj * kTile, c0 = ti * kTile;
  for (int idx = threadIdx.x; idx < kTile * kTile; idx += 256) {
    const int r = idx >> 6, c = idx & 63;
    if (r0 + r < p && c0 + c < p) tile[r][c] = A[(r0 + r) * p + c0 + c];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < kTile * kTile; idx += 256) {
    const int r = idx >> 6, c = idx & 63;  // destination (c0 + r, r0 + c)
    const int64_t gi = c0 + r, gj = r0 + c;
    if (gi < p && gj < p && gj > gi) A[gi * p + gj] = tile[c][r];
  }
}

template <typename T>
hipError_t gram_typed(int64_t p, int64_t N, const T* X, double alpha, T* A, hipStream_t s) {
  const int64_t nt = cdiv(p, kTile);
  const int64_t tiles = nt * (nt + 1) / 2;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  // every buffer range handed to the tile GEMM stays below 2^31 bytes
  int64_t kchunk = (((int64_t)1 << 31) - 1) / ((int64_t)sizeof(T) * p) - 1;
  if (kchunk < 1 || (double)p * (double)p * sizeof(T) >= 2147483647.0) return hipErrorInvalidValue;
  if (kchunk > N) kchunk = N;
  prof_begin(KC_GRAM, s);
  k_gram<T><<<(unsigned)tiles, 256, 0, s>>>(X, A, p, N, kchunk, (T)alpha);
  k_mirror<T><<<(unsigned)tiles, 256, 0, s>>>(A, p);
  const double es = sizeof(T);
  prof_end(KC_GRAM, s, (double)N * (double)p * (double)(p + 1),
           es * ((double)N * (double)p + 2.0 * (double)p * (double)p));
  return hipGetLastError();
}

}  // namespace

hipError_t gram_enqueue(int64_t p, int64_t N, int dtype, const void* X, double alpha, void* A,
                        hipStream_t s) {
  if (dtype == 0) return gram_typed<float>(p, N, (const float*)X, alpha, (float*)A, s);
  return gram_typed<double>(p, N, (const double*)X, alpha, (double*)A, s);
}

}  // namespace g2d
