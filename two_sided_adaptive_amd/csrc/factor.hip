// Factor stage for gfx950: the unit upper triangular feedback factor U' of an SPD
// matrix, U' = diag(U)^-1 U with A^-1 = U^T U.
//
// Page reference: mind-verse article "Neue Ansaetze ... durch GPTQ-2D", section
// "GPTQ-2D: Eine Weiterentwicklung der adaptiven Rundung" (errors propagate through
// a triangular feedback matrix); arxivlens page "GPTQ-2D: Cubic-Time Two-Sided
// Adaptive Rounding", Limitations (fixed bases, factorisations computed once).
//
// Route (float64 throughout; MFMA f64 for the cubic parts):
//   J A J = L L^T (lower Cholesky of the index-reversed matrix, blocked, right-looking)
//   X = L^-1 (diagonal 64-blocks inverted in the panel kernel, the rest by recursive
//            doubling: X21 = -X22 L21 X11)
//   U = J X J is the upper Cholesky factor of A^-1; U'[i][j] = U[i][j] / U[i][i].
// Diagonal-block inverses double as the panel solve: L21 = A21 (L11^-1)^T is a GEMM.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace g2d {
namespace {

constexpr int NB = 64;  // panel width = tile edge

// Ar[i][j] = A[p-1-min(i,j)][p-1-max(i,j)]: the reversed matrix, filled symmetric from
// the lower triangle of A.
template <typename T>
__global__ __launch_bounds__(256) void k_reverse_sym(int64_t p, const T* __restrict__ A,
                                                     double* __restrict__ Ar) {
  const int64_t j = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t i = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  if (i >= p || j >= p) return;
  const int64_t a = i > j ? i : j, b = i > j ? j : i;
  Ar[i * p + j] = (double)A[(p - 1 - b) * p + (p - 1 - a)];
}

// One diagonal 64x64 block: Cholesky in LDS, then its inverse.  Writes L into Ar
// (lower part), X_kk = L_kk^-1 into X (zeros above the diagonal) and its transpose
// into DinvT.  Rows beyond p are padded with the identity.
__global__ __launch_bounds__(64) void k_potrf_diag(int64_t p, int kb, double* __restrict__ Ar,
                                                   double* __restrict__ X,
                                                   double* __restrict__ DinvT, int* info,
                                                   int side_code) {
  __shared__ double a[NB][NB + 1];
  __shared__ double x[NB][NB + 1];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)kb * NB;
  const int nv = (p - r0) < NB ? (int)(p - r0) : NB;
  for (int c = 0; c < NB; ++c) {
    double v;
    if (t < nv && c < nv)
      v = (c <= t) ? Ar[(r0 + t) * p + r0 + c] : 0.0;
    else
      v = (t == c) ? 1.0 : 0.0;
    a[t][c] = v;
    x[t][c] = 0.0;
  }
  __syncthreads();
  int bad = -1;
  for (int j = 0; j < NB; ++j) {
    double d = a[j][j];
    if (!(d > 0.0) && bad < 0) bad = j;
    d = sqrt(d);
    __syncthreads();
    if (t == j) a[j][j] = d;
    if (t > j) a[t][j] = a[t][j] / d;
    __syncthreads();
    if (t > j) {
      const double lij = a[t][j];
      for (int k = j + 1; k <= t; ++k) a[t][k] -= lij * a[k][j];
    }
    __syncthreads();
  }
  // X = L^-1, row by row: x[i][c] = (delta_ic - sum_{k<i} a[i][k] x[k][c]) / a[i][i]
  for (int i = 0; i < NB; ++i) {
    double s = (i == t) ? 1.0 : 0.0;
    for (int k = 0; k < i; ++k) s -= a[i][k] * x[k][t];
    if (t <= i) x[i][t] = s / a[i][i];
    __syncthreads();
  }
  if (t < nv) {
    for (int c = 0; c < nv; ++c) {
      if (c <= t) Ar[(r0 + t) * p + r0 + c] = a[t][c];
      X[(r0 + t) * p + r0 + c] = x[t][c];
    }
  }
  for (int c = 0; c < NB; ++c) DinvT[(int64_t)kb * NB * NB + (int64_t)c * NB + t] = x[t][c];
  if (t == 0 && bad >= 0 && bad < nv) record_info(info, side_code, (int)(r0 + bad + 1));
}

// Panel solve L[i][kb] = A[i][kb] (L_kk^-1)^T for row tiles below the diagonal block.
__global__ __launch_bounds__(256) void k_panel_solve(int64_t p, int kb, double* Ar,
                                                     const double* __restrict__ DinvT) {
  __shared__ TileSmem<double> sm;
  const int64_t r0 = (int64_t)(kb + 1 + blockIdx.x) * NB;
  const int64_t c0 = (int64_t)kb * NB;
  const int M = (p - r0) < NB ? (int)(p - r0) : NB;
  const int K = (p - c0) < NB ? (int)(p - c0) : NB;
  double* tile = Ar + r0 * p + c0;
  tile_gemm<double, false, false>(tile, p, DinvT + (int64_t)kb * NB * NB, NB, tile, p, M, K, 0, K,
                                  1.0, 0.0, sm);
}

// Trailing update of the lower triangle: Ar[i][j] -= L[i][kb] L[j][kb]^T, kb < j <= i.
__global__ __launch_bounds__(256) void k_trailing(int64_t p, int kb, double* Ar) {
  __shared__ TileSmem<double> sm;
  const int i = kb + 1 + blockIdx.y, j = kb + 1 + blockIdx.x;
  if (j > i) return;
  const int64_t r0 = (int64_t)i * NB, cj = (int64_t)j * NB, ck = (int64_t)kb * NB;
  const int M = (p - r0) < NB ? (int)(p - r0) : NB;
  const int N = (p - cj) < NB ? (int)(p - cj) : NB;
  const int K = (p - ck) < NB ? (int)(p - ck) : NB;
  tile_gemm<double, false, true>(Ar + r0 * p + ck, p, Ar + cj * p + ck, p, Ar + r0 * p + cj, p, M,
                                 N, 0, K, -1.0, 1.0, sm);
}

// Recursive doubling, step 1: T = L21 X11 for every pair of h-blocks (group z).
// X11 is lower triangular, so column tile tj only needs k >= 64*tj.
__global__ __launch_bounds__(256) void k_trtri_step1(int64_t p, int64_t h, const double* Ar,
                                                     const double* X, double* Tb, int64_t ldt) {
  __shared__ TileSmem<double> sm;
  const int64_t g0 = (int64_t)blockIdx.z * 2 * h;
  const int64_t h1 = (p - g0) < h ? (p - g0) : h;
  const int64_t h2 = (p - g0 - h) < h ? (p - g0 - h) : h;
  const int64_t ti = blockIdx.y, tj = blockIdx.x;
  if (h2 <= 0 || ti * NB >= h2 || tj * NB >= h1) return;
  const int M = (h2 - ti * NB) < NB ? (int)(h2 - ti * NB) : NB;
  const int N = (h1 - tj * NB) < NB ? (int)(h1 - tj * NB) : NB;
  const int64_t rA = g0 + h + ti * NB;
  tile_gemm<double, false, false>(Ar + rA * p + g0, p, X + g0 * p + g0 + tj * NB, p,
                                  Tb + rA * ldt + tj * NB, ldt, M, N, (int)(tj * NB), (int)h1, 1.0,
                                  0.0, sm);
}

// Step 2: X21 = -X22 T.  X22 is lower triangular, so row tile ti only needs k < 64*(ti+1).
__global__ __launch_bounds__(256) void k_trtri_step2(int64_t p, int64_t h, double* X,
                                                     const double* Tb, int64_t ldt) {
  __shared__ TileSmem<double> sm;
  const int64_t g0 = (int64_t)blockIdx.z * 2 * h;
  const int64_t h1 = (p - g0) < h ? (p - g0) : h;
  const int64_t h2 = (p - g0 - h) < h ? (p - g0 - h) : h;
  const int64_t ti = blockIdx.y, tj = blockIdx.x;
  if (h2 <= 0 || ti * NB >= h2 || tj * NB >= h1) return;
  const int M = (h2 - ti * NB) < NB ? (int)(h2 - ti * NB) : NB;
  const int N = (h1 - tj * NB) < NB ? (int)(h1 - tj * NB) : NB;
  const int64_t rA = g0 + h + ti * NB;
  const int kend = (int)((ti + 1) * NB < h2 ? (ti + 1) * NB : h2);
  tile_gemm<double, false, false>(X + rA * p + g0 + h, p, Tb + (g0 + h) * ldt + tj * NB, ldt,
                                  X + rA * p + g0 + tj * NB, p, M, N, 0, kend, -1.0, 0.0, sm);
}

// U'[i][j] = X[p-1-i][p-1-j] / X[p-1-i][p-1-i] for i <= j, zero below the diagonal.
template <typename T>
__global__ __launch_bounds__(256) void k_finalize(int64_t p, const double* __restrict__ X,
                                                  T* __restrict__ U) {
  const int64_t j = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t i = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  if (i >= p || j >= p) return;
  T v = T(0);
  if (i <= j) {
    const int64_t a = p - 1 - i, b = p - 1 - j;
    v = (T)(X[a * p + b] / X[a * p + a]);
  }
  U[i * p + j] = v;
}

struct FactorWs {
  double* Ar;
  double* X;
  double* DinvT;
  double* Tb;
  int64_t ldt;
};

// Largest half-size used by the recursive doubling (the leading dimension of T).
int64_t trtri_ldt(int64_t p) {
  int64_t h = NB;
  while (2 * h < p) h *= 2;
  return h;
}

FactorWs carve(int64_t p, void* ws) {
  FactorWs f;
  char* c = (char*)ws;
  const int64_t nblk = cdiv(p, NB);
  f.ldt = trtri_ldt(p);
  f.Ar = (double*)c;
  c += align_up((size_t)p * p * sizeof(double));
  f.X = (double*)c;
  c += align_up((size_t)p * p * sizeof(double));
  f.DinvT = (double*)c;
  c += align_up((size_t)nblk * NB * NB * sizeof(double));
  f.Tb = (double*)c;
  return f;
}

}  // namespace

size_t factor_workspace(int64_t p) {
  const int64_t nblk = cdiv(p, NB);
  const int64_t ldt = trtri_ldt(p);
  return 2 * align_up((size_t)p * p * sizeof(double)) +
         align_up((size_t)nblk * NB * NB * sizeof(double)) +
         align_up((size_t)p * ldt * sizeof(double));
}

hipError_t factor_enqueue(int64_t p, int dtype, const void* A, void* U, void* ws, int* info,
                          int side_code, hipStream_t s) {
  FactorWs f = carve(p, ws);
  const int64_t nblk = cdiv(p, NB);
  dim3 eg((unsigned)cdiv(p, 64), (unsigned)cdiv(p, 4));
  if (dtype == 0)
    k_reverse_sym<float><<<eg, 256, 0, s>>>(p, (const float*)A, f.Ar);
  else
    k_reverse_sym<double><<<eg, 256, 0, s>>>(p, (const double*)A, f.Ar);
  for (int kb = 0; kb < nblk; ++kb) {
    k_potrf_diag<<<1, 64, 0, s>>>(p, kb, f.Ar, f.X, f.DinvT, info, side_code);
    const int rest = (int)(nblk - kb - 1);
    if (rest > 0) {
      k_panel_solve<<<rest, 256, 0, s>>>(p, kb, f.Ar, f.DinvT);
      k_trailing<<<dim3(rest, rest), 256, 0, s>>>(p, kb, f.Ar);
    }
  }
  for (int64_t h = NB; h < p; h *= 2) {
    const int64_t groups = cdiv(p, 2 * h);
    dim3 g((unsigned)cdiv(h, NB), (unsigned)cdiv(h, NB), (unsigned)groups);
    k_trtri_step1<<<g, 256, 0, s>>>(p, h, f.Ar, f.X, f.Tb, f.ldt);
    k_trtri_step2<<<g, 256, 0, s>>>(p, h, f.X, f.Tb, f.ldt);
  }
  if (dtype == 0)
    k_finalize<float><<<eg, 256, 0, s>>>(p, f.X, (float*)U);
  else
    k_finalize<double><<<eg, 256, 0, s>>>(p, f.X, (double*)U);
  return hipGetLastError();
}

}  // namespace g2d
