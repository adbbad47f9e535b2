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
#include "prof.hpp"

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

// One diagonal 64x64 block: Cholesky, then its inverse.  Writes L into Ar (lower
// part), X_kk = L_kk^-1 into X (zeros above the diagonal) and its transpose into DinvT.
// Rows beyond p are padded with the identity.  256 threads, no branches in the loops.
//  * Cholesky: thread t owns row i = t/4, columns k = 4u + t%4 (u < 16) in registers.
//    Step j publishes the still unscaled column j (pivot included) through a double-
//    buffered LDS column, one barrier, after which every thread applies
//    a[i][k] -= a[i][j] a[k][j] / a[j][j] to its elements and the owners of column j
//    scale it by 1/sqrt(a[j][j]).
//  * Inverse: the quad of threads 4c..4c+3 forward-substitutes column c of L^-1 with
//    the reciprocal diagonal; thread q keeps the right-hand side of rows 4u + q, and
//    the new entry x[i][c] is broadcast inside the quad with DPP (no barrier).
__device__ inline double quad_bcast(double v, int src) {
  // quad_perm [src, src, src, src] on both 32-bit halves (src is a literal after unrolling)
  int lo = __double2loint(v), hi = __double2hiint(v);
  switch (src) {
    case 0:
      lo = __builtin_amdgcn_mov_dpp(lo, 0x00, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0x00, 0xF, 0xF, false);
      break;
    case 1:
      lo = __builtin_amdgcn_mov_dpp(lo, 0x55, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0x55, 0xF, 0xF, false);
      break;
    case 2:
      lo = __builtin_amdgcn_mov_dpp(lo, 0xAA, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0xAA, 0xF, 0xF, false);
      break;
    default:
      lo = __builtin_amdgcn_mov_dpp(lo, 0xFF, 0xF, 0xF, false);
      hi = __builtin_amdgcn_mov_dpp(hi, 0xFF, 0xF, 0xF, false);
      break;
  }
  return __hiloint2double(hi, lo);
}

// 1/x and 1/sqrt(x) from the hardware estimates refined by one Newton step (a few
// ulp; the factorisation does not need IEEE-rounded quotients).
__device__ inline double rcp_nr(double x) {
  double r = __builtin_amdgcn_rcp(x);
  r = fma(r, fma(-x, r, 1.0), r);
  return r;
}
__device__ inline double rsq_nr(double x) {
  double r = __builtin_amdgcn_rsq(x);
  const double h = 0.5 * x * r;
  r = fma(r, fma(-h, r, 0.5), r);
  return r;
}

__global__ __launch_bounds__(256) void k_potrf_diag(int64_t p, int kb, double* __restrict__ Ar,
                                                    double* __restrict__ X,
                                                    double* __restrict__ DinvT, int* info,
                                                    int side_code) {
  __shared__ double col[2][NB];
  __shared__ double piv[NB];                // a[j][j] before scaling (for the SPD check)
  __shared__ double rdiag[NB];              // 1 / L[j][j]
  __shared__ double lt[NB][4][NB / 4 + 2];  // lt[c][q][u] = L[4u+q][c] (zero above diagonal)
  const int t = threadIdx.x;
  const int i = t >> 2, q = t & 3;
  const int64_t r0 = (int64_t)kb * NB;
  const int nv = (p - r0) < NB ? (int)(p - r0) : NB;
  double a[NB / 4];
  {
    // all loads in flight together; rows past the matrix read as zero
    const rsrc_t rr = make_rsrc(Ar + r0 * p + r0, ((int64_t)(nv - 1) * p + nv) * 8);
#pragma unroll
    for (int u = 0; u < NB / 4; ++u) a[u] = buf_load<double>(rr, (uint32_t)(i * p + 4 * u + q));
#pragma unroll
    for (int u = 0; u < NB / 4; ++u) {
      const int k = 4 * u + q;
      const bool in = i < nv && k < nv;
      a[u] = in ? (k <= i ? a[u] : 0.0) : (i == k ? 1.0 : 0.0);
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int uj = j >> 2, qj = j & 3;
    double* cj = col[j & 1];
    if (q == qj) cj[i] = a[uj];  // column j, unscaled (rows < j hold finished L values)
    __syncthreads();
    const double pj = cj[j];
    const double inv = rcp_nr(pj);
    const double rs = rsq_nr(pj);
    const double coef = (i > j) ? cj[i] * inv : 0.0;
#pragma unroll
    for (int u = 0; u < NB / 4; ++u) {
      const int k = 4 * u + q;
      const double ck = (k > j) ? cj[k] : 0.0;
      a[u] = fma(-coef, ck, a[u]);
    }
    if (q == qj) a[uj] = (i >= j) ? a[uj] * rs : a[uj];
    if (t == 0) {
      piv[j] = pj;
      rdiag[j] = rs;  // 1 / L[j][j]
    }
  }
  // publish L (transposed, quad-split, zero above the diagonal) for the inverse
#pragma unroll
  for (int u = 0; u < NB / 4; ++u) {
    const int k = 4 * u + q;
    lt[k][i & 3][i >> 2] = (k <= i) ? a[u] : 0.0;
  }
  __syncthreads();
  if (t < 64) {  // first non-positive (or NaN) pivot, found by one wave
    const bool bad = t < nv && !(piv[t] > 0.0);
    const unsigned long long mask = __ballot(bad);
    if (t == 0 && mask != 0ull) record_info(info, side_code, (int)(r0 + __ffsll((long long)mask)));
  }
  if (i < nv) {
#pragma unroll
    for (int u = 0; u < NB / 4; ++u) {
      const int k = 4 * u + q;
      if (k <= i && k < nv) Ar[(r0 + i) * p + r0 + k] = a[u];
    }
  }
  __syncthreads();
  // inverse: quad c = t/4 solves column c
  const int c = i;
  double rhs[NB / 4], xv[NB / 4];
#pragma unroll
  for (int u = 0; u < NB / 4; ++u) {
    rhs[u] = (4 * u + q == c) ? 1.0 : 0.0;
    xv[u] = 0.0;
  }
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    const int ur = r >> 2, qr = r & 3;
    double x = quad_bcast(rhs[ur] * rdiag[r], qr);  // meaningful in lane q == qr
    x = (r < c) ? 0.0 : x;
    xv[ur] = (q == qr) ? x : xv[ur];
    const double* lr = &lt[r][q][0];
#pragma unroll
    for (int u = 0; u < NB / 4; ++u) rhs[u] = fma(-lr[u], x, rhs[u]);
  }
  // X rows 4u+q, column c; DinvT[c][row] = X[row][c]
  double* dt = DinvT + (int64_t)kb * NB * NB + (int64_t)c * NB;
#pragma unroll
  for (int u = 0; u < NB / 4; ++u) {
    const int row = 4 * u + q;
    dt[row] = xv[u];
    if (row < nv && c < nv) X[(r0 + row) * p + r0 + c] = xv[u];
  }
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

// Dense GEMM flops of one launch (only evaluated while the measurement hook is on).
double trailing_flops(int64_t p, int kb) {
  const int64_t nblk = cdiv(p, NB);
  const double K = (double)((p - kb * NB) < NB ? (p - kb * NB) : NB);
  double f = 0.0;
  for (int64_t i = kb + 1; i < nblk; ++i) {
    const double M = (double)((p - i * NB) < NB ? (p - i * NB) : NB);
    for (int64_t j = kb + 1; j <= i; ++j) {
      const double N = (double)((p - j * NB) < NB ? (p - j * NB) : NB);
      f += 2.0 * M * N * K;
    }
  }
  return f;
}

void trtri_flops(int64_t p, int64_t h, double* f1, double* f2) {
  *f1 = *f2 = 0.0;
  for (int64_t g0 = 0; g0 < p; g0 += 2 * h) {
    const int64_t h1 = (p - g0) < h ? (p - g0) : h;
    const int64_t h2 = (p - g0 - h) < h ? (p - g0 - h) : h;
    if (h2 <= 0) continue;
    for (int64_t ti = 0; ti * NB < h2; ++ti) {
      const double M = (double)((h2 - ti * NB) < NB ? (h2 - ti * NB) : NB);
      const double kend = (double)((ti + 1) * NB < h2 ? (ti + 1) * NB : h2);
      for (int64_t tj = 0; tj * NB < h1; ++tj) {
        const double N = (double)((h1 - tj * NB) < NB ? (h1 - tj * NB) : NB);
        *f1 += 2.0 * M * N * (double)(h1 - tj * NB);
        *f2 += 2.0 * M * N * kend;
      }
    }
  }
}

hipError_t factor_enqueue(int64_t p, int dtype, const void* A, void* U, void* ws, int* info,
                          int side_code, hipStream_t s) {
  FactorWs f = carve(p, ws);
  const int64_t nblk = cdiv(p, NB);
  const bool pr = prof_on();
  const double es = dtype == 0 ? 4.0 : 8.0, pp = (double)p * (double)p;
  dim3 eg((unsigned)cdiv(p, 64), (unsigned)cdiv(p, 4));
  prof_begin(KC_OTHER, s);
  if (dtype == 0)
    k_reverse_sym<float><<<eg, 256, 0, s>>>(p, (const float*)A, f.Ar);
  else
    k_reverse_sym<double><<<eg, 256, 0, s>>>(p, (const double*)A, f.Ar);
  prof_end(KC_OTHER, s, 0.0, pp * (es + 8.0));
  for (int kb = 0; kb < nblk; ++kb) {
    const double nv = (double)((p - kb * NB) < NB ? (p - kb * NB) : NB);
    prof_begin(KC_POTRF, s);
    k_potrf_diag<<<1, 256, 0, s>>>(p, kb, f.Ar, f.X, f.DinvT, info, side_code);
    prof_end(KC_POTRF, s, 2.0 / 3.0 * nv * nv * nv, 8.0 * (nv * nv * 2.5 + NB * NB));
    const int rest = (int)(nblk - kb - 1);
    if (rest > 0) {
      const double rows = (double)(p - (int64_t)(kb + 1) * NB);
      prof_begin(KC_PANEL, s);
      k_panel_solve<<<rest, 256, 0, s>>>(p, kb, f.Ar, f.DinvT);
      prof_end(KC_PANEL, s, 2.0 * rows * nv * nv, 8.0 * (2.0 * rows * nv + nv * nv));
      prof_begin(KC_TRAILING, s);
      k_trailing<<<dim3(rest, rest), 256, 0, s>>>(p, kb, f.Ar);
      prof_end(KC_TRAILING, s, pr ? trailing_flops(p, kb) : 0.0,
               8.0 * (rows * (rows + NB) + rows * nv));
    }
  }
  for (int64_t h = NB; h < p; h *= 2) {
    const int64_t groups = cdiv(p, 2 * h);
    dim3 g((unsigned)cdiv(h, NB), (unsigned)cdiv(h, NB), (unsigned)groups);
    double f1 = 0.0, f2 = 0.0;
    if (pr) trtri_flops(p, h, &f1, &f2);
    prof_begin(KC_TRTRI, s);
    k_trtri_step1<<<g, 256, 0, s>>>(p, h, f.Ar, f.X, f.Tb, f.ldt);
    k_trtri_step2<<<g, 256, 0, s>>>(p, h, f.X, f.Tb, f.ldt);
    prof_end(KC_TRTRI, s, f1 + f2, 8.0 * 4.0 * (double)h * (double)p);
  }
  prof_begin(KC_OTHER, s);
  if (dtype == 0)
    k_finalize<float><<<eg, 256, 0, s>>>(p, f.X, (float*)U);
  else
    k_finalize<double><<<eg, 256, 0, s>>>(p, f.X, (double*)U);
  prof_end(KC_OTHER, s, 0.0, pp * (8.0 / 2.0 + es));
  return hipGetLastError();
}

}  // namespace g2d
