// Factor stage for gfx950: the unit upper triangular feedback factor U' of an SPD
// matrix, U' = diag(U)^-1 U with A^-1 = U^T U.
//
// Page reference: mind-verse article "Neue Ansaetze ... durch GPTQ-2D", section
// "GPTQ-2D: Eine Weiterentwicklung der adaptiven Rundung" (errors propagate through
// a triangular feedback matrix); arxivlens page "GPTQ-2D: Cubic-Time Two-Sided
// Adaptive Rounding", Limitations (fixed bases, factorisations computed once).
//
// Route (float64 throughout; MFMA f64 for the cubic parts):
//   J A J = L L^T (lower Cholesky of the index-reversed matrix, blocked, right-looking,
//            one launch per 64-wide step)
//   X = L^-1 (diagonal 64-blocks inverted with their factorisation, the rest by
//            recursive doubling: X21 = -X22 L21 X11)
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

// Quad broadcast of a double: every lane of a quad receives lane `src`'s value.
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

// LDS of the diagonal-block factorisation.  Before it starts, lf and xf stage the
// panel tiles of the previous step.
constexpr int PD = NB + 2;
struct BlockSmem {
  double lf[NB][PD];  // L (zeros above the diagonal)
  double xf[NB][PD];  // X = L^-1 (zeros above the diagonal)
  union {
    struct {
      double pub[NB][4];  // the group's four columns, current values
      double lc[NB][4];   // the group's four columns of L
    } g;
    double tsc[4][16][18];  // per-wave 16x16 temporaries of the inverse
  } u;
  double piv[NB];  // pivots before the square root (SPD check)
};

// Cholesky and inverse of one 64x64 diagonal block held in MFMA accumulator layout by
// the four waves of the workgroup (wave w: rows 16w..16w+15, acc[t] the 16x16 tile of
// columns 16t..16t+15; only the lower triangle is read; padding rows/columns hold the
// identity).  Leaves L in sm.lf and X = L^-1 in sm.xf; ends with a barrier.
//  * Cholesky, four columns at a time: the group's columns are published to LDS; lanes
//    0..15 of every wave (one per row) factor the 4x4 diagonal block (redundantly) and
//    solve their row's four L entries; the rank-4 update of the trailing tiles is one
//    MFMA per tile.
//  * Inverse by 16x16 tiles: wave t inverts diagonal tile t by forward substitution
//    (quad c solves column c, the new entry broadcast inside the quad with DPP); the
//    tiles below follow by distance, X_ij = -X_ii (sum_{j<=k<i} L_ik X_kj), with MFMA.
__device__ inline void chol_inv_block(Mfma<double>::acc_t (&acc)[4], BlockSmem& sm) {
  typedef Mfma<double>::acc_t acc_t;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, cl = lane & 15, kq = lane >> 4;
  for (int idx = tid; idx < NB * NB; idx += 256) sm.xf[idx >> 6][idx & 63] = 0.0;
#pragma unroll
  for (int g = 0; g < NB / 4; ++g) {
    const int tg = g >> 2, cg = 4 * (g & 3), d0 = 4 * g;
    if (cl >= cg && cl < cg + 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sm.u.g.pub[16 * w + Mfma<double>::row(lane, e)][cl - cg] = acc[tg][e];
    }
    __syncthreads();
    if (lane < 16) {
      const int i = 16 * w + lane;
      const double(*pub)[4] = sm.u.g.pub;
      const double b00 = pub[d0][0];
      const double b10 = pub[d0 + 1][0], b11 = pub[d0 + 1][1];
      const double b20 = pub[d0 + 2][0], b21 = pub[d0 + 2][1], b22 = pub[d0 + 2][2];
      const double b30 = pub[d0 + 3][0], b31 = pub[d0 + 3][1], b32 = pub[d0 + 3][2];
      const double b33 = pub[d0 + 3][3];
      const double q0 = b00, s0 = rsq_nr(q0);
      const double l00 = q0 * s0, l10 = b10 * s0, l20 = b20 * s0, l30 = b30 * s0;
      const double q1 = fma(-l10, l10, b11), s1 = rsq_nr(q1);
      const double l11 = q1 * s1, l21 = fma(-l20, l10, b21) * s1, l31 = fma(-l30, l10, b31) * s1;
      const double q2 = fma(-l21, l21, fma(-l20, l20, b22)), s2 = rsq_nr(q2);
      const double l22 = q2 * s2, l32 = fma(-l31, l21, fma(-l30, l20, b32)) * s2;
      const double q3 = fma(-l32, l32, fma(-l31, l31, fma(-l30, l30, b33))), s3 = rsq_nr(q3);
      const double l33 = q3 * s3;
      double x0, x1, x2, x3;
      if (i >= d0 + 4) {
        x0 = pub[i][0] * s0;
        x1 = fma(-x0, l10, pub[i][1]) * s1;
        x2 = fma(-x1, l21, fma(-x0, l20, pub[i][2])) * s2;
        x3 = fma(-x2, l32, fma(-x1, l31, fma(-x0, l30, pub[i][3]))) * s3;
      } else {
        const int rr = i - d0;  // < 0 above the group: zeros
        x0 = rr == 0 ? l00 : (rr == 1 ? l10 : (rr == 2 ? l20 : (rr == 3 ? l30 : 0.0)));
        x1 = rr == 1 ? l11 : (rr == 2 ? l21 : (rr == 3 ? l31 : 0.0));
        x2 = rr == 2 ? l22 : (rr == 3 ? l32 : 0.0);
        x3 = rr == 3 ? l33 : 0.0;
      }
      sm.u.g.lc[i][0] = x0;
      sm.u.g.lc[i][1] = x1;
      sm.u.g.lc[i][2] = x2;
      sm.u.g.lc[i][3] = x3;
      sm.lf[i][d0] = x0;
      sm.lf[i][d0 + 1] = x1;
      sm.lf[i][d0 + 2] = x2;
      sm.lf[i][d0 + 3] = x3;
      if (i == 0) {
        sm.piv[d0] = q0;
        sm.piv[d0 + 1] = q1;
        sm.piv[d0 + 2] = q2;
        sm.piv[d0 + 3] = q3;
      }
    }
    __syncthreads();
    // rank-4 update a[i][k] -= sum_c L[i][d0+c] L[k][d0+c] of the tiles not yet finished
    const double af = -sm.u.g.lc[16 * w + cl][kq];
#pragma unroll
    for (int t = tg; t < 4; ++t) acc[t] = Mfma<double>::run(af, sm.u.g.lc[16 * t + cl][kq], acc[t]);
  }
  __syncthreads();  // pub/lc are dead; tsc (same storage) is used below
  // inverse of the diagonal tile of wave w: quad c solves column c; lane q keeps the
  // right-hand side of rows 4u + q of the tile
  {
    const int c = lane >> 2, q = lane & 3, o = 16 * w;
    double rhs[4], xv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      rhs[u] = (4 * u + q == c) ? 1.0 : 0.0;
      xv[u] = 0.0;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ur = r >> 2, qr = r & 3;
      double x = quad_bcast(rhs[ur] * rcp_nr(sm.lf[o + r][o + r]), qr);  // valid in lane qr
      x = (r < c) ? 0.0 : x;
      xv[ur] = (q == qr) ? x : xv[ur];
#pragma unroll
      for (int u = 0; u < 4; ++u) rhs[u] = fma(-sm.lf[o + 4 * u + q][o + r], x, rhs[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) sm.xf[o + 4 * u + q][o + c] = xv[u];
  }
  __syncthreads();
  // tiles below the diagonal, by distance d: wave w < 4 - d handles tile (w + d, w)
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int ti = w + d, tj = w;
      acc_t t = acc_t{0, 0, 0, 0};
#pragma unroll
      for (int tk = tj; tk < ti; ++tk)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          t = Mfma<double>::run(sm.lf[16 * ti + cl][16 * tk + 4 * s4 + kq],
                                sm.xf[16 * tk + 4 * s4 + kq][16 * tj + cl], t);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.tsc[w][Mfma<double>::row(lane, e)][cl] = t[e];
      __asm__ volatile("" ::: "memory");  // same wave: LDS keeps program order
      acc_t x = acc_t{0, 0, 0, 0};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        x = Mfma<double>::run(-sm.xf[16 * ti + cl][16 * ti + 4 * s4 + kq],
                              sm.u.tsc[w][4 * s4 + kq][cl], x);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sm.xf[16 * ti + Mfma<double>::row(lane, e)][16 * tj + cl] = x[e];
    }
    __syncthreads();
  }
}

// Loads and stores of the Cholesky steps.  Inside one launch per step plain cached
// accesses suffice (the launch boundary makes the previous step's results visible); the
// persistent kernel below passes DEV = true: data that other workgroups of the same launch
// write is then read and written at device scope, past the per-XCD L2s, which are not
// coherent with each other.
constexpr int kDevAux = 16;  // buffer cache policy: device-coherent
template <bool DEV>
__device__ inline double ld(rsrc_t r, uint32_t elem) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, elem * 8u, 0, DEV ? kDevAux : 0);
  return __hiloint2double((int)v[1], (int)v[0]);
}
template <bool DEV>
__device__ inline void st(double* p, double v) {
  if (DEV)
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                       (unsigned long long)__double_as_longlong(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// The trailing update of one tile by one panel: A_ij -= L_ik L_jk^T (all 64 x 64 tiles of
// the reversed matrix, k = panel block column).
template <bool DEV>
__device__ inline void chol_bulk(int64_t p, int k, int i, int j, double* Ar,
                                 TileSmem<double>& sm) {
  const int64_t ri = (int64_t)i * NB, cj = (int64_t)j * NB, ck = (int64_t)k * NB;
  const int M = (p - ri) < NB ? (int)(p - ri) : NB;
  const int N = (p - cj) < NB ? (int)(p - cj) : NB;
  if (!DEV) {
    tile_gemm<double, false, true>(Ar + ri * p + ck, p, Ar + cj * p + ck, p, Ar + ri * p + cj, p,
                                   M, N, 0, NB, -1.0, 1.0, sm);
    return;
  }
  // the same product with device-scope accesses: both operands i-major 64 x 64, staged
  // k-major through LDS in two chunks
  typedef Mfma<double>::acc_t acc_t;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = w >> 1, wc = w & 1, kr = lane >> 4, cl = lane & 15;
  const rsrc_t ra = make_rsrc(Ar + ri * p + ck, ((int64_t)(M - 1) * p + NB) * 8);
  const rsrc_t rb = make_rsrc(Ar + cj * p + ck, ((int64_t)(N - 1) * p + NB) * 8);
  const rsrc_t rc = make_rsrc(Ar + ri * p + cj, ((int64_t)(M - 1) * p + N) * 8);
  acc_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = acc_t{0, 0, 0, 0};
  const int i4 = tid >> 2, k8 = (tid & 3) * 8;
  double va[2][8], vb[2][8], old[2][2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      va[h][u] = ld<true>(ra, (uint32_t)((int64_t)i4 * p + 32 * h + k8 + u));
      vb[h][u] = ld<true>(rb, (uint32_t)((int64_t)i4 * p + 32 * h + k8 + u));
    }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = 32 * wr + 16 * a + Mfma<double>::row(lane, e), jj = 32 * wc + 16 * b + cl;
        old[a][b][e] = ld<true>(rc, (uint32_t)((int64_t)ii * p + jj));
      }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sm.a[k8 + u][i4] = va[h][u];
      sm.b[k8 + u][i4] = vb[h][u];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKc; kk += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = sm.a[kk + kr][32 * wr + 16 * t + cl];
        bv[t] = sm.b[kk + kr][32 * wc + 16 * t + cl];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = Mfma<double>::run(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = 32 * wr + 16 * a + Mfma<double>::row(lane, e), jj = 32 * wc + 16 * b + cl;
        if (ii < M && jj < N) st<true>(&Ar[(ri + ii) * p + cj + jj], old[a][b][e] - acc[a][b][e]);
      }
}

// The panel step of row tile i of block column s: subtract the previous panel's
// contribution from the diagonal tile (s, s) and tile (i, s), factor (s, s) (every row
// tile does this identically, so none waits for another), then the diagonal row tile
// writes L_ss and X_ss = L_ss^-1 and the others solve L_is = A_is X_ss^T.
template <bool DEV>
__device__ inline void chol_crit(int64_t p, int s, int i, double* Ar, double* X, int* info,
                                 int side_code, BlockSmem& sm) {
  typedef Mfma<double>::acc_t acc_t;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, cl = lane & 15, kq = lane >> 4;
  const int64_t r0 = (int64_t)s * NB, ri = (int64_t)i * NB;
  const int nv = (p - r0) < NB ? (int)(p - r0) : NB;  // rows/columns of block s
  const int mi = (p - ri) < NB ? (int)(p - ri) : NB;  // rows of tile i
  const bool diag = i == s;
  acc_t acc[4], pt[4];
  {
    // all loads in flight together; entries outside the matrix read as zero.  The
    // previous panel's tiles (s, s-1) and (i, s-1) are staged in lf / xf.
    const rsrc_t rd = make_rsrc(Ar + r0 * p + r0, ((int64_t)(nv - 1) * p + nv) * 8);
    const rsrc_t rp = make_rsrc(Ar + ri * p + r0, ((int64_t)(mi - 1) * p + nv) * 8);
    double v[4][4], u[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + Mfma<double>::row(lane, e), k = 16 * t + cl;
        v[t][e] = ld<DEV>(rd, (uint32_t)(r * p + k));
        u[t][e] = diag ? 0.0 : ld<DEV>(rp, (uint32_t)(r * p + k));
      }
    if (s > 0) {
      const int64_t cp = (int64_t)(s - 1) * NB;  // block column s-1 is full width
      const rsrc_t rs = make_rsrc(Ar + r0 * p + cp, ((int64_t)(nv - 1) * p + NB) * 8);
      const rsrc_t rq = make_rsrc(Ar + ri * p + cp, ((int64_t)(mi - 1) * p + NB) * 8);
      double a1[16], a2[16];
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int idx = tid + 256 * it, r = idx >> 6, k = idx & 63;
        a1[it] = ld<DEV>(rs, (uint32_t)(r * p + k));
        a2[it] = diag ? 0.0 : ld<DEV>(rq, (uint32_t)(r * p + k));
      }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int idx = tid + 256 * it, r = idx >> 6, k = idx & 63;
        sm.lf[r][k] = a1[it];
        sm.xf[r][k] = a2[it];
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + Mfma<double>::row(lane, e), k = 16 * t + cl;
        acc[t][e] = (r < nv && k < nv) ? (k <= r ? v[t][e] : 0.0) : (r == k ? 1.0 : 0.0);
        pt[t][e] = u[t][e];
      }
  }
  if (s > 0) {
    __syncthreads();
    // A_ss -= L_s,s-1 L_s,s-1^T and A_is -= L_i,s-1 L_s,s-1^T (rows of L past the matrix
    // are zero, so the identity padding stays)
#pragma unroll
    for (int ks = 0; ks < NB / 4; ++ks) {
      const double as = -sm.lf[16 * w + cl][4 * ks + kq];
      const double ai = -sm.xf[16 * w + cl][4 * ks + kq];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const double b = sm.lf[16 * t + cl][4 * ks + kq];
        acc[t] = Mfma<double>::run(as, b, acc[t]);
        if (!diag) pt[t] = Mfma<double>::run(ai, b, pt[t]);
      }
    }
    __syncthreads();  // the staging is consumed before the factorisation reuses lf / xf
  }
  chol_inv_block(acc, sm);
  if (diag) {
    if (tid < 64) {  // first non-positive (or NaN) pivot, found by one wave
      const bool bad = tid < nv && !(sm.piv[tid] > 0.0);
      const unsigned long long mask = __ballot(bad);
      if (tid == 0 && mask != 0ull)
        record_info(info, side_code, (int)(r0 + __ffsll((long long)mask)));
    }
    for (int idx = tid; idx < NB * NB; idx += 256) {
      const int r = idx >> 6, k = idx & 63;
      if (r < nv && k < nv) {
        // (L_ss itself is read by nothing later; in the persistent kernel other panel
        // steps of this block column may still be reading the tile, so it stays)
        if (!DEV && k <= r) st<DEV>(&Ar[(r0 + r) * p + r0 + k], sm.lf[r][k]);
        st<DEV>(&X[(r0 + r) * p + r0 + k], sm.xf[r][k]);
      }
    }
    return;
  }
  // L_is = A_is X_ss^T: A_is goes through lf (free after the factorisation)
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.lf[16 * w + Mfma<double>::row(lane, e)][16 * t + cl] = pt[t][e];
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    acc_t o = acc_t{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < NB / 4; ++ks)
      o = Mfma<double>::run(sm.lf[16 * w + cl][4 * ks + kq], sm.xf[16 * t + cl][4 * ks + kq], o);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * w + Mfma<double>::row(lane, e), k = 16 * t + cl;
      if (r < mi && k < nv) st<DEV>(&Ar[(ri + r) * p + r0 + k], o[e]);
    }
  }
}

// One step s of the blocked right-looking Cholesky of the reversed matrix, in one launch.
//  * Workgroups 0 .. nblk-s-1 ("critical"): workgroup c runs the panel step of row tile
//    i = s + c of block column s (chol_crit).
//  * The remaining workgroups ("bulk") apply the previous panel to the trailing tiles
//    (i, j), s < j <= i: A_ij -= L_i,s-1 L_j,s-1^T.
// So the panel chain and the bulk trailing update of the previous step share a launch.
__global__ __launch_bounds__(256, 2) void k_chol_step(int64_t p, int s, double* __restrict__ Ar,
                                                      double* __restrict__ X, int* info,
                                                      int side_code) {
  __shared__ union {
    BlockSmem b;
    TileSmem<double> t;
  } sh;
  const int nblk = (int)((p + NB - 1) / NB);
  const int crit = nblk - s;
  if ((int)blockIdx.x >= crit) {
    const int rest = nblk - s - 1, idx = (int)blockIdx.x - crit;
    const int bi = idx / rest, bj = idx % rest;
    if (bj > bi) return;
    chol_bulk<false>(p, s - 1, s + 1 + bi, s + 1 + bj, Ar, sh.t);
    return;
  }
  chol_crit<false>(p, s, s + (int)blockIdx.x, Ar, X, info, side_code, sh.b);
}

// ---------------------------------------------------------------------------
// The whole blocked Cholesky of one or two matrices as one persistent kernel
// ---------------------------------------------------------------------------
// The per-step launches above serialise the panel chain with a launch boundary per step.
// Here every workgroup takes tasks from one queue in a fixed order; a task waits (bounded)
// until the tasks it depends on are done, so the chain of panel steps runs back to back
// while the trailing updates fill the other CUs.  Tasks of matrix q, step s:
//   bulk(s): tile (i, j), s + 1 <= j <= i, takes panel s - 1 (needs L_i,s-1 and L_j,s-1
//            and the tile's panels 0 .. s - 2; afterwards the tile has s panels);
//   crit(s): the panel step of row tile i >= s (needs L_s,s-1 and L_i,s-1 and the tiles
//            (s, s), (i, s) with panels 0 .. s - 2; afterwards (i, s) holds L_is, final).
// Group (q, s) lists bulk(s) of column s + 1 first, then crit(s), then the rest of bulk(s)
// column by column; groups go by step, the matrices alternating.  Every task depends only
// on earlier tasks, so the queue always drains.
constexpr int kMaxChol = 2;
struct CholMat {
  int64_t p;
  int nblk, side_code;
  double* Ar;
  double* X;
  int* tile_cnt;   // [nblk * nblk] panels applied to each tile by bulk tasks (kFinal: L)
};
struct CholArgs {
  CholMat mat[kMaxChol];
  int nmat, maxn;
  int64_t total;  // tasks of the steps [s0, s1) of this launch
  int64_t toff;   // tasks of all matrices before step s0
  int* ctl;  // [0] next task, [32] abort
  int* info;
};
constexpr int kCholSpin = 1 << 20;
constexpr int kFinal = 1 << 24;  // tile counter of a panel tile whose L is written

// Tasks in group (q, s): n - s - 1 + n - s + (n - s - 2)(n - s - 1) / 2 = u (u + 1) / 2 with
// u = n - s for s >= 1, and n for s = 0 (panel steps only).  Tasks of one matrix before
// step S: n + sum_{u = n-S+1}^{n-1} u (u + 1) / 2 = n + T(n - 1) - T(n - S), T(k) =
// k (k + 1) (k + 2) / 6.
__host__ __device__ inline int64_t chol_tet(int64_t k) { return k * (k + 1) * (k + 2) / 6; }
__host__ __device__ inline int64_t chol_group_size(int n, int s) {
  const int64_t u = n - s;
  return s == 0 ? n : u * (u + 1) / 2;
}
__host__ __device__ inline int64_t chol_before(int n, int S) {
  if (S <= 0) return 0;
  if (S > n) S = n;
  return n + chol_tet(n - 1) - chol_tet(n - S);
}

// whole-wave bounded wait until *cnt >= v (false after an abort or a timeout)
__device__ inline bool chol_wait(const int* cnt, int v, int* ctl, int* info) {
  for (int it = 0;; ++it) {
    const int x = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (x >= v) return true;
    if ((it & 15) == 15) {
      if (__hip_atomic_load(ctl + 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
        return false;
      if (it > kCholSpin) {
        if ((threadIdx.x & 63) == 0 && atomicCAS(ctl + 32, 0, 1) == 0) record_info(info, 4, 0);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

__global__ __launch_bounds__(256, 2) void k_chol_persistent(CholArgs a) {
  __shared__ union {
    BlockSmem b;
    TileSmem<double> t;
  } sh;
  __shared__ int task[4];  // kind, matrix, row tile, step << 16 | column tile
  const int tid = threadIdx.x, lane = tid & 63;
  // Every branch on the wave index is on a wave-uniform value, so that the compiler emits
  // scalar branches: a barrier inside lane-divergent control flow would be reached a
  // different number of times by different waves.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (;;) {
    if (w == 0) {
      // wave 0 claims the next task (lane 0's atomic, broadcast) and decodes it
      int tl = 0;
      if (lane == 0) {
        const bool ab =
            __hip_atomic_load(a.ctl + 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
        tl = ab ? -1 : atomicAdd(a.ctl, 1);
      }
      tl = __builtin_amdgcn_readfirstlane(tl);
      const int64_t t = (tl < 0 ? a.total : (int64_t)(unsigned)tl) + a.toff;
      int kind = -1, q = 0, s = 0, i = 0, j = 0;
      if (t < a.total + a.toff) {
        // the step: last s with (tasks of all matrices before step s) <= t
        const int n0 = a.mat[0].nblk, n1 = a.nmat > 1 ? a.mat[1].nblk : 0;
        int lo = 0, hi = a.maxn - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (chol_before(n0, mid) + chol_before(n1, mid) <= t) lo = mid;
          else hi = mid - 1;
        }
        s = lo;
        int64_t r = t - chol_before(n0, s) - chol_before(n1, s);
        if (s < n0 && r < chol_group_size(n0, s)) {
          q = 0;
        } else {
          if (s < n0) r -= chol_group_size(n0, s);
          q = 1;
        }
        const int n = q == 0 ? n0 : n1;
        int k = (int)r;
        const int c1 = s >= 1 ? n - s - 1 : 0, c2 = n - s;
        if (k < c1) {
          kind = 0;
          i = s + 1 + k;
          j = s + 1;
        } else if (k < c1 + c2) {
          kind = 1;
          i = s + (k - c1);
        } else {
          kind = 0;
          k -= c1 + c2;
          j = s + 2;
          while (k >= n - j && j < n) {
            k -= n - j;
            ++j;
          }
          i = j + k;
        }
      }
      if (lane == 0) {
        task[0] = kind;
        task[1] = q;
        task[2] = i;
        task[3] = (s << 16) | j;
      }
    }
    __syncthreads();
    const int kind = __builtin_amdgcn_readfirstlane(task[0]);
    const int q = __builtin_amdgcn_readfirstlane(task[1]);
    const int i = __builtin_amdgcn_readfirstlane(task[2]);
    const int sj = __builtin_amdgcn_readfirstlane(task[3]);
    const int s = sj >> 16, j = sj & 0xFFFF;
    __syncthreads();  // task[] is rewritten by the next claim
    if (kind < 0) return;
    // select the matrix with branches (a runtime index into the kernel argument would
    // copy it to scratch memory)
    const CholMat m = q == 0 ? a.mat[0] : a.mat[1];
    const int64_t p = m.p;
    const int n = m.nblk;
    // dependencies (wave 0 waits, the barrier releases the others)
    if (w == 0) {
      // the panel tiles this task reads are final (kFinal), and its own tiles carry panels
      // 0 .. s - 2; every task polls only the few tiles it reads, so the waiters of one
      // step spread over many words
      const int* tc = m.tile_cnt;
      const int r2 = kind == 0 ? j : s;  // the second panel row read
      bool ok = true;
      if (s >= 1) {
        ok = chol_wait(tc + (int64_t)i * n + (s - 1), kFinal, a.ctl, a.info);
        if (ok && r2 != i) ok = chol_wait(tc + (int64_t)r2 * n + (s - 1), kFinal, a.ctl, a.info);
      }
      if (ok && kind == 0) ok = chol_wait(tc + (int64_t)i * n + j, s - 1, a.ctl, a.info);
      if (ok && kind == 1 && s >= 2) {
        ok = chol_wait(tc + (int64_t)s * n + s, s - 1, a.ctl, a.info);
        if (ok && i != s) ok = chol_wait(tc + (int64_t)i * n + s, s - 1, a.ctl, a.info);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __syncthreads();
    if (kind == 0)
      chol_bulk<true>(p, s - 1, i, j, m.Ar, sh.t);
    else
      chol_crit<true>(p, s, i, m.Ar, m.X, a.info, m.side_code, sh.b);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (w == 0 && lane == 0)
      __hip_atomic_store(m.tile_cnt + (int64_t)i * n + (kind == 0 ? j : s), kind == 0 ? s : kFinal,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Recursive doubling, step 1: T = L21 X11 for every pair of h-blocks (group z).
// X11 is lower triangular, so column tile tj only needs k >= 64*tj.
__global__ __launch_bounds__(256) void k_trtri_step1(int64_t p, int64_t h, int zoff,
                                                     const double* Ar, const double* X, double* Tb,
                                                     int64_t ldt) {
  __shared__ TileSmem<double> sm;
  const int64_t g0 = (int64_t)(blockIdx.z + zoff) * 2 * h;
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
__global__ __launch_bounds__(256) void k_trtri_step2(int64_t p, int64_t h, int zoff, double* X,
                                                     const double* Tb, int64_t ldt) {
  __shared__ TileSmem<double> sm;
  const int64_t g0 = (int64_t)(blockIdx.z + zoff) * 2 * h;
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
  double* Tb;
  int64_t ldt;
  double* Tt;  // the top doubling level's T (rows ldt .. p-1, ldt wide): computed while the
               // lower levels of the trailing block, which reuse Tb, are still to come
  int* sync;   // persistent Cholesky: control words, then its counters (chol_sync_ints)
};

// ints of the persistent Cholesky's sync area: 64 control words, then the tile counters
int64_t chol_sync_ints(int64_t p) {
  const int64_t nb = cdiv(p, NB);
  return 64 + nb * nb;
}

// Largest half-size used by the recursive doubling (the leading dimension of T).
int64_t trtri_ldt(int64_t p) {
  int64_t h = NB;
  while (2 * h < p) h *= 2;
  return h;
}

FactorWs carve(int64_t p, void* ws) {
  FactorWs f;
  char* c = (char*)ws;
  f.ldt = trtri_ldt(p);
  f.Ar = (double*)c;
  c += align_up((size_t)p * p * sizeof(double));
  f.X = (double*)c;
  c += align_up((size_t)p * p * sizeof(double));
  f.Tb = (double*)c;
  c += align_up((size_t)p * f.ldt * sizeof(double));
  f.Tt = (double*)c;
  c += align_up((size_t)(p > f.ldt ? p - f.ldt : 1) * f.ldt * sizeof(double));
  f.sync = (int*)c;
  return f;
}

}  // namespace

size_t factor_workspace(int64_t p) {
  const int64_t ldt = trtri_ldt(p);
  return 2 * align_up((size_t)p * p * sizeof(double)) + align_up((size_t)p * ldt * sizeof(double)) +
         align_up((size_t)(p > ldt ? p - ldt : 1) * ldt * sizeof(double)) +
         align_up((size_t)chol_sync_ints(p) * sizeof(int));
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

namespace {

// The launches of one factorisation, in order: reversal, one per Cholesky step, one per
// doubling level of the inverse (two kernels), finalisation.
struct FactorPlan {
  int64_t p;
  int dtype;
  const void* A;
  void* U;
  FactorWs f;
  int* info;
  int side_code;
  hipStream_t s;
  int nblk, nlev;
  int stages() const { return 1 + nblk + nlev + 1; }
};

FactorPlan plan(int64_t p, int dtype, const void* A, void* U, void* ws, int* info, int side_code,
                hipStream_t s) {
  FactorPlan q{p, dtype, A, U, carve(p, ws), info, side_code, s, (int)cdiv(p, NB), 0};
  for (int64_t h = NB; h < p; h *= 2) ++q.nlev;
  return q;
}

// One doubling level of the inverse over the groups [z0, z1) of width 2h: step 1
// (T = L21 X11) if bit 0 of `steps` is set, step 2 (X21 = -X22 T) if bit 1 is.  The top
// level (h == ldt) keeps T in its own buffer.
void trtri_level(const FactorPlan& q, int64_t h, int z0, int z1, int steps) {
  if (z1 <= z0) return;
  const int64_t p = q.p;
  FactorWs f = q.f;
  // (T rows are addressed by their absolute index g0 + h + ..., >= ldt at the top level)
  if (h == f.ldt) f.Tb = (double*)((char*)f.Tt - (size_t)f.ldt * f.ldt * sizeof(double));
  const dim3 g((unsigned)cdiv(h, NB), (unsigned)cdiv(h, NB), (unsigned)(z1 - z0));
  double f1 = 0.0, f2 = 0.0;
  if (prof_on()) trtri_flops(p, h, &f1, &f2);
  const double frac = (double)(z1 - z0) / (double)cdiv(p, 2 * h);  // (measurement only)
  prof_begin(KC_TRTRI, q.s);
  if (steps & 1) k_trtri_step1<<<g, 256, 0, q.s>>>(p, h, z0, f.Ar, f.X, f.Tb, f.ldt);
  if (steps & 2) k_trtri_step2<<<g, 256, 0, q.s>>>(p, h, z0, f.X, f.Tb, f.ldt);
  prof_end(KC_TRTRI, q.s, frac * (((steps & 1) ? f1 : 0.0) + ((steps & 2) ? f2 : 0.0)),
           frac * 8.0 * 2.0 * (double)h * (double)p * (((steps & 1) ? 1 : 0) + ((steps & 2) ? 1 : 0)));
}

void stage(const FactorPlan& q, int idx) {
  const int64_t p = q.p;
  const bool pr = prof_on();
  const double es = q.dtype == 0 ? 4.0 : 8.0, pp = (double)p * (double)p;
  hipStream_t s = q.s;
  const FactorWs& f = q.f;
  const dim3 eg((unsigned)cdiv(p, 64), (unsigned)cdiv(p, 4));
  if (idx == 0) {
    prof_begin(KC_OTHER, s);
    if (q.dtype == 0)
      k_reverse_sym<float><<<eg, 256, 0, s>>>(p, (const float*)q.A, f.Ar);
    else
      k_reverse_sym<double><<<eg, 256, 0, s>>>(p, (const double*)q.A, f.Ar);
    prof_end(KC_OTHER, s, 0.0, pp * (es + 8.0));
    return;
  }
  if (idx <= q.nblk) {
    const int st = idx - 1;
    const int crit = q.nblk - st, rest = q.nblk - st - 1;
    const unsigned grid = (unsigned)(crit + (st > 0 ? rest * rest : 0));
    double fl = 0.0, by = 0.0;
    if (pr) {
      const double nv = (double)((p - st * NB) < NB ? (p - st * NB) : NB);
      const double rows = (double)(p - (int64_t)st * NB) - nv;
      fl = 2.0 / 3.0 * nv * nv * nv + 2.0 * rows * nv * nv +
           (st > 0 ? trailing_flops(p, st - 1) : 0.0);
      const double trail = st > 0 ? (rows + nv) * (rows + nv + NB) / 2.0 : 0.0;
      by = 8.0 * (3.0 * (rows + nv) * NB + 3.0 * trail);
    }
    prof_begin(KC_POTRF, s);
    k_chol_step<<<grid, 256, 0, s>>>(p, st, f.Ar, f.X, q.info, q.side_code);
    prof_end(KC_POTRF, s, fl, by);
    return;
  }
  if (idx <= q.nblk + q.nlev) {
    const int64_t h = (int64_t)NB << (idx - q.nblk - 1);
    trtri_level(q, h, 0, (int)cdiv(p, 2 * h), 3);
    return;
  }
  prof_begin(KC_OTHER, s);
  if (q.dtype == 0)
    k_finalize<float><<<eg, 256, 0, s>>>(p, f.X, (float*)q.U);
  else
    k_finalize<double><<<eg, 256, 0, s>>>(p, f.X, (double*)q.U);
  prof_end(KC_OTHER, s, 0.0, pp * (8.0 / 2.0 + es));
}

}  // namespace

// control words and counters start at zero (a fill kernel: the call may be captured)
__global__ __launch_bounds__(256) void k_zero_ints(int* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

// Steps [s0, s1) of the Cholesky of one or two matrices (plans qs[0..nmat)) as one
// persistent launch on s, on at most `per_cu` workgroups per CU.  The first launch
// (s0 == 0) clears the counters; a later one only the task counter and abort flag.
hipError_t chol_persistent_enqueue(const FactorPlan* const* qs, int nmat, int s0, int s1,
                                   int per_cu, int* info, hipStream_t s) {
  CholArgs a{};
  a.nmat = nmat;
  a.maxn = 0;
  a.total = 0;
  a.toff = 0;
  double fl = 0.0, by = 0.0;
  const bool pr = prof_on();
  for (int q = 0; q < nmat; ++q) {
    const FactorPlan& pl = *qs[q];
    const int nb = (int)cdiv(pl.p, NB);
    a.mat[q].p = pl.p;
    a.mat[q].nblk = nb;
    a.mat[q].side_code = pl.side_code;
    a.mat[q].Ar = pl.f.Ar;
    a.mat[q].X = pl.f.X;
    a.mat[q].tile_cnt = pl.f.sync + 64;
    a.maxn = nb > a.maxn ? nb : a.maxn;
    a.total += chol_before(nb, s1) - chol_before(nb, s0);
    a.toff += chol_before(nb, s0);
    const int64_t words = s0 == 0 ? chol_sync_ints(pl.p) : (q == 0 ? 64 : 0);
    const int64_t zg = cdiv(words, 256) < 1024 ? cdiv(words, 256) : 1024;
    if (words > 0) k_zero_ints<<<(unsigned)zg, 256, 0, s>>>(pl.f.sync, words);
    if (pr) {
      const int64_t p = pl.p;
      for (int st = s0; st < (s1 < nb ? s1 : nb); ++st) {
        const double nv = (double)((p - st * NB) < NB ? (p - st * NB) : NB);
        const double rows = (double)(p - (int64_t)st * NB) - nv;
        fl += 2.0 / 3.0 * nv * nv * nv + 2.0 * rows * nv * nv +
              (st > 0 ? trailing_flops(p, st - 1) : 0.0);
        const double trail = st > 0 ? (rows + nv) * (rows + nv + NB) / 2.0 : 0.0;
        by += 8.0 * (3.0 * (rows + nv) * NB + 3.0 * trail);
      }
    }
  }
  a.ctl = qs[0]->f.sync;
  a.info = info;
  int dev = 0, ncu = 0, occ = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_chol_persistent, 256, 0)) !=
      hipSuccess)
    return e;
  if (occ < 1) return hipErrorInvalidConfiguration;
  if (occ > per_cu) occ = per_cu;
  prof_begin(KC_POTRF, s);
  k_chol_persistent<<<ncu * occ, 256, 0, s>>>(a);
  prof_end(KC_POTRF, s, fl, by);
  return hipGetLastError();
}

hipError_t factor_enqueue(int64_t p, int dtype, const void* A, void* U, void* ws, int* info,
                          int side_code, hipStream_t s) {
  const FactorPlan q = plan(p, dtype, A, U, ws, info, side_code, s);
  stage(q, 0);
  const FactorPlan* qs[1] = {&q};
  hipError_t e = chol_persistent_enqueue(qs, 1, 0, q.nblk, 2, info, s);
  if (e != hipSuccess) return e;
  for (int i = q.nblk + 1; i < q.stages(); ++i) stage(q, i);
  return hipGetLastError();
}

hipError_t factor_pair_enqueue(int64_t m, const void* A, void* Ua, void* ws_a, hipStream_t sa,
                               int64_t n, const void* B, void* Ub, void* ws_b, hipStream_t sb,
                               int dtype, int* info) {
  // Reversal of each on its stream; both Cholesky factorisations together in persistent
  // launches on sa; the inverses and the finalisation of each on its stream again.  The
  // Cholesky is split at step S = H / 64, H = the inverse's top-level half-size: once
  // block columns < S are final, the inverse of the leading H x H block and the product
  // T = L21 X11 of the top level need nothing else, so they run on sb while the rest of
  // the Cholesky (a dependency chain that leaves most CUs idle) runs on sa with one
  // workgroup per CU.
  const FactorPlan qa = plan(m, dtype, A, Ua, ws_a, info, 1, sa);
  const FactorPlan qb = plan(n, dtype, B, Ub, ws_b, info, 2, sb);
  hipStream_t aux = nullptr;
  hipEvent_t* ev = nullptr;
  hipError_t e = aux_resources(kAuxEvents, &aux, &ev);
  if (e != hipSuccess) return e;
  stage(qa, 0);
  stage(qb, 0);
  if ((e = hipEventRecord(ev[3], sb)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sa, ev[3], 0)) != hipSuccess) return e;
  const FactorPlan* qs[2] = {&qa, &qb};
  const FactorPlan* pl[2] = {&qa, &qb};
  const int maxn = qa.nblk > qb.nblk ? qa.nblk : qb.nblk;
  // split step: the smallest H / 64 of the matrices that have an inverse to compute
  int S = maxn;
  for (int k = 0; k < 2; ++k)
    if (pl[k]->nlev > 0 && (int)(pl[k]->f.ldt / NB) < S) S = (int)(pl[k]->f.ldt / NB);
  bool early[2];
  for (int k = 0; k < 2; ++k) early[k] = pl[k]->nlev > 0 && pl[k]->f.ldt / NB <= S && S < maxn;
  if ((e = chol_persistent_enqueue(qs, 2, 0, S, 2, info, sa)) != hipSuccess) return e;
  if ((e = hipEventRecord(ev[2], sa)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sb, ev[2], 0)) != hipSuccess) return e;
  // sb: the leading blocks' inverse levels and the top level's step 1 of each matrix
  for (int k = 0; k < 2; ++k) {
    if (!early[k]) continue;
    FactorPlan q = *pl[k];
    q.s = sb;
    const int64_t H = q.f.ldt;
    for (int64_t h = NB; h < H; h *= 2) trtri_level(q, h, 0, (int)(H / (2 * h)), 3);
    trtri_level(q, H, 0, 1, 1);
  }
  if ((e = hipEventRecord(ev[4], sb)) != hipSuccess) return e;
  if (S < maxn) {
    if ((e = chol_persistent_enqueue(qs, 2, S, maxn, 1, info, sa)) != hipSuccess) return e;
  }
  if ((e = hipEventRecord(ev[5], sa)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sa, ev[4], 0)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sb, ev[5], 0)) != hipSuccess) return e;
  // the rest of each inverse and the finalisation, A on sa and B on sb
  for (int k = 0; k < 2; ++k) {
    FactorPlan q = *pl[k];
    q.s = k == 0 ? sa : sb;
    if (early[k]) {
      const int64_t H = q.f.ldt;
      for (int64_t h = NB; h < H; h *= 2)
        trtri_level(q, h, (int)(H / (2 * h)), (int)cdiv(q.p, 2 * h), 3);
      trtri_level(q, H, 0, 1, 2);
    } else {
      for (int i = q.nblk + 1; i <= q.nblk + q.nlev; ++i) stage(q, i);
    }
    stage(q, q.nblk + q.nlev + 1);
  }
  return hipGetLastError();
}

}  // namespace g2d
