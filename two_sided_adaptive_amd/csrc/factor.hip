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
//            64-wide steps)
//   X = L^-1 by 64-row blocks: X_ii = L_ii^-1 with the diagonal block's factorisation,
//            X_is = -X_ii sum_{s<=k<i} L_ik X_ks below it, as soon as L's row block i is
//            final; both in one persistent launch
//   U = J X J is the upper Cholesky factor of A^-1; U'[i][j] = U[i][j] / U[i][i].
// Diagonal-block inverses double as the panel solve: L21 = A21 (L11^-1)^T is a GEMM.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "prof.hpp"
#include "schedule.hpp"

namespace g2d {
namespace {

constexpr int NB = 64;  // panel width = tile edge

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
      double pub[2][NB][4];  // the group's four columns, current values (by group parity)
      double lc[4][NB][4];   // per wave: the group's four columns of L, every row
    } g;
    double tsc[4][16][18];  // per-wave 16x16 temporaries of the inverse
  } u;
  double piv[NB];  // pivots before the square root (SPD check)
};

// Cholesky and inverse of one 64x64 diagonal block held in MFMA accumulator layout by
// the four waves of the workgroup (wave w: rows 16w..16w+15, acc[t] the 16x16 tile of
// columns 16t..16t+15; only the lower triangle is read; padding rows/columns hold the
// identity).  Leaves L in sm.lf and X = L^-1 in sm.xf; ends with a barrier.
//  * Cholesky, four columns at a time: the group's columns are published to LDS; every
//    wave factors the 4x4 diagonal block and solves the four L entries of all 64 rows
//    (lane i: row i), so that it has every operand of its rank-4 update (one MFMA per
//    tile of its own rows) in its own LDS area, and one barrier per group suffices (the
//    published columns alternate between two buffers).
//  * Inverse by 16x16 tiles: wave t inverts diagonal tile t by forward substitution
//    (quad c solves column c, the new entry broadcast inside the quad with DPP); the
//    tiles below follow by distance, X_ij = -X_ii (sum_{j<=k<i} L_ik X_kj), with MFMA.
__device__ inline void chol_inv_block(Mfma<double>::acc_t (&acc)[4], BlockSmem& sm) {
  typedef Mfma<double>::acc_t acc_t;
  const int tid = threadIdx.x, lane = tid & 63, cl = lane & 15, kq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int idx = tid; idx < NB * NB; idx += 256) sm.xf[idx >> 6][idx & 63] = 0.0;
#pragma unroll
  for (int g = 0; g < NB / 4; ++g) {
    const int tg = g >> 2, cg = 4 * (g & 3), d0 = 4 * g, pb = g & 1;
    if (cl >= cg && cl < cg + 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sm.u.g.pub[pb][16 * w + Mfma<double>::row(lane, e)][cl - cg] = acc[tg][e];
    }
    __syncthreads();
    {
      const int i = lane;
      const double(*pub)[4] = sm.u.g.pub[pb];
      const double b00 = pub[d0][0];
      const double b10 = pub[d0 + 1][0], b11 = pub[d0 + 1][1];
      const double b20 = pub[d0 + 2][0], b21 = pub[d0 + 2][1], b22 = pub[d0 + 2][2];
      const double b30 = pub[d0 + 3][0], b31 = pub[d0 + 3][1], b32 = pub[d0 + 3][2];
      const double b33 = pub[d0 + 3][3];
      const double a0 = pub[i][0], a1 = pub[i][1], a2 = pub[i][2], a3 = pub[i][3];
      const double q0 = b00, s0 = rsq_nr(q0);
      const double l10 = b10 * s0, l20 = b20 * s0, l30 = b30 * s0;
      const double q1 = fma(-l10, l10, b11), s1 = rsq_nr(q1);
      const double l21 = fma(-l20, l10, b21) * s1, l31 = fma(-l30, l10, b31) * s1;
      const double q2 = fma(-l21, l21, fma(-l20, l20, b22)), s2 = rsq_nr(q2);
      const double l32 = fma(-l31, l21, fma(-l30, l20, b32)) * s2;
      const double q3 = fma(-l32, l32, fma(-l31, l31, fma(-l30, l30, b33))), s3 = rsq_nr(q3);
      // row i's four entries; for the group's own rows the same expressions give its L
      // entries (the diagonal one as q * rsqrt(q)); above the diagonal they are zero
      const int rr = i - d0;
      double x0 = a0 * s0;
      double x1 = fma(-x0, l10, a1) * s1;
      double x2 = fma(-x1, l21, fma(-x0, l20, a2)) * s2;
      double x3 = fma(-x2, l32, fma(-x1, l31, fma(-x0, l30, a3))) * s3;
      x0 = rr >= 0 ? x0 : 0.0;
      x1 = rr >= 1 ? x1 : 0.0;
      x2 = rr >= 2 ? x2 : 0.0;
      x3 = rr >= 3 ? x3 : 0.0;
      double* lcw = sm.u.g.lc[w][i];
      lcw[0] = x0;
      lcw[1] = x1;
      lcw[2] = x2;
      lcw[3] = x3;
      if ((i >> 4) == w) {
        sm.lf[i][d0] = x0;
        sm.lf[i][d0 + 1] = x1;
        sm.lf[i][d0 + 2] = x2;
        sm.lf[i][d0 + 3] = x3;
      }
      if (w == 0 && i == 0) {
        sm.piv[d0] = q0;
        sm.piv[d0 + 1] = q1;
        sm.piv[d0 + 2] = q2;
        sm.piv[d0 + 3] = q3;
      }
    }
    __asm__ volatile("" ::: "memory");  // same wave: LDS keeps program order
    // rank-4 update a[i][k] -= sum_c L[i][d0+c] L[k][d0+c] of this wave's tiles that are
    // not finished (columns k of tiles t in [tg, w]: the lower triangle)
    const double af = -sm.u.g.lc[w][16 * w + cl][kq];
#pragma unroll
    for (int t = tg; t < 4; ++t)
      if (t <= w) acc[t] = Mfma<double>::run(af, sm.u.g.lc[w][16 * t + cl][kq], acc[t]);
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

// Loads and stores of the Cholesky tasks.  Tiles that other workgroups of the same launch
// update are read and written at device scope (DEV = true), past the per-XCD L2s, which
// are not coherent with each other.  Final panel tiles are also copied, once, to a tiled
// buffer that nothing else writes during the launch (Lt); their many readers load them
// through the caches (DEV = false): a line of Lt can only enter a cache after the tile is
// final, so no cached copy is ever stale.
constexpr int kDevAux = 16;  // buffer cache policy: device-coherent
// elem: per-lane element offset; sbytes: a wave-uniform byte offset (a compile-time
// constant at every use, so that unrolled loads share one address register)
template <bool DEV>
__device__ inline double ld(rsrc_t r, uint32_t elem, uint32_t sbytes = 0) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, elem * 8u, sbytes, DEV ? kDevAux : 0);
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

// Lt holds the strictly lower tiles (i, k), k < i, of L, each 64 x 64 row-major and
// contiguous; rows past the matrix are never written and never read (a tile's buffer
// descriptor covers its rows only, so loads past them return zeros).
__device__ inline const double* lt_tile(const double* Lt, int i, int k) {
  return Lt + ((int64_t)i * (i - 1) / 2 + k) * (NB * NB);
}
// Xt holds the final tiles (i, s), s <= i, of X = L^-1 the same way (written once).
__device__ inline const double* xt_tile(const double* Xt, int i, int s) {
  return Xt + ((int64_t)i * (i + 1) / 2 + s) * (NB * NB);
}
__device__ inline int tile_rows(int64_t p, int i) {
  return (p - (int64_t)i * NB) < NB ? (int)(p - (int64_t)i * NB) : NB;
}

// Element (r, c) of the reversed matrix J A J, read from the lower triangle of the input
// A (fp32 or fp64, never written): A[p-1-min(r,c)][p-1-max(r,c)], zero past the matrix.
// The tasks that touch a tile first read it this way, so no reversed copy is made.
__device__ inline double ld_src(const void* A, bool f32, int64_t p, int64_t r, int64_t c) {
  if (r >= p || c >= p) return 0.0;
  const int64_t a = r > c ? r : c, b = r > c ? c : r;
  const int64_t idx = (p - 1 - b) * p + (p - 1 - a);
  return f32 ? (double)((const float*)A)[idx] : ((const double*)A)[idx];
}
// U'[a][b] of the output factor in its dtype
__device__ inline void st_u(void* U, bool f32, int64_t idx, double v) {
  if (f32)
    ((float*)U)[idx] = (float)v;
  else
    ((double*)U)[idx] = v;
}

// LDS of a trailing-update task: two stages of a 32-deep chunk of both operands, k-major.
struct BulkSmem {
  double a[2][kKc][kTile + kPad];
  double b[2][kKc][kTile + kPad];
};

// The trailing update of one tile by the panels k0 .. k1 - 1: A_ij -= sum_k L_ik L_jk^T
// (64 x 64 tiles of the reversed matrix, k = panel block column).  The tile is read once
// (from A itself when k0 = 0: no update has touched it) and written once; the panel tiles
// stream through LDS in 32-deep chunks, the next chunk's loads in flight while the current
// one is multiplied.
__device__ inline void chol_bulk(int64_t p, int k0, int k1, int i, int j, double* Ar,
                                 const double* Lt, const void* A, bool f32, BulkSmem& sm) {
  const int64_t ri = (int64_t)i * NB, cj = (int64_t)j * NB;
  const int M = tile_rows(p, i), N = tile_rows(p, j);
  typedef Mfma<double>::acc_t acc_t;
  // an opaque copy of the thread index: values derived from it are recomputed per task
  // instead of being held (and spilled) across the persistent loop
  int tid = threadIdx.x;
  __asm__ volatile("" : "+v"(tid));
  const int lane = tid & 63, w = tid >> 6;
  const int wr = w >> 1, wc = w & 1, kr = lane >> 4, cl = lane & 15;
  const rsrc_t rc = make_rsrc(Ar + ri * p + cj, ((int64_t)(M - 1) * p + N) * 8);
  const int i4 = tid >> 2, k8 = (tid & 3) * 8;
  // chunk c: half c & 1 of panel k0 + c / 2, both operands i-major 64 x 64 in Lt
  double va[8], vb[8];
  auto fetch = [&](int c) {
    const int k = k0 + (c >> 1), h = c & 1;
    const rsrc_t ra = make_rsrc(lt_tile(Lt, i, k), (int64_t)M * NB * 8);
    const rsrc_t rb = make_rsrc(lt_tile(Lt, j, k), (int64_t)N * NB * 8);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      va[u] = ld<false>(ra, (uint32_t)(i4 * NB + 32 * h + k8 + u));
      vb[u] = ld<false>(rb, (uint32_t)(i4 * NB + 32 * h + k8 + u));
    }
  };
  auto stage = [&](int st) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sm.a[st][k8 + u][i4] = va[u];
      sm.b[st][k8 + u][i4] = vb[u];
    }
  };
  acc_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = acc_t{0, 0, 0, 0};
  const int nc = 2 * (k1 - k0);
  fetch(0);
  double old[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = 32 * wr + 16 * a + Mfma<double>::row(lane, e), jj = 32 * wc + 16 * b + cl;
        old[a][b][e] = k0 == 0 ? ld_src(A, f32, p, ri + ii, cj + jj)
                               : ld<true>(rc, (uint32_t)((int64_t)ii * p + jj));
      }
  stage(0);
  if (nc > 1) fetch(1);
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    const int st = c & 1;
    if (c + 1 < nc) {
      stage(st ^ 1);  // (stage st ^ 1 was last read before the previous barrier)
      if (c + 2 < nc) fetch(c + 2);
    }
#pragma unroll
    for (int kk = 0; kk < kKc; kk += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = sm.a[st][kk + kr][32 * wr + 16 * t + cl];
        bv[t] = sm.b[st][kk + kr][32 * wc + 16 * t + cl];
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
// writes X_ss = L_ss^-1 to Xt and the diagonal block of U', and the others solve
// L_is = A_is X_ss^T and write it to Ar and Lt.  Steps 0 and 1 read their tiles from A
// (no trailing update has touched them).
// (L_ss itself is read by nothing later; other panel steps of this block column may still
// be reading tile (s, s), so it stays.)
__device__ inline void chol_crit(int64_t p, int s, int i, double* Ar, double* Lt, double* Xt,
                                 const void* A, void* U, bool f32, int* info, int side_code,
                                 BlockSmem& sm) {
  constexpr bool DEV = true;
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
        if (s <= 1) {
          v[t][e] = ld_src(A, f32, p, r0 + r, r0 + k);
          u[t][e] = diag ? 0.0 : ld_src(A, f32, p, ri + r, r0 + k);
        } else {
          v[t][e] = ld<DEV>(rd, (uint32_t)(r * p + k));
          u[t][e] = diag ? 0.0 : ld<DEV>(rp, (uint32_t)(r * p + k));
        }
      }
    if (s > 0) {
      // L_s,s-1 and L_i,s-1 from Lt (rows past the matrix read as zeros)
      const rsrc_t rs = make_rsrc(lt_tile(Lt, s, s - 1), (int64_t)nv * NB * 8);
      const rsrc_t rq = make_rsrc(lt_tile(Lt, i, s - 1), (int64_t)mi * NB * 8);
      double a1[16], a2[16];
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        a1[it] = ld<false>(rs, (uint32_t)tid, 2048u * it);
        a2[it] = diag ? 0.0 : ld<false>(rq, (uint32_t)tid, 2048u * it);
      }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int r = (tid >> 6) + 4 * it, k = tid & 63;  // element tid + 256 it
        sm.lf[r][k] = a1[it];
        sm.xf[r][k] = a2[it];
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int r = 16 * w + Mfma<double>::row(lane, e);
        const int k = 16 * t + cl;
        // (an opaque copy of the row: otherwise the compiler keeps all 16 padding values of
        // the lane live across the task loop)
        __asm__ volatile("" : "+v"(r));
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
      // the whole tile, padding included (identity past the matrix), for the row inverse
      st<DEV>(const_cast<double*>(xt_tile(Xt, s, s)) + idx, sm.xf[r][k]);
      // U'[p-1-a][p-1-b] = X[a][b] / X[a][a] for b <= a, zero above (the lower U')
      if (r < nv && k < nv)
        st_u(U, f32, (p - 1 - r0 - r) * p + (p - 1 - r0 - k), k <= r ? sm.xf[r][k] / sm.xf[r][r] : 0.0);
    }
    return;
  }
  // L_is = A_is X_ss^T: A_is goes through lf (free after the factorisation); block column
  // s is full width (i > s)
  double* lt = const_cast<double*>(lt_tile(Lt, i, s));
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
      if (r < mi) {
        st<DEV>(&Ar[(ri + r) * p + r0 + k], o[e]);
        st<DEV>(&lt[r * NB + k], o[e]);
      }
    }
  }
}

// One chunk of the row-block inverse.  For i > s, X_is = -X_ii Y_is with
// Y_is = sum_{k=s}^{i-1} L_ik X_ks (from L X = I, block row i).  The sum is split into
// chunks of at most kInvDepth tiles of k, added oldest first: this task adds the tiles
// k in [klo, khi) to the partial sum kept in X (the first chunk starts it), and the chunk
// that ends at k = i - 1 (last) forms X_is, writes it to Xt and its block of U', and
// clears the mirrored block of U'.  L_ik and X_ks come from Lt and Xt through the caches;
// the partial sums, which other workgroups rewrite, at device scope.
__device__ inline void chol_xchunk(int64_t p, int i, int s, int klo, int khi, bool first,
                                   bool last, double* X, const double* Lt, double* Xt, void* U,
                                   bool f32, BlockSmem& sm) {
  typedef Mfma<double>::acc_t acc_t;
  // an opaque copy of the thread index: values derived from it are recomputed per task
  // instead of being held (and spilled) across the persistent loop
  int tid = threadIdx.x;
  __asm__ volatile("" : "+v"(tid));
  const int lane = tid & 63, w = tid >> 6;
  const int wr = w >> 1, wc = w & 1, kr = lane >> 4, cl = lane & 15;
  const int mi = tile_rows(p, i);
  const int64_t ri = (int64_t)i * NB, cs = (int64_t)s * NB;  // block column s is full width
  // staging: thread (column c, rows 16 h .. 16 h + 15) of both 64 x 64 operands, so that a
  // wave loads whole rows and writes whole LDS rows
  const int c = tid & 63, h16 = (tid >> 6) * 16;
  double va[16], vb[16];
  auto fetch = [&](int k) {
    const rsrc_t ra = make_rsrc(lt_tile(Lt, i, k), (int64_t)mi * NB * 8);
    const rsrc_t rb = make_rsrc(xt_tile(Xt, k, s), (int64_t)NB * NB * 8);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      va[u] = ld<false>(ra, (uint32_t)(h16 * NB + c), 512u * u);
      vb[u] = ld<false>(rb, (uint32_t)(h16 * NB + c), 512u * u);
    }
  };
  fetch(klo);
  acc_t acc[2][2];
  {
    const rsrc_t rc = make_rsrc(X + ri * p + cs, ((int64_t)(mi - 1) * p + NB) * 8);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ii = 32 * wr + 16 * a + Mfma<double>::row(lane, e), jj = 32 * wc + 16 * b + cl;
          acc[a][b][e] = first ? 0.0 : ld<true>(rc, (uint32_t)((int64_t)ii * p + jj));
        }
  }
  // acc += A B with A (row-major in lf) and B (row-major in xf), one 64-deep tile
  auto mma = [&](double sign) {
#pragma unroll
    for (int kk = 0; kk < NB; kk += 4) {
      double av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = sign * sm.lf[32 * wr + 16 * t + cl][kk + kr];
        bv[t] = sm.xf[kk + kr][32 * wc + 16 * t + cl];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = Mfma<double>::run(av[a], bv[b], acc[a][b]);
    }
  };
  for (int k = klo; k < khi; ++k) {
    __syncthreads();  // the previous tile's reads of lf / xf are done
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      sm.lf[h16 + u][c] = va[u];
      sm.xf[h16 + u][c] = vb[u];
    }
    __syncthreads();
    if (k + 1 < khi) fetch(k + 1);  // in flight during the products
    mma(1.0);
  }
  if (last) {
    // X_is = -X_ii Y_is: X_ii (padded with the identity past the matrix) in lf, Y in xf
    const rsrc_t rd = make_rsrc(xt_tile(Xt, i, i), (int64_t)NB * NB * 8);
#pragma unroll
    for (int u = 0; u < 16; ++u) va[u] = ld<false>(rd, (uint32_t)(h16 * NB + c), 512u * u);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16; ++u) sm.lf[h16 + u][c] = va[u];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sm.xf[32 * wr + 16 * a + Mfma<double>::row(lane, e)][32 * wc + 16 * b + cl] = acc[a][b][e];
          acc[a][b][e] = 0.0;
        }
    __syncthreads();
    mma(-1.0);
  }
  if (!last) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ii = 32 * wr + 16 * a + Mfma<double>::row(lane, e), jj = 32 * wc + 16 * b + cl;
          if (ii < mi) st<true>(&X[(ri + ii) * p + cs + jj], acc[a][b][e]);
        }
    return;
  }
  double* xt = const_cast<double*>(xt_tile(Xt, i, s));
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = 32 * wr + 16 * a + Mfma<double>::row(lane, e), jj = 32 * wc + 16 * b + cl;
        st<true>(&xt[ii * NB + jj], acc[a][b][e]);
        // U'[p-1-a][p-1-b] = X[a][b] / X[a][a] (lf still holds X_ii)
        if (ii < mi)
          st_u(U, f32, (p - 1 - ri - ii) * p + (p - 1 - cs - jj), acc[a][b][e] / sm.lf[ii][ii]);
      }
  // the mirrored block (rows of tile s, columns of tile i, reversed) lies below U''s
  // diagonal
  for (int idx = tid; idx < NB * NB; idx += 256) {
    const int rr = idx >> 6, cc = idx & 63;
    if (cc < mi) st_u(U, f32, (p - 1 - cs - rr) * p + (p - 1 - ri - cc), 0.0);
  }
}

// ---------------------------------------------------------------------------
// The Cholesky and the inverse of one or two matrices as one persistent kernel
// ---------------------------------------------------------------------------
// Every workgroup takes tasks from one queue in a fixed order; a task waits (bounded)
// until the tasks it depends on are done, so the chain of panel steps runs back to back,
// with no launch boundary per step, while the trailing updates and the inverse fill the
// other CUs.  Tasks of matrix q, step g:
//   bulk(g): tile (i, j), g + 1 <= j <= i, takes panel g - 1 (needs L_i,g-1 and L_j,g-1
//            and the tile's panels 0 .. g - 2; afterwards the tile has g panels);
//   crit(g): the panel step of row tile i >= g (needs L_g,g-1 and L_i,g-1 and the tiles
//            (g, g), (i, g) with panels 0 .. g - 2; afterwards (i, g) holds L_ig, final;
//            crit(g) of i = g also writes X_gg);
//   xrow(g): chunk jj of X_is for i = g + kInvStride jj and every s with a non-empty
//            chunk.  Chunk 0, the last one added, covers k in [i - kInvFirst, i) and
//            multiplies by -X_ii; chunk jj >= 1 covers kInvDepth tiles below
//            khi = i - kInvFirst - kInvDepth (jj - 1) (all clipped at s).  A chunk needs
//            L_i,khi-1 and X_khi-1,s final and the tile's previous chunk; chunk 0 also
//            X_ii.  A row's chunks thus sit in the steps just before its own, oldest chunk
//            first, and the chain from one row of X to the next is one short chunk.
// Group (q, g) lists bulk(g) of column g + 1 first, then crit(g), then the rest of
// bulk(g) column by column, then xrow(g) by jj and s; groups go by step, the matrices
// alternating.  Every task depends only on earlier tasks, so the queue always drains.
using namespace sched;  // task order, waits and signals (schedule.hpp)
constexpr int kMaxChol = 2;
struct CholMat {
  int64_t p;
  int nblk, side_code;
  const void* A;   // the input matrix (lower triangle read), fp32 or fp64
  void* U;         // the output U' in the same dtype
  int f32;
  double* Ar;      // the reversed matrix, updated in place; L's panels
  double* X;       // partial sums of the row inverse
  double* Lt;      // final off-diagonal tiles of L, tiled (written once)
  double* Xt;      // final tiles of X, tiled (written once)
  int* tile_cnt;   // [nblk * nblk] panels applied to each tile by bulk tasks (kFinal: L)
  int* xcnt;       // [nblk * nblk] chunks added to each tile of X (kFinal: X final)
  const int* tab;  // [nblk + 1] tasks of this matrix before each step
};
struct CholArgs {
  CholMat mat[kMaxChol];
  int nmat, maxn;
  int64_t total;  // tasks of all matrices
  int* ctl;       // [0] next task, [32] abort
  int* info;
};
constexpr int kCholSpin = 1 << 20;

// Clears the control words and tile counters of up to two matrices and writes each
// matrix's task table tab[g] = tasks of the matrix before step g (n + 1 entries).  One
// launch: block 0 also computes the tables (group sizes in parallel, a sequential scan).
struct CholSetup {
  int* zero[kMaxChol];
  int64_t words[kMaxChol];
  int* tab[kMaxChol];
  int n[kMaxChol];
  int nmat;
};
__global__ __launch_bounds__(256) void k_chol_setup(CholSetup c) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int q = 0; q < c.nmat; ++q) {
    int* z = q == 0 ? c.zero[0] : c.zero[1];
    const int64_t words = q == 0 ? c.words[0] : c.words[1];
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < words; x += stride) z[x] = 0;
  }
  if (blockIdx.x != 0) return;
  __shared__ int gs[256];
  for (int q = 0; q < c.nmat; ++q) {
    int* tab = q == 0 ? c.tab[0] : c.tab[1];
    const int n = q == 0 ? c.n[0] : c.n[1];
    int run = 0;  // thread 0's running total
    for (int base = 0; base < n; base += 256) {
      const int g = base + (int)threadIdx.x;
      gs[threadIdx.x] = g < n ? (int)group_size(n, g) : 0;
      __syncthreads();
      if (threadIdx.x == 0) {
        const int cnt = n - base < 256 ? n - base : 256;
        for (int k = 0; k < cnt; ++k) {
          tab[base + k] = run;
          run += gs[k];
        }
        if (base + cnt == n) tab[n] = run;
      }
      __syncthreads();
    }
  }
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

__device__ inline int ld_uniform(const int* p) { return __builtin_amdgcn_readfirstlane(*p); }

__global__ __launch_bounds__(256, 2) void k_chol_persistent(CholArgs a) {
  __shared__ union {
    BlockSmem b;
    BulkSmem t;
  } sh;
  __shared__ int task[4];  // kind, matrix, row tile, step (or column) << 16 | column (or jj)
  const int tid = threadIdx.x, lane = tid & 63;
  // Every branch on the wave index is on a wave-uniform value, so that the compiler emits
  // scalar branches: a barrier inside lane-divergent control flow would be reached a
  // different number of times by different waves.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = a.mat[0].nblk, n1 = a.nmat > 1 ? a.mat[1].nblk : 0;
  // wave 0's decode state: the step g of the last task and the task range [lo, hi) of
  // step g (both matrices), with the size of matrix 0's group in it.  A workgroup's tasks
  // only move forward, so the step is found by stepping on from the last one.
  int g = 0;
  int64_t lo = 0, hi = 0, sz0 = 0;
  if (w == 0) {
    sz0 = ld_uniform(a.mat[0].tab + 1);
    hi = sz0 + (n1 > 0 ? ld_uniform(a.mat[1].tab + 1) : 0);
  }
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
      const int64_t t = tl < 0 ? a.total : (int64_t)(unsigned)tl;
      int kind = -1, q = 0, i = 0, x = 0;
      if (t < a.total) {
        while (t >= hi && g + 1 < a.maxn) {
          ++g;
          lo = hi;
          const int g1 = g + 1;
          const int64_t e0 = g < n0 ? ld_uniform(a.mat[0].tab + g1) : 0;
          const int64_t b0 = g < n0 ? ld_uniform(a.mat[0].tab + g) : 0;
          const int64_t e1 = g < n1 ? ld_uniform(a.mat[1].tab + g1) : 0;
          const int64_t b1 = g < n1 ? ld_uniform(a.mat[1].tab + g) : 0;
          sz0 = e0 - b0;
          hi = lo + sz0 + (e1 - b1);
        }
        int64_t r = t - lo;
        if (r >= sz0) {
          r -= sz0;
          q = 1;
        }
        const CholTask ct = chol_decode(q == 0 ? n0 : n1, g, r);
        kind = ct.kind;
        i = ct.i;
        x = (ct.s << 16) | ct.j;
      }
      if (lane == 0) {
        task[0] = kind;
        task[1] = q;
        task[2] = i;
        task[3] = x;
      }
    }
    __syncthreads();
    const int kind = __builtin_amdgcn_readfirstlane(task[0]);
    const int q = __builtin_amdgcn_readfirstlane(task[1]);
    const int i = __builtin_amdgcn_readfirstlane(task[2]);
    const int x = __builtin_amdgcn_readfirstlane(task[3]);
    const int s = x >> 16, j = x & 0xFFFF;  // kind 2: s = column tile, j = chunk index
    __syncthreads();  // task[] is rewritten by the next claim
    if (kind < 0) return;
    // select the matrix with branches (a runtime index into the kernel argument would
    // copy it to scratch memory)
    const CholMat m = q == 0 ? a.mat[0] : a.mat[1];
    const int64_t p = m.p;
    const int n = m.nblk;
    const CholTask ct{kind, i, s, j};
    // kind 2: chunk j of tile (i, s) covers k in [klo, khi)
    int klo = 0, khi = 0;
    xrow_range(ct, &klo, &khi);
    const int nch = xrow_chunks(i, s);
    // dependencies (wave 0 waits, the barrier releases the others); every task polls only
    // the few tiles it reads, so the waiters of one step spread over many words
    if (w == 0) {
      bool ok = true;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        CholWait cw;
        if (ok && chol_wait_at(n, ct, q, &cw))
          ok = chol_wait((cw.arr == 0 ? m.tile_cnt : m.xcnt) + cw.idx, cw.val, a.ctl, a.info);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __syncthreads();
    const bool f32 = m.f32 != 0;
    // The panel steps are the chain that sets the launch's length, and the next block
    // column's trailing update feeds it: their waves take the SIMDs first when they share a
    // CU with the inverse chunks and the rest of the trailing update.
    if (kind == 1)
      __builtin_amdgcn_s_setprio(3);
    else if (kind == 0 && j == s + 1)
      __builtin_amdgcn_s_setprio(2);
    if (kind == 0)
      chol_bulk(p, bulk_lo(j, s), s, i, j, m.Ar, m.Lt, m.A, f32, sh.t);
    else if (kind == 1)
      chol_crit(p, s, i, m.Ar, m.Lt, m.Xt, m.A, m.U, f32, a.info, m.side_code, sh.b);
    else
      chol_xchunk(p, i, s, klo, khi, j == nch - 1, j == 0, m.X, m.Lt, m.Xt, m.U, f32, sh.b);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (w == 0 && lane == 0) {
      const CholWait sg = chol_signal(n, ct);
      __hip_atomic_store((sg.arr == 0 ? m.tile_cnt : m.xcnt) + sg.idx, sg.val, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

struct FactorWs {
  double* Ar;
  double* X;
  double* Lt;  // the Cholesky's tiled copy of the final off-diagonal tiles of L
  double* Xt;  // the tiled copy of the final tiles of X
  int* sync;   // persistent kernel: control words, counters, task table (chol_sync_ints)
};

// ints of the persistent kernel's sync area: 64 control words, the tile counters of L and
// of X, then the task table
int64_t chol_sync_ints(int64_t p) {
  const int64_t nb = cdiv(p, NB);
  return 64 + 2 * nb * nb + nb + 1;
}

// Bytes of Lt (the strictly lower 64 x 64 tiles, nb (nb - 1) / 2) and of Xt (the lower
// tiles with the diagonal, nb (nb + 1) / 2).
size_t lt_bytes(int64_t p) {
  const int64_t nb = cdiv(p, NB);
  return (size_t)(nb * (nb - 1) / 2 > 0 ? nb * (nb - 1) / 2 : 1) * NB * NB * sizeof(double);
}
size_t xt_bytes(int64_t p) {
  const int64_t nb = cdiv(p, NB);
  return (size_t)(nb * (nb + 1) / 2) * NB * NB * sizeof(double);
}

FactorWs carve(int64_t p, void* ws) {
  FactorWs f;
  char* c = (char*)ws;
  f.Ar = (double*)c;
  c += align_up((size_t)p * p * sizeof(double));
  f.X = (double*)c;
  c += align_up((size_t)p * p * sizeof(double));
  f.Lt = (double*)c;
  c += align_up(lt_bytes(p));
  f.Xt = (double*)c;
  c += align_up(xt_bytes(p));
  f.sync = (int*)c;
  return f;
}

}  // namespace

size_t factor_workspace(int64_t p) {
  return 2 * align_up((size_t)p * p * sizeof(double)) + align_up(lt_bytes(p)) +
         align_up(xt_bytes(p)) + align_up((size_t)chol_sync_ints(p) * sizeof(int));
}

// Dense GEMM flops of the trailing update by panel kb (only evaluated while the
// measurement hook is on).
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

namespace {

struct FactorPlan {
  int64_t p;
  int dtype;
  const void* A;
  void* U;
  FactorWs f;
  int side_code;
};

FactorPlan plan(int64_t p, int dtype, const void* A, void* U, void* ws, int side_code) {
  return FactorPlan{p, dtype, A, U, carve(p, ws), side_code};
}

}  // namespace

// The factor of one or two matrices (plans qs[0..nmat)): a setup launch (counters cleared,
// task tables) and the persistent launch, which reads A, computes L and X = L^-1 and writes
// U', on at most `per_cu` workgroups per CU, both on s.
hipError_t chol_persistent_enqueue(const FactorPlan* const* qs, int nmat, int per_cu, int* info,
                                   hipStream_t s) {
  CholArgs a{};
  CholSetup su{};
  a.nmat = su.nmat = nmat;
  a.maxn = 0;
  a.total = 0;
  double fl = 0.0, by = 0.0;
  const bool pr = prof_on();
  int64_t words = 0;
  for (int q = 0; q < nmat; ++q) {
    const FactorPlan& pl = *qs[q];
    const int nb = (int)cdiv(pl.p, NB);
    CholMat& m = a.mat[q];
    m.p = pl.p;
    m.nblk = nb;
    m.side_code = pl.side_code;
    m.A = pl.A;
    m.U = pl.U;
    m.f32 = pl.dtype == 0 ? 1 : 0;
    m.Ar = pl.f.Ar;
    m.X = pl.f.X;
    m.Lt = pl.f.Lt;
    m.Xt = pl.f.Xt;
    m.tile_cnt = pl.f.sync + 64;
    m.xcnt = pl.f.sync + 64 + (int64_t)nb * nb;
    m.tab = pl.f.sync + 64 + 2 * (int64_t)nb * nb;
    su.zero[q] = pl.f.sync;
    su.words[q] = 64 + 2 * (int64_t)nb * nb;
    su.tab[q] = pl.f.sync + 64 + 2 * (int64_t)nb * nb;
    su.n[q] = nb;
    words += su.words[q];
    a.maxn = nb > a.maxn ? nb : a.maxn;
    for (int g = 0; g < nb; ++g) a.total += group_size(nb, g);
    if (pr) {
      const int64_t p = pl.p;
      const double es = pl.dtype == 0 ? 4.0 : 8.0, pp = (double)p * (double)p;
      for (int st = 0; st < nb; ++st) {
        const double nv = (double)((p - st * NB) < NB ? (p - st * NB) : NB);
        const double rows = (double)(p - (int64_t)st * NB) - nv;
        fl += 2.0 / 3.0 * nv * nv * nv + 2.0 * rows * nv * nv +
              (st > 0 ? trailing_flops(p, st - 1) : 0.0);
        const double trail = st > 0 ? (rows + nv) * (rows + nv + NB) / 2.0 : 0.0;
        by += 8.0 * (3.0 * (rows + nv) * NB + 3.0 * trail);
      }
      // row inverse: X_is = -X_ii sum_k L_ik X_ks over the tiles below the diagonal
      for (int i = 1; i < nb; ++i) {
        const double M = (double)((p - (int64_t)i * NB) < NB ? (p - (int64_t)i * NB) : NB);
        for (int sc = 0; sc < i; ++sc) {
          fl += 2.0 * M * NB * NB * (double)(i - sc + 1);
          by += 8.0 * (2.0 * NB * NB * (double)(i - sc) + 2.0 * M * NB * xrow_chunks(i, sc));
        }
      }
      by += pp * (es / 2.0 + es);  // A's lower triangle in, U' out
    }
  }
  if (a.total > 0x7FFFFFFF) return hipErrorInvalidValue;  // task indices are 32-bit
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
  const int64_t zg = cdiv(words, 256) < 1024 ? cdiv(words, 256) : 1024;
  prof_begin(KC_OTHER, s);
  k_chol_setup<<<(unsigned)(zg > 0 ? zg : 1), 256, 0, s>>>(su);
  prof_end(KC_OTHER, s, 0.0, 4.0 * (double)words);
  prof_begin(KC_FACTOR, s);
  k_chol_persistent<<<ncu * occ, 256, 0, s>>>(a);
  prof_end(KC_FACTOR, s, fl, by);
  return hipGetLastError();
}

hipError_t factor_enqueue(int64_t p, int dtype, const void* A, void* U, void* ws, int* info,
                          int side_code, hipStream_t s) {
  const FactorPlan q = plan(p, dtype, A, U, ws, side_code);
  const FactorPlan* qs[1] = {&q};
  return chol_persistent_enqueue(qs, 1, 2, info, s);
}

hipError_t factor_pair_enqueue(int64_t m, const void* A, void* Ua, void* ws_a, int64_t n,
                               const void* B, void* Ub, void* ws_b, int dtype, int* info,
                               hipStream_t s, int code_a, int code_b) {
  const FactorPlan qa = plan(m, dtype, A, Ua, ws_a, code_a);
  const FactorPlan qb = plan(n, dtype, B, Ub, ws_b, code_b);
  const FactorPlan* qs[2] = {&qa, &qb};
  return chol_persistent_enqueue(qs, 2, 2, info, s);
}

}  // namespace g2d
