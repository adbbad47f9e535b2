// Sweep stage for gfx950: anti-diagonal two-sided adaptive rounding with
// separable band feedback.
//
// Page reference: arxivlens page "GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding",
// Results (entries of one anti-diagonal are independent and are rounded together;
// feedback is rank-one and separable, realised by a few band-like matrix products),
// Methodology (anti-diagonal rounds with a buffer of accumulated feedback), Abstract
// (two levels of blocking); mind-verse article, section "Die algorithmische Neuerung
// und ihre Auswirkungen" (anti-diagonal processing, parallel inside each one).
//
// With unit factors U'a, U'b the rounding target of entry (k,l) is
//   t[k,l] = W[k,l] - sum_{i<k} U'a[i,k] R[i,l] - sum_{j<l} Delta[k,j] U'b[j,l]
// where R (vertical residual) = W - G - Q and Delta = t - Q.  (k,l) depends only on
// entries above it in its column and left of it in its row, so every anti-diagonal
// is an antichain.
//
// Blocking (64 x 64 blocks; outer blocks of 4 x 4 blocks):
//   * k_round rounds all blocks of one block anti-diagonal D.  It first pulls the band
//     feedback of the two neighbours just finished on D-1 (block above: Ua'^T R, 64
//     deep; block to the left: Delta Ub', 64 deep) with MFMA, adds what k_push has
//     accumulated in Vf/Hf, and then rounds the block: the four waves own 16-row
//     micro-rows and walk 16x16 micro-tiles along micro anti-diagonals; feedback
//     between micro-tiles is an MFMA product from LDS, feedback inside a micro-tile is
//     applied entry by entry along its 31 anti-diagonal steps.
//   * k_push (second stream, off the critical path) pushes everything else into Vf
//     (vertical, -Ua'^T R) and Hf (horizontal, +Delta Ub'): 64 deep from a block to
//     the blocks two or more past it up to the first block of the next outer block,
//     and, when a block closes an outer block, 256 deep from the whole outer block to
//     every block beyond.  All those targets lie two or more block diagonals ahead,
//     which is the slack that lets it overlap the rounding.
#include <math.h>

#include <mutex>
#include <vector>

#include "common.hpp"
#include "launch.hpp"
#include "prof.hpp"

namespace g2d {
namespace {

constexpr int BB = 64;   // block edge
constexpr int MU = 16;   // micro-tile edge
constexpr int GOUT = 4;  // blocks per outer block edge (outer block = 256)

template <typename T>
struct SweepArgs {
  int64_t m, n;
  int Mb, Nb, lo, hi, bits;
  const T* Ua;
  const T* Ub;
  const T* s;
  const T* W;
  T* Vf;   // vertical feedback pushed by k_push (subtracted from W)
  T* Hf;   // horizontal feedback pushed by k_push
  T* R;    // vertical residual, row-major m x n
  T* DT;   // Delta transposed, n x m
  int8_t* codes;
  T* Q;
};

// Row strides keep 4-element groups 16-byte aligned for vector LDS reads.
template <typename T>
struct Pad;
template <>
struct Pad<float> {
  static constexpr int v = 68;
};
template <>
struct Pad<double> {
  static constexpr int v = 66;
};

template <typename T>
struct RoundSmem {
  static constexpr int P = Pad<T>::v;
  T ua[BB][P];           // diagonal block of U'a, row-major, strictly upper
  T ubT[BB][P];          // diagonal block of U'b, transposed: ubT[c][k] = U'b[k][c]
  T rT[BB][P];           // R of this block, transposed: rT[c][i] = R[i][c]
  T dd[BB][P];           // Delta of this block, row-major
  T g0s[4][MU][MU];      // per wave, skewed: g0s[r][sl] = (W - G outside)[r][(sl - r) % 16]
  T h0s[4][MU][MU];      // per wave, skewed: H pushed from outside; scratch during a sweep
  T sc[BB];              // scales
  T rs[BB];              // fl(1 / scale)
  int8_t zz[BB][BB];     // codes of this block
};

// Orders the LDS accesses of one wave: the LDS unit executes a wave's operations in
// issue order, so it is enough that the compiler keeps program order here (no wait
// on outstanding global loads is wanted).
__device__ inline void lds_wave_sync() { __asm__ volatile("" ::: "memory"); }

__device__ inline float rint_t(float x) { return rintf(x); }
__device__ inline double rint_t(double x) { return rint(x); }
__device__ inline float abs_t(float x) { return fabsf(x); }
__device__ inline double abs_t(double x) { return fabs(x); }

template <typename T>
struct Eps;
template <>
struct Eps<float> {
  static constexpr float v = 1.1920929e-07f;
};
template <>
struct Eps<double> {
  static constexpr double v = 2.220446049250313e-16;
};

// rint(t / s) with IEEE semantics.  y = t * fl(1/s) is within eps*|y| of t/s, so it
// decides the rounding unless t/s lies that close to a half-integer; those rare lanes
// redo the IEEE division.  Quotients beyond 2^bits are clamped whichever way they
// round, so the tolerance `tol` = 4 eps 2^bits covers every decision that matters.
template <typename T>
__device__ inline T round_quot(T t, T s, T rs, T tol) {
  const T y = t * rs;
  T z = rint_t(y);
  if (__builtin_expect(abs_t(y - z) > T(0.5) - tol, 0)) z = rint_t(t / s);
  return z;
}

// Neighbour row's value for lane layout lane = 4 r + q: lane - 4 inside a 16-lane DPP
// row, and from lane 15 of the previous DPP row for r = 4, 8, 12 (all four lanes of a
// row hold the same value).  r = 0 reads 0.
__device__ inline int dpp_up4(int v) {
  int x = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  x = __builtin_amdgcn_update_dpp(x, v, 0x142, 0xE, 0x1, false);     // row_bcast:15
  return x;
}
__device__ inline float up_row(float v) { return __int_as_float(dpp_up4(__float_as_int(v))); }
__device__ inline double up_row(double v) {
  return __hiloint2double(dpp_up4(__double2hiint(v)), dpp_up4(__double2loint(v)));
}
// Sum over the four lanes of a quad (the same value in each).
__device__ inline float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  return v;
}
__device__ inline double quad_sum(double v) {
  double w = __hiloint2double(__builtin_amdgcn_mov_dpp(__double2hiint(v), 0xB1, 0xF, 0xF, false),
                              __builtin_amdgcn_mov_dpp(__double2loint(v), 0xB1, 0xF, 0xF, false));
  v += w;
  w = __hiloint2double(__builtin_amdgcn_mov_dpp(__double2hiint(v), 0x4E, 0xF, 0xF, false),
                       __builtin_amdgcn_mov_dpp(__double2loint(v), 0x4E, 0xF, 0xF, false));
  return v + w;
}

__device__ inline float min_t(float a, float b) { return fminf(a, b); }
__device__ inline double min_t(double a, double b) { return fmin(a, b); }
__device__ inline float max_t(float a, float b) { return fmaxf(a, b); }
__device__ inline double max_t(double a, double b) { return fmax(a, b); }

// Four consecutive elements from LDS (16-byte aligned), as one or two vector reads.
template <typename T>
struct Vec4 {
  T v[4];
};
__device__ inline Vec4<float> lds_read4(const float* p) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 x = *(const f4*)p;
  return Vec4<float>{{x[0], x[1], x[2], x[3]}};
}
__device__ inline Vec4<double> lds_read4(const double* p) {
  typedef double d2 __attribute__((ext_vector_type(2)));
  const d2 x = *(const d2*)p;
  const d2 y = *(const d2*)(p + 2);
  return Vec4<double>{{x[0], x[1], y[0], y[1]}};
}

// Rounds all blocks of block anti-diagonal D.  Wave w owns micro-row w (16 rows) and at
// micro anti-diagonal d handles micro-tile (w, d - w).  In the micro sweep, lane
// (r, q) = (lane / 4, lane % 4) works on row r; at step st the active lanes hold the
// micro anti-diagonal r + l = st.  The target of (r, l) is
//     t = g0[r][l] - h0[r][l] - (vertical + horizontal feedback inside the micro-tile)
// where the two nearest terms (row r-1 at the previous step, reached by a DPP row
// shift, and the lane's own previous Delta) are added on the critical path and the
// older ones (rows <= r-2, columns <= l-2) are summed one step ahead from LDS, each
// quarter q taking four of them, then reduced across the quad.
template <typename T>
__global__ __launch_bounds__(256) void k_round(SweepArgs<T> a, int D) {
  typedef typename Mfma<T>::acc_t acc_t;
  constexpr int P = Pad<T>::v;
  __shared__ RoundSmem<T> sm;
  const int kmin = D - (a.Nb - 1) > 0 ? D - (a.Nb - 1) : 0;
  const int K = kmin + blockIdx.x;
  const int L = D - K;
  const int64_t m = a.m, n = a.n;
  const int64_t r0 = (int64_t)K * BB, c0 = (int64_t)L * BB;
  const int mr = (m - r0) < BB ? (int)(m - r0) : BB;
  const int nc = (n - c0) < BB ? (int)(n - c0) : BB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // Global loads first, all in flight together: the wave's four micro-tiles of
  // W - G and H pushed from outside (MFMA accumulator layout), the diagonal factor
  // blocks and the scales.
  // Reads past the block's last row come back as zero; columns past the edge read
  // neighbouring (finite) data that only ever feeds padded entries.
  const int64_t es = sizeof(T);
  const int64_t blk_bytes = ((int64_t)(mr - 1) * n + nc) * es;
  const int64_t o0 = r0 * n + c0;
  const rsrc_t rw = make_rsrc(a.W + o0, blk_bytes), rvf = make_rsrc(a.Vf + o0, blk_bytes);
  const rsrc_t rhf = make_rsrc(a.Hf + o0, blk_bytes);
  const rsrc_t rua = make_rsrc(a.Ua + r0 * m + r0, ((int64_t)(mr - 1) * m + mr) * es);
  const rsrc_t rub = make_rsrc(a.Ub + c0 * n + c0, ((int64_t)(nc - 1) * n + nc) * es);
  T gin[BB / MU][4], hin[BB / MU][4];
#pragma unroll
  for (int jm = 0; jm < BB / MU; ++jm)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = MU * w + Mfma<T>::row(lane, e), c = MU * jm + (lane & 15);
      const uint32_t o = (uint32_t)(i * n + c);
      gin[jm][e] = buf_load<T>(rw, o) - buf_load<T>(rvf, o);
      hin[jm][e] = buf_load<T>(rhf, o);
    }
  T fua[BB * BB / 256], fub[BB * BB / 256];
#pragma unroll
  for (int it = 0; it < BB * BB / 256; ++it) {
    const int idx = tid + 256 * it, i = idx >> 6, j = idx & 63;
    fua[it] = buf_load<T>(rua, (uint32_t)(i * m + j));
    fub[it] = buf_load<T>(rub, (uint32_t)(i * n + j));
  }
  // Operands of the two 64-deep neighbour pulls (block above: U'a^T R; block to the
  // left: Delta U'b), all k-major.  The shared B panels (R and U'b rows of the
  // previous blocks) are staged through LDS; each wave keeps its own A fragments
  // (16 k-steps) in registers.  Buffer ranges end at the last valid element.
  const int kq = lane >> 4, cl = lane & 15;
  const int rows_w = mr - MU * w;
  const int rv_w = rows_w < 0 ? 0 : (rows_w > MU ? MU : rows_w);
  const bool up = K > 0, left = L > 0;
  T bv_st[BB * BB / 256], bh_st[BB * BB / 256];
  T av_fr[BB / 4], ah_fr[BB / 4];
  {
    const rsrc_t rbv = make_rsrc(up ? a.R + (r0 - BB) * n + c0 : a.R, up ? ((int64_t)(BB - 1) * n + nc) * es : 0);
    const rsrc_t rbh = make_rsrc(left ? a.Ub + (c0 - BB) * n + c0 : a.Ub, left ? ((int64_t)(BB - 1) * n + nc) * es : 0);
    const rsrc_t rav = make_rsrc(up ? a.Ua + (r0 - BB) * m + r0 + MU * w : a.Ua,
                                 up ? ((int64_t)(BB - 1) * m + rv_w) * es : 0);
    const rsrc_t rah = make_rsrc(left ? a.DT + (c0 - BB) * m + r0 + MU * w : a.DT,
                                 left ? ((int64_t)(BB - 1) * m + rv_w) * es : 0);
#pragma unroll
    for (int it = 0; it < BB * BB / 256; ++it) {
      const int idx = tid + 256 * it, k = idx >> 6, c = idx & 63;
      bv_st[it] = buf_load<T>(rbv, (uint32_t)(k * n + c));
      bh_st[it] = buf_load<T>(rbh, (uint32_t)(k * n + c));
    }
#pragma unroll
    for (int sk = 0; sk < BB / 4; ++sk) {
      av_fr[sk] = buf_load<T>(rav, (uint32_t)((4 * sk + kq) * m + cl));
      ah_fr[sk] = buf_load<T>(rah, (uint32_t)((4 * sk + kq) * m + cl));
    }
  }
  const T sv0 = buf_load<T>(make_rsrc(a.s + r0, (int64_t)mr * es), (uint32_t)(tid & 63));
  const T sv = tid < mr ? sv0 : T(1);
#pragma unroll
  for (int it = 0; it < BB * BB / 256; ++it) {
    const int idx = tid + 256 * it, i = idx >> 6, j = idx & 63;
    fua[it] = (i < mr && j < mr && i < j) ? fua[it] : T(0);
    fub[it] = (i < nc && j < nc && i < j) ? fub[it] : T(0);
  }
#pragma unroll
  for (int it = 0; it < BB * BB / 256; ++it) {
    const int idx = tid + 256 * it, i = idx >> 6, j = idx & 63;
    sm.ua[i][j] = fua[it];
    sm.ubT[j][i] = fub[it];
    sm.rT[i][j] = bv_st[it];  // staging: R panel of the block above, rT[k][c]
    sm.dd[i][j] = bh_st[it];  // staging: U'b panel of the block to the left, dd[k][c]
  }
  if (tid < BB) {
    sm.sc[tid] = sv;
    sm.rs[tid] = T(1) / sv;
  }
  __syncthreads();
  // neighbour pulls into this wave's inputs (MFMA accumulator layout = gin/hin layout)
  if (up) {
    acc_t acc[BB / MU];
#pragma unroll
    for (int jm = 0; jm < BB / MU; ++jm) acc[jm] = acc_t{0, 0, 0, 0};
#pragma unroll
    for (int sk = 0; sk < BB / 4; ++sk)
#pragma unroll
      for (int jm = 0; jm < BB / MU; ++jm)
        acc[jm] = Mfma<T>::run(av_fr[sk], sm.rT[4 * sk + kq][MU * jm + cl], acc[jm]);
#pragma unroll
    for (int jm = 0; jm < BB / MU; ++jm)
#pragma unroll
      for (int e = 0; e < 4; ++e) gin[jm][e] -= acc[jm][e];
  }
  if (left) {
    acc_t acc[BB / MU];
#pragma unroll
    for (int jm = 0; jm < BB / MU; ++jm) acc[jm] = acc_t{0, 0, 0, 0};
#pragma unroll
    for (int sk = 0; sk < BB / 4; ++sk)
#pragma unroll
      for (int jm = 0; jm < BB / MU; ++jm)
        acc[jm] = Mfma<T>::run(ah_fr[sk], sm.dd[4 * sk + kq][MU * jm + cl], acc[jm]);
#pragma unroll
    for (int jm = 0; jm < BB / MU; ++jm)
#pragma unroll
      for (int e = 0; e < 4; ++e) hin[jm][e] += acc[jm][e];
  }
  __syncthreads();
  // the staging areas become this block's R and Delta, which start at zero
#pragma unroll
  for (int it = 0; it < BB * BB / 256; ++it) {
    const int idx = tid + 256 * it, i = idx >> 6, j = idx & 63;
    sm.rT[i][j] = T(0);
    sm.dd[i][j] = T(0);
  }
  __syncthreads();

  // micro sweep lane layout: lane = 4 r + q (row r of the micro-tile, quarter q)
  const int rr_ = lane >> 2, qq = lane & 3;
  const int gr = MU * w + rr_;  // block row handled by this lane in the micro sweep
  const T s_r = sm.sc[gr], rs_r = sm.rs[gr];
  const T tlo = T(a.lo), thi = T(a.hi);
  const T tol = T(4) * Eps<T>::v * T(1 << (a.bits));
  // in-micro-tile vertical coefficients: U'a[i][r] for the quarter's rows i = 4q+u
  // (rows >= r hold zeros), and U'a[r-1][r] for the nearest row
  T cu[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) cu[u] = sm.ua[MU * w + 4 * qq + u][gr];
  const T cup = (rr_ > 0) ? sm.ua[gr - 1][gr] : T(0);

  for (int d = 0; d < 2 * (BB / MU) - 1; ++d) {
    const int j = d - w;  // micro-column of this wave's micro-tile (wave-uniform)
    if (j >= 0 && j < BB / MU) {
      const int mc0 = MU * j;
      // this micro-tile's inputs are at the front of the queue; rotate (static indices)
      T wv[4], hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wv[e] = gin[0][e];
        hv[e] = hin[0][e];
#pragma unroll
        for (int jm = 0; jm + 1 < BB / MU; ++jm) {
          gin[jm][e] = gin[jm + 1][e];
          hin[jm][e] = hin[jm + 1][e];
        }
      }
      // feedback from outside the micro-tile but inside the block (two MFMA chains each)
      acc_t av0 = acc_t{0, 0, 0, 0}, av1 = acc_t{0, 0, 0, 0};
      acc_t ah0 = acc_t{0, 0, 0, 0}, ah1 = acc_t{0, 0, 0, 0};
      for (int k0 = 0; k0 < MU * w; k0 += 8) {
        av0 = Mfma<T>::run(sm.ua[k0 + (lane >> 4)][MU * w + (lane & 15)],
                           sm.rT[mc0 + (lane & 15)][k0 + (lane >> 4)], av0);
        av1 = Mfma<T>::run(sm.ua[k0 + 4 + (lane >> 4)][MU * w + (lane & 15)],
                           sm.rT[mc0 + (lane & 15)][k0 + 4 + (lane >> 4)], av1);
      }
      for (int k0 = 0; k0 < mc0; k0 += 8) {
        ah0 = Mfma<T>::run(sm.dd[MU * w + (lane & 15)][k0 + (lane >> 4)],
                           sm.ubT[mc0 + (lane & 15)][k0 + (lane >> 4)], ah0);
        ah1 = Mfma<T>::run(sm.dd[MU * w + (lane & 15)][k0 + 4 + (lane >> 4)],
                           sm.ubT[mc0 + (lane & 15)][k0 + 4 + (lane >> 4)], ah1);
      }
      // skewed staging: slot sl of row r holds column (sl - r) mod 16
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = Mfma<T>::row(lane, e), col = lane & 15;
        sm.g0s[w][row][(col + row) & (MU - 1)] = wv[e] - (av0[e] + av1[e]);
        sm.h0s[w][row][(col + row) & (MU - 1)] = hv[e] + (ah0[e] + ah1[e]);
      }
      lds_wave_sync();
      T g0r[MU], h0r[MU], sdr[MU];
#pragma unroll
      for (int sl = 0; sl < MU; sl += 4) {
        const Vec4<T> gv = lds_read4(&sm.g0s[w][rr_][sl]);
        const Vec4<T> hv4 = lds_read4(&sm.h0s[w][rr_][sl]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          g0r[sl + u] = gv.v[u];
          h0r[sl + u] = hv4.v[u];
        }
      }
#pragma unroll
      for (int sl = 0; sl < MU; ++sl) {
        const int col = (sl - rr_) & (MU - 1);
        sdr[sl] = col > 0 ? sm.ubT[mc0 + col][mc0 + col - 1] : T(0);  // U'b[l-1][l]
      }
      lds_wave_sync();
      const T* rtq = &sm.rT[mc0][MU * w + 4 * qq];  // + P * column
      const T* ddq = &sm.dd[gr][mc0 + 4 * qq];
      const T* ubq = &sm.ubT[mc0][mc0 + 4 * qq];    // + P * column
      // inactive lanes store into this wave's staging row, which is dead until the
      // next micro-tile
      T* dummy = &sm.h0s[w][rr_][0];
      T pv = T(0), ph = T(0);
      T rprev = T(0), dprev = T(0);
#pragma unroll
      for (int st = 0; st < 2 * MU - 1; ++st) {
        const int l = st - rr_;
        const bool act = (l >= 0) && (l < MU);
        // (A) operands of the next step's older-term sums (written up to step st-1)
        const int l1 = st + 1 - rr_;
        const int lc1 = (l1 >= 0 && l1 < MU) ? l1 : 0;
        const Vec4<T> rv = lds_read4(rtq + P * lc1);
        const Vec4<T> dv = lds_read4(ddq);
        const Vec4<T> bv = lds_read4(ubq + P * lc1);
        // (B) critical chain of this step
        const T rup = up_row(rprev);
        const T g = g0r[st & (MU - 1)] - (pv + cup * rup);
        const T hh = h0r[st & (MU - 1)] + (ph + sdr[st & (MU - 1)] * dprev);
        const T t = g - hh;
        T z = round_quot(t, s_r, rs_r, tol);
        z = min_t(max_t(z, tlo), thi);
        const T qv = s_r * z;
        const T rv_new = g - qv, dv_new = t - qv;
        const int lw = act ? l : 0;
        T* prt = act ? &sm.rT[mc0 + lw][gr] : dummy;
        T* pdd = act ? &sm.dd[gr][mc0 + lw] : dummy + 1;
        int8_t* pzz = act ? &sm.zz[gr][mc0 + lw] : (int8_t*)(dummy + 2);
        *prt = rv_new;
        *pdd = dv_new;
        *pzz = (int8_t)(int)z;
        rprev = rv_new;
        dprev = dv_new;
        // (C) older-term sums of the next step
        T sv = T(0), sh = T(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sv += cu[u] * rv.v[u];
          sh += dv.v[u] * bv.v[u];
        }
        pv = quad_sum(sv);
        ph = quad_sum(sh);
        lds_wave_sync();
      }
    }
    __syncthreads();
  }
  // R row-major; Delta transposed (DT[col][row]) for the k-major band products
  for (int idx = tid; idx < BB * BB; idx += 256) {
    const int i = idx >> 6, j = idx & 63;
    if (i < mr && j < nc) {
      const int64_t o = (r0 + i) * n + c0 + j;
      const int z = sm.zz[i][j];
      a.R[o] = sm.rT[j][i];
      a.codes[o] = (int8_t)z;
      a.Q[o] = sm.sc[i] * T(z);
    }
    const int jt = idx >> 6, it = idx & 63;
    if (it < mr && jt < nc) a.DT[(c0 + jt) * m + r0 + it] = sm.dd[it][jt];
  }
}

// One 64x64 output tile, C[i][j] += alpha * sum_{k<K} A[k*lda + i] * B[k*ldb + j]
// (both operands k-major).  Four waves in a 2x2 arrangement, each 32x32 = 2x2 MFMA
// tiles; operand fragments are read straight from global memory (16 consecutive
// elements per k, coalesced) into a ring of PF k-steps kept in flight ahead of the
// MFMAs that use them.  All loads are branch-free (clamped address, zero select).
template <typename T>
__device__ inline void tile_tn(const T* A, int64_t lda, const T* B, int64_t ldb, T* C,
                               int64_t ldc, int M, int N, int K, T alpha) {
  typedef typename Mfma<T>::acc_t acc_t;
  constexpr int PF = 4;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i0 = 32 * (w >> 1), j0 = 32 * (w & 1);
  const int kq = lane >> 4, c = lane & 15;
  const int64_t es = sizeof(T);
  // k-major views end after row K: reads of k >= K are zero.  Rows/columns past M/N
  // read neighbouring data that only reaches outputs which are never stored.
  const rsrc_t ra = make_rsrc(A, ((int64_t)(K - 1) * lda + M) * es);
  const rsrc_t rb = make_rsrc(B, ((int64_t)(K - 1) * ldb + N) * es);
  const rsrc_t rc = make_rsrc(C, ((int64_t)(M - 1) * ldc + N) * es);
  acc_t acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = acc_t{0, 0, 0, 0};
  T fa[PF][2], fb[PF][2];
  auto fetch = [&](int slot, int k) {
    const uint32_t oa = (uint32_t)((int64_t)k * lda + i0 + c);
    const uint32_t ob = (uint32_t)((int64_t)k * ldb + j0 + c);
    fa[slot][0] = buf_load<T>(ra, oa);
    fa[slot][1] = buf_load<T>(ra, oa + 16);
    fb[slot][0] = buf_load<T>(rb, ob);
    fb[slot][1] = buf_load<T>(rb, ob + 16);
  };
#pragma unroll
  for (int sl = 0; sl < PF; ++sl) fetch(sl, 4 * sl + kq);
  for (int k0 = 0; k0 < K; k0 += 4 * PF) {
#pragma unroll
    for (int sl = 0; sl < PF; ++sl) {
      const T a0 = fa[sl][0], a1 = fa[sl][1], b0 = fb[sl][0], b1 = fb[sl][1];
      fetch(sl, k0 + 4 * (sl + PF) + kq);
      acc[0][0] = Mfma<T>::run(a0, b0, acc[0][0]);
      acc[0][1] = Mfma<T>::run(a0, b1, acc[0][1]);
      acc[1][0] = Mfma<T>::run(a1, b0, acc[1][0]);
      acc[1][1] = Mfma<T>::run(a1, b1, acc[1][1]);
    }
  }
  T old[2][2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 16 * x + Mfma<T>::row(lane, e), j = j0 + 16 * y + c;
        old[x][y][e] = buf_load<T>(rc, (uint32_t)((int64_t)i * ldc + j));
      }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 16 * x + Mfma<T>::row(lane, e), j = j0 + 16 * y + c;
        if (i < M && j < N) C[(int64_t)i * ldc + j] = old[x][y][e] + alpha * acc[x][y][e];
      }
}

// Band pushes of the blocks on diagonal D that the next diagonal does not pull
// itself.  z = 0: vertical into Vf from block (K, L) to row block t = K+2+x of column L;
// z = 1: horizontal into Hf from (K, L) to column block t = L+2+x of row K.  Targets up
// to the first block of the next outer block take the 64-deep panel of (K, L); beyond
// that, a block that closes an outer block pushes the whole outer block (256 deep).
template <typename T>
__global__ __launch_bounds__(256) void k_push(SweepArgs<T> a, int D) {
  const int kmin = D - (a.Nb - 1) > 0 ? D - (a.Nb - 1) : 0;
  const int K = kmin + blockIdx.y;
  const int L = D - K;
  const int64_t m = a.m, n = a.n;
  if (blockIdx.z == 0) {
    const int t = K + 2 + blockIdx.x;
    if (t >= a.Mb) return;
    int64_t src0;
    int ks;
    if (t <= GOUT * (K / GOUT + 1)) {
      src0 = (int64_t)K * BB;
      ks = (m - src0) < BB ? (int)(m - src0) : BB;
    } else if (K % GOUT == GOUT - 1) {
      src0 = (int64_t)(K - (GOUT - 1)) * BB;
      ks = GOUT * BB;
    } else {
      return;
    }
    const int64_t tr0 = (int64_t)t * BB, c0 = (int64_t)L * BB;
    const int M = (m - tr0) < BB ? (int)(m - tr0) : BB;
    const int N = (n - c0) < BB ? (int)(n - c0) : BB;
    tile_tn<T>(a.Ua + src0 * m + tr0, m, a.R + src0 * n + c0, n, a.Vf + tr0 * n + c0, n, M, N, ks,
               T(1));
  } else {
    const int t = L + 2 + blockIdx.x;
    if (t >= a.Nb) return;
    int64_t src0;
    int ks;
    if (t <= GOUT * (L / GOUT + 1)) {
      src0 = (int64_t)L * BB;
      ks = (n - src0) < BB ? (int)(n - src0) : BB;
    } else if (L % GOUT == GOUT - 1) {
      src0 = (int64_t)(L - (GOUT - 1)) * BB;
      ks = GOUT * BB;
    } else {
      return;
    }
    const int64_t r0 = (int64_t)K * BB, tc0 = (int64_t)t * BB;
    const int M = (m - r0) < BB ? (int)(m - r0) : BB;
    const int N = (n - tc0) < BB ? (int)(n - tc0) : BB;
    tile_tn<T>(a.DT + src0 * m + r0, m, a.Ub + src0 * n + tc0, n, a.Hf + r0 * n + tc0, n, M, N, ks,
               T(1));
  }
}

// Vf = Hf = 0.
template <typename T>
__global__ __launch_bounds__(256) void k_init(int64_t count, T* Vf, T* Hf) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256) {
    Vf[i] = T(0);
    Hf[i] = T(0);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_check_scales(int64_t m, const T* __restrict__ s,
                                                      int* info) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  const T v = s[i];
  if (!(v > T(0)) || !isfinite(v)) record_info(info, 3, (int)(i + 1));
}

// Algorithmic work of one launch (only evaluated while the measurement hook is on).
// Round: in-block feedback flops, the two 64-deep neighbour pulls (2 M N K), and the
// HBM bytes every block must move (W, Vf, Hf, the neighbour panels, the diagonal
// factor blocks and scales in; R, Delta, Q out, one byte per code).
void round_work(int64_t m, int64_t n, int D, int Mb, int Nb, double es, double* flops,
                double* bytes) {
  *flops = *bytes = 0.0;
  const int kmin = D - (Nb - 1) > 0 ? D - (Nb - 1) : 0;
  const int kmax = D < Mb - 1 ? D : Mb - 1;
  for (int K = kmin; K <= kmax; ++K) {
    const int L = D - K;
    const double mr = (double)((m - (int64_t)K * BB) < BB ? (m - (int64_t)K * BB) : BB);
    const double nc = (double)((n - (int64_t)L * BB) < BB ? (n - (int64_t)L * BB) : BB);
    *flops += mr * nc * (mr + nc - 2.0);
    *bytes += es * (6.0 * mr * nc + mr * mr + nc * nc + mr) + mr * nc;
    if (K > 0) {
      *flops += 2.0 * mr * nc * BB;
      *bytes += es * (BB * mr + BB * nc);
    }
    if (L > 0) {
      *flops += 2.0 * mr * nc * BB;
      *bytes += es * (BB * mr + BB * nc);
    }
  }
}

// Push: dense GEMM flops (2 M N K per tile) and operand/RMW bytes of k_push at D.
// Returns false when no block on D has anything to push.
bool push_work(int64_t m, int64_t n, int D, int Mb, int Nb, double es, double* flops,
               double* bytes) {
  *flops = *bytes = 0.0;
  bool any = false;
  const int kmin = D - (Nb - 1) > 0 ? D - (Nb - 1) : 0;
  const int kmax = D < Mb - 1 ? D : Mb - 1;
  auto ext = [](int64_t total, int64_t start) {
    return (double)((total - start) < BB ? (total - start) : BB);
  };
  for (int K = kmin; K <= kmax; ++K) {
    const int L = D - K;
    const double nc = ext(n, (int64_t)L * BB), mr = ext(m, (int64_t)K * BB);
    for (int t = K + 2; t < Mb; ++t) {
      double ks;
      if (t <= GOUT * (K / GOUT + 1)) ks = mr;
      else if (K % GOUT == GOUT - 1) ks = GOUT * BB;
      else continue;
      any = true;
      const double M = ext(m, (int64_t)t * BB);
      *flops += 2.0 * M * nc * ks;
      *bytes += es * (ks * M + ks * nc + 2.0 * M * nc);
    }
    for (int t = L + 2; t < Nb; ++t) {
      double ks;
      if (t <= GOUT * (L / GOUT + 1)) ks = nc;
      else if (L % GOUT == GOUT - 1) ks = GOUT * BB;
      else continue;
      any = true;
      const double N = ext(n, (int64_t)t * BB);
      *flops += 2.0 * mr * N * ks;
      *bytes += es * (mr * ks + ks * N + 2.0 * mr * N);
    }
  }
  return any;
}

template <typename T>
hipError_t sweep_typed(int64_t m, int64_t n, int bits, const T* W, const T* Ua, const T* Ub,
                       const T* scales, int8_t* codes, T* Q, void* ws, int* info, hipStream_t s) {
  const size_t mn = (size_t)m * n;
  char* c = (char*)ws;
  auto take = [&]() {
    T* p = (T*)c;
    c += align_up(mn * sizeof(T));
    return p;
  };
  SweepArgs<T> a;
  a.m = m;
  a.n = n;
  a.Mb = (int)cdiv(m, BB);
  a.Nb = (int)cdiv(n, BB);
  a.lo = -(1 << (bits - 1));
  a.hi = (1 << (bits - 1)) - 1;
  a.bits = bits;
  a.Ua = Ua;
  a.Ub = Ub;
  a.s = scales;
  a.W = W;
  a.Vf = take();
  a.Hf = take();
  a.R = take();
  a.DT = take();
  a.codes = codes;
  a.Q = Q;
  const int Mb = a.Mb, Nb = a.Nb, nD = Mb + Nb - 1;

  std::lock_guard<std::recursive_mutex> lock(lib_mutex());
  hipStream_t s1 = nullptr;
  hipEvent_t* evs = nullptr;
  // events 0..1 belong to the caller of this function; the sweep uses the rest
  hipError_t e = aux_resources(2 + 2 * (size_t)nD + 1, &s1, &evs);
  if (e != hipSuccess) return e;
  hipEvent_t* ev_round = evs + 2;      // [nD]
  hipEvent_t* ev_far = ev_round + nD;  // [nD]
  hipEvent_t ev_init = ev_far[nD];

  const bool pr = prof_on();
  const double es = (double)sizeof(T);
  prof_begin(KC_OTHER, s);
  k_check_scales<T><<<(unsigned)cdiv(m, 256), 256, 0, s>>>(m, scales, info);
  const int64_t ig = cdiv((int64_t)mn, 256) < 8192 ? cdiv((int64_t)mn, 256) : 8192;
  k_init<T><<<(unsigned)ig, 256, 0, s>>>((int64_t)mn, a.Vf, a.Hf);
  prof_end(KC_OTHER, s, 0.0, es * (2.0 * (double)mn + (double)m));
  if ((e = hipEventRecord(ev_init, s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(s1, ev_init, 0)) != hipSuccess) return e;

  int last_far = -1;
  const int maxt = (Mb > Nb ? Mb : Nb);
  std::vector<int> far_list;  // diagonals that issued pushes, increasing
  size_t fp = 0;
  int waited = -1;
  for (int D = 0; D < nD; ++D) {
    const int kmin = D - (Nb - 1) > 0 ? D - (Nb - 1) : 0;
    const int kmax = D < Mb - 1 ? D : Mb - 1;
    const int nblk = kmax - kmin + 1;
    // pushes issued at D-2 or earlier may target blocks on D (the second stream runs
    // them in order, so waiting for the newest such launch covers all of them)
    while (fp < far_list.size() && far_list[fp] <= D - 2) ++fp;
    if (fp > 0 && far_list[fp - 1] != waited) {
      waited = far_list[fp - 1];
      if ((e = hipStreamWaitEvent(s, ev_far[waited], 0)) != hipSuccess) return e;
    }
    double fl = 0.0, by = 0.0;
    if (pr) round_work(m, n, D, Mb, Nb, es, &fl, &by);
    prof_begin(KC_ROUND, s);
    k_round<T><<<nblk, 256, 0, s>>>(a, D);
    prof_end(KC_ROUND, s, fl, by);
    if (!push_work(m, n, D, Mb, Nb, es, &fl, &by)) continue;
    if ((e = hipEventRecord(ev_round[D], s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(s1, ev_round[D], 0)) != hipSuccess) return e;
    prof_begin(KC_FAR, s1);
    k_push<T><<<dim3(maxt, nblk, 2), 256, 0, s1>>>(a, D);
    prof_end(KC_FAR, s1, fl, by);
    if ((e = hipEventRecord(ev_far[D], s1)) != hipSuccess) return e;
    far_list.push_back(D);
    last_far = D;
  }
  // the call completes on the caller's stream only after the second stream drains
  if (last_far >= 0 && (e = hipStreamWaitEvent(s, ev_far[last_far], 0)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

size_t sweep_workspace(int64_t m, int64_t n, int dtype) {
  const size_t es = dtype == 0 ? sizeof(float) : sizeof(double);
  return 4 * align_up((size_t)m * n * es);
}

hipError_t sweep_enqueue(int64_t m, int64_t n, int bits, int dtype, const void* W,
                         const void* Ua, const void* Ub, const void* scales, int8_t* codes,
                         void* Q, void* ws, int* info, hipStream_t s) {
  if (dtype == 0)
    return sweep_typed<float>(m, n, bits, (const float*)W, (const float*)Ua, (const float*)Ub,
                              (const float*)scales, codes, (float*)Q, ws, info, s);
  return sweep_typed<double>(m, n, bits, (const double*)W, (const double*)Ua, (const double*)Ub,
                             (const double*)scales, codes, (double*)Q, ws, info, s);
}

}  // namespace g2d
