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
  T sup[BB][2];          // sup[c] = (U'b[c-2][c], U'b[c-1][c]) inside c's micro-tile
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
// Two consecutive elements (aligned to their pair size).
template <typename T>
struct Vec2 {
  T v[2];
};
__device__ inline Vec2<float> lds_read2(const float* p) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 x = *(const f2*)p;
  return Vec2<float>{{x[0], x[1]}};
}
__device__ inline Vec2<double> lds_read2(const double* p) {
  typedef double d2 __attribute__((ext_vector_type(2)));
  const d2 x = *(const d2*)p;
  return Vec2<double>{{x[0], x[1]}};
}

// LDS operands of one step of the micro sweep for lane (r, q) at column l: the quarter's
// four R values of column l (rows 4q..4q+3), its four Delta values of row r and the four
// U'b entries of column l (rows 4q..4q+3), and the two superdiagonal factors of column l.
template <typename T>
struct StepOps {
  Vec4<T> rv, dv, bv;
  Vec2<T> sp;
};

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
  // coupling to columns of an earlier micro-tile is applied by the MFMA pulls, so the
  // table is zero where l-1 or l-2 falls outside l's micro-tile
  if (tid < BB) {
    const int lm = tid & (MU - 1);
    sm.sup[tid][0] = lm >= 2 ? sm.ubT[tid][tid - 2] : T(0);
    sm.sup[tid][1] = lm >= 1 ? sm.ubT[tid][tid - 1] : T(0);
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
  const T cup2 = (rr_ > 1) ? sm.ua[gr - 2][gr] : T(0);

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
      T g0r[MU], h0r[MU];
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
      const T* rtq = &sm.rT[mc0][MU * w + 4 * qq];  // + P * column
      const T* ddq = &sm.dd[gr][mc0 + 4 * qq];
      const T* ubq = &sm.ubT[mc0][mc0 + 4 * qq];    // + P * column
      const T* spq = &sm.sup[mc0][0];                // + 2 * column
      // Operands of step st are read during step st - 2.  At that point rows <= r - 3
      // (columns <= l - 3) are written and the two nearer ones still read as zero, so
      // the LDS sums hold exactly the older terms; rows r-1, r-2 and columns l-1, l-2
      // are added from registers (DPP row shifts and the lane's own previous Deltas).
      auto fetch = [&](int st2) {
        const int l2 = st2 - rr_;
        const int lc = (l2 >= 0 && l2 < MU) ? l2 : 0;
        StepOps<T> o;
        o.rv = lds_read4(rtq + P * lc);
        o.dv = lds_read4(ddq);
        o.bv = lds_read4(ubq + P * lc);
        o.sp = lds_read2(spq + 2 * lc);
        return o;
      };
      StepOps<T> x0 = fetch(0);
      StepOps<T> x1 = fetch(1);
      lds_wave_sync();
      // inactive lanes store into this wave's staging row, which is dead until the
      // next micro-tile
      T* dummy = &sm.h0s[w][rr_][0];
      T pv = T(0), ph = T(0);
      T rprev = T(0), rup = T(0), dprev = T(0), dprev2 = T(0);
#pragma unroll
      for (int st = 0; st < 2 * MU - 1; ++st) {
        const int l = st - rr_;
        const bool act = (l >= 0) && (l < MU);
        // (A) operands two steps ahead
        StepOps<T> x2;
        if (st + 2 < 2 * MU - 1) x2 = fetch(st + 2);
        // (B) critical chain of this step; the second-nearest terms are ready early
        const T pv2 = pv + cup2 * up_row(rup);      // + U'a[r-2][r] R[r-2][l]
        const T ph2 = ph + x0.sp.v[0] * dprev2;     // + Delta[r][l-2] U'b[l-2][l]
        rup = up_row(rprev);                        // R[r-1][l]
        const T g = g0r[st & (MU - 1)] - (pv2 + cup * rup);
        const T hh = h0r[st & (MU - 1)] + (ph2 + x0.sp.v[1] * dprev);
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
        dprev2 = dprev;
        dprev = dv_new;
        // (C) the next step's terms other than its nearest row and column
        if (st + 1 < 2 * MU - 1) {
          T sv = T(0), sh = T(0);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            sv += cu[u] * x1.rv.v[u];
            sh += x1.dv.v[u] * x1.bv.v[u];
          }
          pv = quad_sum(sv);
          ph = quad_sum(sh);
        }
        x0 = x1;
        x1 = x2;
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

// Depth of one LDS stage of the push GEMM: 32 doubles or 64 floats per chunk of k-rows,
// so both element types stage the same number of bytes.
template <typename T>
struct PushKc;
template <>
struct PushKc<float> {
  static constexpr int v = 64;
};
template <>
struct PushKc<double> {
  static constexpr int v = 32;
};
// LDS row strides (elements) of the staged operands: a multiple of 16 plus 16, so the
// four k-rows read by one MFMA operand load start 32 dwords (f64) or 16 dwords (f32)
// apart and fall in different banks.
constexpr int kPanel = 2;                   // target blocks per push task
constexpr int kPadWide = kPanel * 64 + 16;  // panel-wide operand
constexpr int kPadNarrow = 64 + 16;         // 64-wide operand
constexpr int kPushThreads = 512;
constexpr int kNearPanels = (3 + kPanel - 1) / kPanel;  // near targets: at most three
template <typename T>
struct PushSmem {
  static constexpr int KC = PushKc<T>::v;
  // A rows, then B rows; also the 64 x 130 transpose stage of the epilogue
  static constexpr int kElems = KC * (kPadWide + kPadNarrow) > 64 * 130 ? KC * (kPadWide + kPadNarrow) : 64 * 130;
  T buf[kElems];
  int task;
};

// G[x][y] = sum_{k<K} A[k*lda + x] B[k*ldb + y] for x < M <= BM, y < N <= 64 (BM = 128
// or 256), both operands k-major, added into C: C[x*ldc + y] += G[x][y], or with `trans`
// C[y*ldc + x] += G[x][y].  One workgroup of eight waves, two per SIMD; wave w owns rows
// x in [w BM/8, (w+1) BM/8) as (BM/128) x 4 MFMA tiles.  Operands are staged through LDS KC k-rows at a
// time, with the next chunk's global loads in flight in registers while the current
// chunk is multiplied.  k-rows past K read as zero (exact buffer ranges); rows or
// columns past M, N read neighbouring finite data that only reaches outputs that are
// never stored.  The transposed update goes through LDS so that its stores are
// coalesced along x.
template <typename T, int BM>
__device__ inline void panel_gemm(const T* A, int64_t lda, const T* B, int64_t ldb, T* C,
                                  int64_t ldc, int M, int N, int K, bool trans,
                                  PushSmem<T>& sm) {
  typedef typename Mfma<T>::acc_t acc_t;
  constexpr int BN = 64;
  static_assert(BM == 128 || BM == 256, "panel width");
  constexpr int KC = PushKc<T>::v;
  constexpr int SA = BM + 16, SB = kPadNarrow;
  static_assert(SA <= kPadWide, "stage layout");
  constexpr int TH = kPushThreads;
  constexpr int NA = KC * BM / TH, NB = KC * BN / TH;  // staged elements per thread
  constexpr int TM = BM / 128, TN = 4;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi0 = (BM / 8) * w;
  const int kq = lane >> 4, cl = lane & 15;
  const int64_t es = sizeof(T);
  const rsrc_t ra = make_rsrc(A, ((int64_t)(K - 1) * lda + M) * es);
  const rsrc_t rb = make_rsrc(B, ((int64_t)(K - 1) * ldb + N) * es);
  const int nch = (K + KC - 1) / KC;
  // thread tid stages elements tid + TH u of each chunk: k-row tid / BM + u (TH / BM),
  // column tid % BM; the per-u and per-chunk parts of the offset are wave-uniform
  const uint32_t va = (uint32_t)((tid / BM) * lda + tid % BM);
  const uint32_t vb = (uint32_t)((tid / BN) * ldb + tid % BN);
  T pa[NA], pb[NB];
  auto fetch = [&](int c) {
#pragma unroll
    for (int u = 0; u < NA; ++u)
      pa[u] = buf_load_s<T>(ra, va, (uint32_t)((c * KC + u * (TH / BM)) * lda));
#pragma unroll
    for (int u = 0; u < NB; ++u)
      pb[u] = buf_load_s<T>(rb, vb, (uint32_t)((c * KC + u * (TH / BN)) * ldb));
  };
  T* const as0 = sm.buf + (tid / BM) * SA + tid % BM;
  T* const bs0 = sm.buf + SA * KC + (tid / BN) * SB + tid % BN;
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < NA; ++u) as0[u * (TH / BM) * SA] = pa[u];
#pragma unroll
    for (int u = 0; u < NB; ++u) bs0[u * (TH / BN) * SB] = pb[u];
  };
  acc_t acc[TM][TN];
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y) acc[x][y] = acc_t{0, 0, 0, 0};
  auto multiply = [&]() {
    const T* as = sm.buf;
    const T* bs = sm.buf + SA * KC;
#pragma unroll 2
    for (int ks = 0; ks < KC / 4; ++ks) {
      T fa[TM], fb[TN];
#pragma unroll
      for (int x = 0; x < TM; ++x) fa[x] = as[(4 * ks + kq) * SA + wi0 + 16 * x + cl];
#pragma unroll
      for (int y = 0; y < TN; ++y) fb[y] = bs[(4 * ks + kq) * SB + 16 * y + cl];
#pragma unroll
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y) acc[x][y] = Mfma<T>::run(fa[x], fb[y], acc[x][y]);
    }
  };
  fetch(0);
  stage();
  __syncthreads();
  // no branches in the loop body (keeps the accumulators in place); the fetch after the
  // last chunk reads past K, i.e. zeros, without touching memory
  for (int c = 0; c < nch; ++c) {
    fetch(c + 1);
    multiply();
    __syncthreads();
    stage();
    __syncthreads();
  }
  if (!trans) {
    const rsrc_t rc = make_rsrc(C, ((int64_t)(M - 1) * ldc + N) * es);
#pragma unroll
    for (int x = 0; x < TM; ++x) {
      T old[TN][4];
#pragma unroll
      for (int y = 0; y < TN; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = wi0 + 16 * x + Mfma<T>::row(lane, e), j = 16 * y + cl;
          old[y][e] = buf_load<T>(rc, (uint32_t)((int64_t)i * ldc + j));
        }
#pragma unroll
      for (int y = 0; y < TN; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = wi0 + 16 * x + Mfma<T>::row(lane, e), j = 16 * y + cl;
          if (i < M && j < N) C[(int64_t)i * ldc + j] = old[y][e] + acc[x][y][e];
        }
    }
    return;
  }
  // transposed: halves of 128 x-values; the owners write G^T into LDS (pitch 130), then
  // every thread updates whole C rows
  constexpr int PT = 128 + 2;
  static_assert(64 * PT <= PushSmem<T>::kElems, "transpose stage");
  const rsrc_t rc = make_rsrc(C, ((int64_t)(N - 1) * ldc + M) * es);
#pragma unroll
  for (int h = 0; h < BM / 128; ++h) {
    if (wi0 / 128 == h) {
#pragma unroll
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int xi = wi0 - 128 * h + 16 * x + Mfma<T>::row(lane, e), yj = 16 * y + cl;
            sm.buf[yj * PT + xi] = acc[x][y][e];
          }
    }
    __syncthreads();
#pragma unroll 4
    for (int u = 0; u < 64 * 128 / TH; ++u) {
      const int idx = tid + TH * u, yj = idx >> 7, xi = idx & 127;
      const int x = 128 * h + xi;
      const T old = buf_load<T>(rc, (uint32_t)((int64_t)yj * ldc + x));
      if (x < M && yj < N) C[(int64_t)yj * ldc + x] = old + sm.buf[yj * PT + xi];
    }
    __syncthreads();
  }
}

// Band pushes of the blocks on diagonal D that later diagonals do not pull themselves.
// Vertical (into Vf) from block (K, L) to row blocks t >= K+2 of column L, horizontal
// (into Hf) from (K, L) to column blocks t >= L+2 of row K.  Targets up to the first
// block of the next outer block take the 64-deep panel of (K, L) ("near": at most three
// targets); beyond that, a block that closes an outer block pushes the whole outer
// block, 256 deep.  Tasks cover kPanel target blocks each.  Workgroups take tasks
// (panel, direction, source block) from a queue, far panels first; each target tile is
// written by one task, so the order of tasks does not matter for the result.
template <typename T>
__global__ __launch_bounds__(kPushThreads) void k_push(SweepArgs<T> a, int D, int ntask, int P,
                                                       int* queue) {
  __shared__ PushSmem<T> sm;
  const int kmin = D - (a.Nb - 1) > 0 ? D - (a.Nb - 1) : 0;
  const int nblk2 = ntask / P;  // source blocks x 2 directions
  const int64_t m = a.m, n = a.n;
  for (;;) {
    __syncthreads();  // sm.task and the staging area are free
    if (threadIdx.x == 0) sm.task = atomicAdd(queue + D, 1);
    __syncthreads();
    const int task = sm.task;
    if (task >= ntask) break;
    const int panel = P - 1 - task / nblk2, rest = task % nblk2, dir = rest & 1;
    const int K = kmin + (rest >> 1), L = D - K;
    const int own = dir == 0 ? K : L;                // source block index along the push
    const int nt = dir == 0 ? a.Mb : a.Nb;           // blocks along the push
    const int first_next = GOUT * (own / GOUT + 1);  // first block of the next outer block
    const int64_t ext = dir == 0 ? m : n;
    int t0, t1, ks;
    int64_t src0;
    if (panel < kNearPanels) {
      const int nlast = first_next < nt - 1 ? first_next : nt - 1;
      t0 = own + 2 + kPanel * panel;
      t1 = t0 + kPanel - 1 < nlast ? t0 + kPanel - 1 : nlast;
      src0 = (int64_t)own * BB;
      ks = (ext - src0) < BB ? (int)(ext - src0) : BB;
    } else {
      if (own % GOUT != GOUT - 1) continue;
      t0 = first_next + 1 + kPanel * (panel - kNearPanels);
      t1 = t0 + kPanel - 1 < nt - 1 ? t0 + kPanel - 1 : nt - 1;
      src0 = (int64_t)(own - (GOUT - 1)) * BB;
      ks = GOUT * BB;
    }
    if (t0 > t1) continue;
    const int64_t p0 = (int64_t)t0 * BB;  // first pushed row (dir 0) or column (dir 1)
    const int64_t pend = (int64_t)(t1 + 1) * BB < ext ? (int64_t)(t1 + 1) * BB : ext;
    const int PW = (int)(pend - p0);      // <= 64 kPanel
    // vertical: Vf[p0 + x][c0 + y] += sum_k U'a[src0 + k][p0 + x] R[src0 + k][c0 + y];
    // horizontal: Hf[r0 + y][p0 + x] += sum_k U'b[src0 + k][p0 + x] Delta^T[src0 + k][r0 + y]
    const int64_t q0 = (int64_t)(dir == 0 ? L : K) * BB;  // the source block's other side
    const int64_t qext = dir == 0 ? n : m;
    const int QW = (qext - q0) < BB ? (int)(qext - q0) : BB;
    const T* pa = dir == 0 ? a.Ua : a.Ub;
    const T* pb = dir == 0 ? a.R : a.DT;
    const int64_t ldb = dir == 0 ? n : m;
    T* pc = dir == 0 ? a.Vf + p0 * n + q0 : a.Hf + q0 * n + p0;
    panel_gemm<T, 64 * kPanel>(pa + src0 * ext + p0, ext, pb + src0 * ldb + q0, ldb, pc, n, PW,
                               QW, ks, dir != 0, sm);
  }
}

// Vf = Hf = 0 and the push queues (one counter per diagonal) = 0.
template <typename T>
__global__ __launch_bounds__(256) void k_init(int64_t count, T* Vf, T* Hf, int nq, int* queue) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256) {
    Vf[i] = T(0);
    Hf[i] = T(0);
  }
  for (int i = blockIdx.x * 256 + threadIdx.x; i < nq; i += gridDim.x * 256) queue[i] = 0;
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
  int* queue = (int*)c;  // [Mb + Nb - 1] push-task counters
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
  hipStream_t sr = s, sp = s1;
  const bool pr = prof_on();
  const double es = (double)sizeof(T);
  prof_begin(KC_OTHER, s);
  k_check_scales<T><<<(unsigned)cdiv(m, 256), 256, 0, s>>>(m, scales, info);
  const int64_t ig = cdiv((int64_t)mn, 256) < 8192 ? cdiv((int64_t)mn, 256) : 8192;
  k_init<T><<<(unsigned)ig, 256, 0, s>>>((int64_t)mn, a.Vf, a.Hf, nD, queue);
  prof_end(KC_OTHER, s, 0.0, es * (2.0 * (double)mn + (double)m));
  if ((e = hipEventRecord(ev_init, s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sp, ev_init, 0)) != hipSuccess) return e;

  int last_far = -1;
  const int maxt = (Mb > Nb ? Mb : Nb);
  // push panels per (source block, direction): near panels + far panels of kPanel blocks
  const int P = kNearPanels + (maxt + kPanel - 1) / kPanel;
  // The push GEMM holds more LDS than a CU can share with a rounding block, so capping
  // its grid at (CUs - blocks of the longest diagonal) keeps CUs free for the rounding
  // chain, whose latency-bound waves would otherwise share their SIMDs.
  int push_grid = 0;
  {
    int dev = 0, ncu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) !=
        hipSuccess)
      return e;
    const int maxblk = Mb < Nb ? Mb : Nb;
    const int keep = maxblk < ncu / 2 ? maxblk : ncu / 2;
    push_grid = ncu - keep > 1 ? ncu - keep : 1;
  }
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
      if ((e = hipStreamWaitEvent(sr, ev_far[waited], 0)) != hipSuccess) return e;
    }
    double fl = 0.0, by = 0.0;
    if (pr) round_work(m, n, D, Mb, Nb, es, &fl, &by);
    prof_begin(KC_ROUND, sr);
    k_round<T><<<nblk, 256, 0, sr>>>(a, D);
    prof_end(KC_ROUND, sr, fl, by);
    if (!push_work(m, n, D, Mb, Nb, es, &fl, &by)) continue;
    if ((e = hipEventRecord(ev_round[D], sr)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(sp, ev_round[D], 0)) != hipSuccess) return e;
    const int ntask = nblk * 2 * P;
    const int grid = ntask < push_grid ? ntask : push_grid;
    prof_begin(KC_FAR, sp);
    k_push<T><<<grid, kPushThreads, 0, sp>>>(a, D, ntask, P, queue);
    prof_end(KC_FAR, sp, fl, by);
    if ((e = hipEventRecord(ev_far[D], sp)) != hipSuccess) return e;
    far_list.push_back(D);
    last_far = D;
  }
  // the call completes on the caller's stream only after the push stream drains
  if (last_far >= 0 && (e = hipStreamWaitEvent(s, ev_far[last_far], 0)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace

size_t sweep_workspace(int64_t m, int64_t n, int dtype) {
  const size_t es = dtype == 0 ? sizeof(float) : sizeof(double);
  const size_t nD = (size_t)(cdiv(m, BB) + cdiv(n, BB) - 1);
  return 4 * align_up((size_t)m * n * es) + align_up(nD * sizeof(int));
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
