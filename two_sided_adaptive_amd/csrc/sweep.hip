// Sweep stage for gfx950: anti-diagonal two-sided adaptive rounding with
// separable band feedback, as one persistent kernel.
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
// Work decomposition (bands of 64 rows, 16 x 16 micro-tiles, 64-wide column blocks,
// outer blocks of four bands / blocks):
//   * A band worker (one workgroup, four waves) owns a band and walks its micro-columns
//     left to right.  Wave w owns micro-row w; at phase p it rounds micro-tile
//     (w, p - w), so the four waves form a skewed pipeline that follows the
//     anti-diagonals of the band.  The feedback a micro-tile needs is
//       - from its own rows and columns: applied entry by entry along its 31
//         anti-diagonal steps;
//       - from the band's earlier micro-rows (same micro-column) and from the previous
//         band (64 rows): MFMA products, the latter waiting on a per-band progress
//         counter of the band above;
//       - from the band's own micro-columns in the current and the previous column
//         block: MFMA products from the band's Delta history in LDS;
//       - from everything further away: accumulated vertical and horizontal feedback
//         buffers, filled by GEMM workers (one pair per class of task, below).
//     Consecutive bands therefore run one micro-column phase apart per wave: the
//     wavefront of the whole matrix advances one micro-tile anti-diagonal at a time.
//   * GEMM workers take band-update tasks from two queues that band workers fill when
//     they complete a 64 x 64 block: near tasks, 64 deep from one band (block) to the
//     targets up to the first block of the next outer block, and, when the block closes
//     an outer block, far tasks, 256 deep from the whole outer block to every target
//     beyond.  Within each class the contributions to one target tile are applied in
//     the order of their sources, so the result is deterministic.
// Every wait is bounded; a timeout aborts the sweep and reports info[0] = 4.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

#include "common.hpp"
#include "launch.hpp"
#include "prof.hpp"
#include "schedule.hpp"

namespace g2d {
namespace {

using namespace sched;  // task rules shared with the host-side schedule checker

constexpr int BB = 64;      // band height = block edge
constexpr int MU = 16;      // micro-tile edge
constexpr int kThreads = 256;
constexpr int kSpinLimit = 1 << 22;
// accelerator complex dies (XCDs), one L2 each: 8 on an MI355X in its default partition
// mode; the count of the device in use is queried at launch (SweepArgs::nxcd)
constexpr int kMaxXcd = 16;

// control words at the start of the sync area; the per-XCD words sit on their own
// 128-byte lines
enum Ctl : int {
  kAbort = 0,
  kLine = 32,                       // ints per 128-byte line
  kHead = kLine,                    // + kLine c: next slot of queue c to claim
  kTail = kLine * 4,                // + kLine c: slots of queue c reserved by producers
  kBandX = kLine * 7,               // + kLine x: bands claimed by workgroups on XCD x
  kXTicket = kLine * (7 + kMaxXcd),    // + kLine x: workgroups started on XCD x
  kCtlWords = kLine * (7 + 2 * kMaxXcd)
};
// (band-update classes near / next / far: schedule.hpp)

// Cache policy of loads and stores that other workgroups of the same launch produce or
// consume: device scope (sc1), so they bypass the non-coherent caches.
constexpr int kDev = 16;

template <typename T>
struct SweepArgs {
  int64_t m, n;
  int Mb, Nb, Nj, lo, hi, bits;
  int qcap[NCLS]; // band-update tasks of each class in the whole sweep
  int nxcd;   // XCDs of the device (<= kMaxXcd)
  int nbxcd;  // band workers per XCD
  int gs;     // bands are dealt to the XCDs in groups of gs consecutive bands
  int near_mod;  // of the workgroups past the band workers, one in near_mod takes near tasks
  const T* Ua;
  const T* Ub;
  const T* s;
  const T* W;
  T* Vacc[NCLS];  // vertical feedback pushed by GEMM workers (subtracted from W), per class
  T* Hacc[NCLS];  // horizontal feedback pushed by GEMM workers, per class
  T* R;    // vertical residual, row-major m x n
  T* DT;   // Delta transposed, n x m
  int8_t* codes;
  T* Q;
  int* info;
  int* ctl;                  // kCtlWords control words
  int* rdone;                // [Mb] micro-columns of each band whose R is stored
  int* vcnt[NCLS];              // [Mb * Nb] per class: contributions applied, per 64 x 64 tile
  int* hcnt[NCLS];              // [Mb * Nb] per class, horizontal
  unsigned long long* qd[NCLS]; // [qcap] per class: task descriptors (0 = not yet published)
  unsigned long long* stats; // band-update task accounting while profiling, else null
};

// descriptor: bit 63 valid | 62 far | 61 horizontal | [45,60) own | [30,45) other |
// [15,30) last target | [0,15) first target
__device__ inline unsigned long long pack_task(bool far, int dir, int own, int other, int t0,
                                               int t1) {
  return (1ull << 63) | ((unsigned long long)far << 62) | ((unsigned long long)dir << 61) |
         ((unsigned long long)own << 45) | ((unsigned long long)other << 30) |
         ((unsigned long long)t1 << 15) | (unsigned long long)t0;
}

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
__device__ inline int ld_dev(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline bool aborted(const int* ctl) { return ld_dev(ctl + kAbort) != 0; }
// XCD (accelerator complex die) this wave runs on: hardware register XCC_ID
// (hardware register XCC_ID; a partition of the device numbers its XCDs from any base, so
// the id is taken modulo the partition's XCD count)
__device__ inline int xcd_id(int nxcd) {
  return (int)__builtin_amdgcn_s_getreg((3 << 11) | 20) % nxcd;
}
__device__ inline void abort_sweep(int* ctl, int* info) {
  if (atomicCAS(ctl + kAbort, 0, 1) == 0) record_info(info, 4, 0);
}

// Whole-wave wait until *p >= v.  False if the sweep is aborted (or this wait times
// out, which aborts it).
__device__ inline bool wait_ge(const int* p, int v, int* ctl, int* info) {
  for (int it = 0;; ++it) {
    const int x = __builtin_amdgcn_readfirstlane(ld_dev(p));
    if (x >= v) return true;
    if ((it & 15) == 15) {
      if (aborted(ctl)) return false;
      if (it > kSpinLimit) {
        if ((threadIdx.x & 63) == 0) abort_sweep(ctl, info);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Orders this wave's memory operations for the compiler (the hardware keeps a wave's
// LDS operations in issue order).
__device__ inline void lds_wave_sync() { __asm__ volatile("" ::: "memory"); }
// Waits until every memory operation this wave issued has completed.
__device__ inline void drain() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
}

template <typename T>
__device__ inline T buf_load_dev(rsrc_t r, uint32_t elem);
template <>
__device__ inline float buf_load_dev<float>(rsrc_t r, uint32_t elem) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, elem * 4u, 0, kDev));
}
template <>
__device__ inline double buf_load_dev<double>(rsrc_t r, uint32_t elem) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, elem * 8u, 0, kDev);
  return __hiloint2double((int)v[1], (int)v[0]);
}
// Load that bypasses the CU's L1 but may hit the XCD's L2 (data stored through that L2
// by a workgroup of the same XCD).
constexpr int kL2 = 1;
template <typename T>
__device__ inline T buf_load_l2(rsrc_t r, uint32_t elem);
template <>
__device__ inline float buf_load_l2<float>(rsrc_t r, uint32_t elem) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, elem * 4u, 0, kL2));
}
template <>
__device__ inline double buf_load_l2<double>(rsrc_t r, uint32_t elem) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, elem * 8u, 0, kL2);
  return __hiloint2double((int)v[1], (int)v[0]);
}
template <typename T>
__device__ inline void buf_store_dev(T v, rsrc_t r, uint32_t elem);
template <>
__device__ inline void buf_store_dev<float>(float v, rsrc_t r, uint32_t elem) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, elem * 4u, 0, kDev);
}
template <>
__device__ inline void buf_store_dev<double>(double v, rsrc_t r, uint32_t elem) {
  typedef unsigned int u2 __attribute__((ext_vector_type(2)));
  const u2 x = {(unsigned)__double2loint(v), (unsigned)__double2hiint(v)};
  __builtin_amdgcn_raw_buffer_store_b64(x, r, elem * 8u, 0, kDev);
}
template <typename T>
__device__ inline T buf_load_s_dev(rsrc_t r, uint32_t elem, uint32_t uelem);
template <>
__device__ inline float buf_load_s_dev<float>(rsrc_t r, uint32_t elem, uint32_t uelem) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, elem * 4u, uelem * 4u, kDev));
}
template <>
__device__ inline double buf_load_s_dev<double>(rsrc_t r, uint32_t elem, uint32_t uelem) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, elem * 8u, uelem * 8u, kDev);
  return __hiloint2double((int)v[1], (int)v[0]);
}

__device__ inline float rint_t(float x) { return rintf(x); }
__device__ inline double rint_t(double x) { return rint(x); }
__device__ inline float abs_t(float x) { return fabsf(x); }
__device__ inline double abs_t(double x) { return fabs(x); }
__device__ inline float min_t(float a, float b) { return fminf(a, b); }
__device__ inline double min_t(double a, double b) { return fmin(a, b); }
__device__ inline float max_t(float a, float b) { return fmaxf(a, b); }
__device__ inline double max_t(double a, double b) { return fmax(a, b); }

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

// ---------------------------------------------------------------------------
// band worker
// ---------------------------------------------------------------------------
// Row pitches keep 4-element groups 16-byte aligned for vector LDS reads.
template <typename T>
struct Pad;
template <>
struct Pad<float> {
  static constexpr int v = 4;
};
template <>
struct Pad<double> {
  static constexpr int v = 2;
};

template <typename T>
struct BandSmem {
  static constexpr int PR = BB + Pad<T>::v;  // pitch of a transposed R column
  static constexpr int PD = MU + Pad<T>::v;  // pitch of a Delta / U'b micro row
  T rT[4][MU][PR];         // R ring by micro-column j % 4, transposed: rT[.][c][band row]
  T dh[4][8][MU][PD];      // per wave, Delta ring by micro-column j % 8: dh[w][.][r][c]
  T ubT[4][MU][PD];        // per wave: diagonal micro-block of U'b, ubT[c][k] = U'b[k][c]
  T sup[4][MU][2];         // per wave: (U'b[c-2][c], U'b[c-1][c]) inside the micro-block
  T g0s[4][MU][MU];        // per wave, skewed: g0s[r][sl] = (W - G outside)[r][(sl - r) % 16]
  T h0s[4][MU][MU];        // per wave, skewed: H from outside; scratch during a sweep
  int8_t zz[4][MU][MU];    // per wave: codes of the micro-tile
  T sc[BB];                // the band's row scales (1 past the last row)
  int bcast[4];
};

// The loads of micro-tile (w, j) that do not depend on the phase before it: the U'b rows
// of its local window and its diagonal U'b block (k-major B operand), W, and the feedback
// pushed by the GEMM workers of every class (final once the block's counters are
// complete).  A band worker issues them one phase early, before the phase barrier, so
// that their latency passes during the barrier and the hand-over.
template <typename T>
struct TileLoads {
  T win[4];
  T vf[NCLS][4], hf[NCLS][4];
};
template <typename T>
struct UbLoads {
  T bwin[7 * MU / 4];
  T ubd[MU * MU / 64];
};
// The U'b operands of micro-column j (read by every band, so mostly from L2; loaded in
// the phase that uses them).
template <typename T>
__device__ inline void ub_loads(const SweepArgs<T>& a, int j, UbLoads<T>& ub) {
  const int64_t n = a.n;
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, cl = lane & 15;
  const int64_t c0 = (int64_t)j * MU;
  const int nc = (n - c0) < MU ? (int)(n - c0) : MU;
  const int L = j / GOUT;
  const int clo = GOUT * (L > 0 ? L - 1 : 0);
  const int nwin = j - clo;
  const int64_t es = sizeof(T);
  const rsrc_t rb = make_rsrc(a.Ub + (int64_t)clo * MU * n + c0,
                              nwin > 0 ? ((int64_t)(nwin * MU - 1) * n + nc) * es : 0);
#pragma unroll
  for (int s = 0; s < 7 * MU / 4; ++s)
    ub.bwin[s] = buf_load<T>(rb, (uint32_t)((4 * s + kq) * n + cl));
  const rsrc_t rd = make_rsrc(a.Ub + c0 * n + c0, ((int64_t)(nc - 1) * n + nc) * es);
#pragma unroll
  for (int u = 0; u < MU * MU / 64; ++u) {
    const int idx = lane + 64 * u, k = idx >> 4, c = idx & 15;
    ub.ubd[u] = buf_load<T>(rd, (uint32_t)(k * n + c));
  }
}
// parts: bit 0 W, bit 1 the pushed feedback
template <typename T>
__device__ inline void tile_loads(const SweepArgs<T>& a, int K, int w, int j, int parts,
                                  TileLoads<T>& ld) {
  const int64_t m = a.m, n = a.n;
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, cl = lane & 15;
  const int64_t r0 = (int64_t)K * BB;
  const int mr = (m - r0) < BB ? (int)(m - r0) : BB;
  const int64_t c0 = (int64_t)j * MU;
  const int nc = (n - c0) < MU ? (int)(n - c0) : MU;
  const int L = j / GOUT;
  const int clo = GOUT * (L > 0 ? L - 1 : 0);
  const int nwin = j - clo;
  const int64_t es = sizeof(T);
  const int64_t row0 = r0 + MU * w;
  const int rows = mr - MU * w;  // (<= 0 for a wave without rows: nothing is read)
  const int64_t tile_bytes = rows > 0 ? ((int64_t)(rows - 1) * n + nc) * es : 0;
  const int64_t o0 = rows > 0 ? row0 * n + c0 : 0;
  if (parts & 1) {
    const rsrc_t rw = make_rsrc(a.W + o0, tile_bytes);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ld.win[e] = buf_load<T>(rw, (uint32_t)(Mfma<T>::row(lane, e) * n + cl));
  }
  if (parts & 2) {
#pragma unroll
    for (int c = 0; c < NCLS; ++c) {
      const rsrc_t rvf =
          make_rsrc(a.Vacc[c] + o0, expected_class(K, c) > 0 ? tile_bytes : 0);
      const rsrc_t rhf =
          make_rsrc(a.Hacc[c] + o0, expected_class(L, c) > 0 ? tile_bytes : 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t o = (uint32_t)(Mfma<T>::row(lane, e) * n + cl);
        ld.vf[c][e] = buf_load_dev<T>(rvf, o);
        ld.hf[c][e] = buf_load_dev<T>(rhf, o);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCLS; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) ld.vf[c][e] = ld.hf[c][e] = T(0);
  }
}

// At the end of phase p (p = -1: before the first), wave w issues the loads of its
// micro-tile of phase p + 1, j = p + 1 - w (clamped into the band: ld is rewritten in
// full every phase, so that it is dead between its use and the next phase).  The pushed
// feedback is final once wave 0 has found the block's counters complete: wave 0 itself
// checked them unless the tile starts a block; a later wave needs that check in an
// earlier phase.  Returns whether the pushed feedback was loaded.
template <typename T>
__device__ inline bool prefetch_tile(const SweepArgs<T>& a, int K, int w, int p,
                                     TileLoads<T>& ld) {
  const int jn = p + 1 - w;
  const int jc = jn < 0 ? 0 : (jn >= a.Nj ? a.Nj - 1 : jn);
  const bool pushed = jn >= 0 && jn < a.Nj &&
                      (w == 0 ? jn % GOUT != 0 : GOUT * (jn / GOUT) < p);
  tile_loads<T>(a, K, w, jc, pushed ? 3 : 1, ld);
  return pushed;
}

// Rounds micro-tile (w, j) of band K and stores its R, Delta, codes and Q.  Its input
// loads were issued in the phase before (ld), and its pushed feedback too when `pre`.
// Only wave 0 polls the progress and
// contribution counters: a later wave reaches a micro-column or block at least one phase
// (a barrier) after wave 0 found it ready, and skipping the polls keeps their waits, which
// also wait for every load issued before them, off the other waves.
template <typename T>
__device__ inline void round_micro_tile(const SweepArgs<T>& a, BandSmem<T>& sm, int K, int w,
                                        int j, int& vblk, bool pre, TileLoads<T>& ld,
                                        const T (&aVn)[BB / 4], const T (&aVi)[3 * MU / 4],
                                        const T (&cu)[4], T cup, T cup2, T s_r, T rs_r) {
  typedef typename Mfma<T>::acc_t acc_t;
  constexpr int PR = BandSmem<T>::PR, PD = BandSmem<T>::PD;
  const int64_t m = a.m, n = a.n;
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4, cl = lane & 15;
  const int64_t r0 = (int64_t)K * BB;
  const int mr = (m - r0) < BB ? (int)(m - r0) : BB;
  const int64_t c0 = (int64_t)j * MU;
  const int nc = (n - c0) < MU ? (int)(n - c0) : MU;
  const int L = j / GOUT;  // 64-wide column block
  const int clo = GOUT * (L > 0 ? L - 1 : 0);  // first micro-column of the local window
  const int nwin = j - clo;                     // window micro-columns, 0..7
  const int s4 = j & 3, s8 = j & 7;
  const int64_t es = sizeof(T);

  // W and (inside a block) the pushed feedback were loaded in the phase before.  This
  // phase's loads are issued in the order they are consumed (the counter that tracks them
  // retires in order): the U'b window and diagonal block first; then, at a block's first
  // micro-tile, the pushed feedback of every class (once wave 0 has found the block's
  // contribution counters complete); last the R of the band above, whose product is
  // computed after the others so that its latency overlaps them.
  const int64_t row0 = r0 + MU * w;  // first row of this micro-tile
  const int rows = mr - MU * w;      // valid rows (1..16)
  const int64_t tile_bytes = ((int64_t)(rows - 1) * n + nc) * es;
  const int64_t o0 = row0 * n + c0;
  // wave 0's polls come before this phase's loads, so that they only wait for the loads
  // issued in the phase before
  if (w == 0) {
    if (!pre && vblk != L) {
      const int64_t tile = (int64_t)K * a.Nb + L;
#pragma unroll
      for (int c = 0; c < NCLS; ++c) {
        const int evc = expected_class(K, c), ehc = expected_class(L, c);
        if (evc > 0 && !wait_ge(a.vcnt[c] + tile, evc, a.ctl, a.info)) return;
        if (ehc > 0 && !wait_ge(a.hcnt[c] + tile, ehc, a.ctl, a.info)) return;
      }
      vblk = L;
    }
    if (K > 0 && !wait_ge(a.rdone + K - 1, j + 1, a.ctl, a.info)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  UbLoads<T> ub;
  ub_loads<T>(a, j, ub);
  if (!pre) tile_loads<T>(a, K, w, j, 2, ld);
  T gin[4], hin[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    gin[e] = ld.win[e];
    hin[e] = T(0);
  }
#pragma unroll
  for (int c = 0; c < NCLS; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gin[e] -= ld.vf[c][e];
      hin[e] += ld.hf[c][e];
    }
  const T(&bwin)[7 * MU / 4] = ub.bwin;
  const T(&ubd)[MU * MU / 64] = ub.ubd;
  // R of the band above (k-major B operand).  When that band lives on this XCD its stores
  // went through this L2, so the shared L2 serves it; otherwise it is read at device scope.
  // Only in fp64: there a micro-tile row is one whole 128-byte line (n a multiple of 16
  // and 16-element aligned rows), so no line holding it can have been cached before the
  // band above wrote all of it; an fp32 row is half a line.
  T bnb[BB / 4];
  {
    const rsrc_t rr = make_rsrc(K > 0 ? a.R + (r0 - BB) * n + c0 : a.R,
                                K > 0 ? ((int64_t)(BB - 1) * n + nc) * es : 0);
    if (sizeof(T) == 8 && n % MU == 0 && K % a.gs != 0) {
#pragma unroll
      for (int s = 0; s < BB / 4; ++s) bnb[s] = buf_load_l2<T>(rr, (uint32_t)((4 * s + kq) * n + cl));
    } else {
#pragma unroll
      for (int s = 0; s < BB / 4; ++s) bnb[s] = buf_load_dev<T>(rr, (uint32_t)((4 * s + kq) * n + cl));
    }
  }

  // this micro-tile's LDS: R ring rows and Delta slot start at zero; U'b diagonal block
#pragma unroll
  for (int u = 0; u < MU * MU / 64; ++u) {
    const int idx = lane + 64 * u, r = idx & 15, c = idx >> 4;
    sm.rT[s4][c][MU * w + r] = T(0);
    sm.dh[w][s8][c][r] = T(0);
    const int k = idx >> 4, cc = idx & 15;  // ubd[u] holds U'b[c0 + k][c0 + cc]
    sm.ubT[w][cc][k] = (k < cc && cc < nc) ? ubd[u] : T(0);
  }
  lds_wave_sync();
  if (lane < MU) {
    sm.sup[w][lane][0] = lane >= 2 ? sm.ubT[w][lane][lane - 2] : T(0);
    sm.sup[w][lane][1] = lane >= 1 ? sm.ubT[w][lane][lane - 1] : T(0);
  }

  // feedback from outside the micro-tile (MFMA), two chains per product
  {
    // The LDS operands of each pair of products are read one pair ahead, before the
    // (wave-uniform) test that skips the pair, so that a read's latency passes while the
    // products before it run.  (Reads past the pairs a wave uses return data it ignores.)
    acc_t v0 = acc_t{0, 0, 0, 0}, v1 = acc_t{0, 0, 0, 0};
    // earlier micro-rows of this band, same micro-column (written in earlier phases)
    {
      T r0 = sm.rT[s4][cl][kq], r1 = sm.rT[s4][cl][4 + kq];
#pragma unroll
      for (int s = 0; s < 3 * MU / 4; s += 2) {
        const T c0 = r0, c1 = r1;
        if (s + 2 < 3 * MU / 4) {
          r0 = sm.rT[s4][cl][4 * s + 8 + kq];
          r1 = sm.rT[s4][cl][4 * s + 12 + kq];
        }
        if (s < 4 * w) {
          v0 = Mfma<T>::run(aVi[s], c0, v0);
          v1 = Mfma<T>::run(aVi[s + 1], c1, v1);
        }
      }
    }
    acc_t h0 = acc_t{0, 0, 0, 0}, h1 = acc_t{0, 0, 0, 0};
    // the band's Delta over the window columns (this wave's rows) times U'b
    {
      auto dop = [&](int k) { return sm.dh[w][(clo + (k >> 4)) & 7][cl][k & 15]; };
      T d0 = dop(kq), d1 = dop(4 + kq);
#pragma unroll
      for (int s = 0; s < 7 * MU / 4; s += 2) {
        const T c0 = d0, c1 = d1;
        if (s + 2 < 7 * MU / 4) {
          d0 = dop(4 * s + 8 + kq);
          d1 = dop(4 * s + 12 + kq);
        }
        if (s < 4 * nwin) {
          h0 = Mfma<T>::run(c0, bwin[s], h0);
          h1 = Mfma<T>::run(c1, bwin[s + 1], h1);
        }
      }
    }
    // the band above last: its loads were issued last
    if (K > 0) {
#pragma unroll
      for (int s = 0; s < BB / 4; s += 2) {
        v0 = Mfma<T>::run(aVn[s], bnb[s], v0);
        v1 = Mfma<T>::run(aVn[s + 1], bnb[s + 1], v1);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      gin[e] -= v0[e] + v1[e];
      hin[e] += h0[e] + h1[e];
    }
  }
  // skewed staging: slot sl of row r holds column (sl - r) mod 16
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = Mfma<T>::row(lane, e), col = cl;
    sm.g0s[w][row][(col + row) & (MU - 1)] = gin[e];
    sm.h0s[w][row][(col + row) & (MU - 1)] = hin[e];
  }
  lds_wave_sync();

  // micro sweep lane layout: lane = 4 r + q (row r of the micro-tile, quarter q)
  const int rr_ = lane >> 2, qq = lane & 3;
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
  const T tlo = T(a.lo), thi = T(a.hi);
  const T tol = T(4) * Eps<T>::v * T(1 << (a.bits));
  const T* rtq = &sm.rT[s4][0][MU * w + 4 * qq];  // + PR * column
  const T* ddq = &sm.dh[w][s8][rr_][4 * qq];
  const T* ubq = &sm.ubT[w][0][4 * qq];          // + PD * column
  const T* spq = &sm.sup[w][0][0];                // + 2 * column
  // Operands of step st are read during step st - 2.  At that point rows <= r - 3
  // (columns <= l - 3) are written and the two nearer ones still read as zero, so
  // the LDS sums hold exactly the older terms; rows r-1, r-2 and columns l-1, l-2
  // are added from registers (DPP row shifts and the lane's own previous Deltas).
  auto fetch = [&](int st2) {
    const int l2 = st2 - rr_;
    const int lc = (l2 >= 0 && l2 < MU) ? l2 : 0;
    StepOps<T> o;
    o.rv = lds_read4(rtq + PR * lc);
    o.dv = lds_read4(ddq);
    o.bv = lds_read4(ubq + PD * lc);
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
    T* prt = act ? &sm.rT[s4][lw][MU * w + rr_] : dummy;
    T* pdd = act ? &sm.dh[w][s8][rr_][lw] : dummy + 1;
    int8_t* pzz = act ? &sm.zz[w][rr_][lw] : (int8_t*)(dummy + 2);
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

  // R row-major and Delta transposed (read by other workgroups), codes and Q
  const rsrc_t rro = make_rsrc(a.R + o0, tile_bytes);
  const rsrc_t rdt = make_rsrc(a.DT + c0 * m + row0, ((int64_t)(nc - 1) * m + rows) * es);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = cl, r = kq + 4 * u;  // consecutive lanes along a row
    if (r < rows && c < nc) {
      const int64_t o = o0 + (int64_t)r * n + c;
      buf_store_dev<T>(sm.rT[s4][c][MU * w + r], rro, (uint32_t)(r * n + c));
      const int z = sm.zz[w][r][c];
      a.codes[o] = (int8_t)z;
      a.Q[o] = sm.sc[MU * w + r] * T(z);
    }
    const int r2 = cl, c2 = kq + 4 * u;  // consecutive lanes along a column
    if (r2 < rows && c2 < nc) buf_store_dev<T>(sm.dh[w][s8][r2][c2], rdt, (uint32_t)(c2 * m + r2));
  }
}

// Publishes the band-update tasks of completed block (K, L): the tasks of class c go to
// queue slots base[c]... (base[c] is lane c's value of `base`); within a class vertical
// panels come first.  The lanes of one wave write the descriptors in parallel.
template <typename T>
__device__ inline void publish_block(const SweepArgs<T>& a, int K, int L, int base, int lane) {
  // six groups (class, direction): first target, last target, panel count
  int g0[6], g1[6], np[6];
  block_groups(K, L, a.Mb, a.Nb, g0, g1, np);
  int total = 0;
#pragma unroll
  for (int g = 0; g < 6; ++g) total += np[g];
  int bs[NCLS];
#pragma unroll
  for (int c = 0; c < NCLS; ++c) bs[c] = __builtin_amdgcn_readlane(base, c);
  for (int i = lane; i < total; i += 64) {
    // group of item i and its index in the group, by constant-indexed selects
    int g = 0, k = i, t0 = 0, t1 = 0, slot = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q)
      if (g == q && k >= np[q]) {
        k -= np[q];
        g = q + 1;
      }
#pragma unroll
    for (int q = 0; q < 6; ++q)
      if (g == q) {
        t0 = g0[q];
        t1 = g1[q];
        slot = bs[q >> 1] + ((q & 1) ? np[q - 1] : 0);  // after the class's vertical panels
      }
    const int cls = g >> 1, dir = g & 1;
    const int p0 = t0 + kPanel * k;
    const int p1 = p0 + kPanel - 1 < t1 ? p0 + kPanel - 1 : t1;
    const int own = dir == 0 ? K : L, other = dir == 0 ? L : K;
    __hip_atomic_store(a.qd[cls] + slot + k, pack_task(cls != kNear, dir, own, other, p0, p1),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T>
// (inlined into the kernel: as a call it would take the kernel arguments through memory)
__device__ __attribute__((always_inline)) inline void band_worker(const SweepArgs<T>& a,
                                                                  BandSmem<T>& sm) {
  const int64_t m = a.m;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = lane >> 4, cl = lane & 15;
  const int rr_ = lane >> 2, qq = lane & 3;
  const int64_t es = sizeof(T);
  for (;;) {
    __syncthreads();
    // bands go to the XCDs in groups of gs consecutive bands, so a band usually has the
    // band above it on its own XCD and reads its R from the shared L2
    if (tid == 0) {
      int K = a.Mb;
      if (!aborted(a.ctl)) {
        const int x = xcd_id(a.nxcd), c = atomicAdd(a.ctl + kBandX + kLine * x, 1);
        K = a.gs * (x + a.nxcd * (c / a.gs)) + c % a.gs;
      }
      sm.bcast[0] = K < a.Mb ? K : a.Mb;
    }
    __syncthreads();
    const int K = sm.bcast[0];
    if (K >= a.Mb) return;
    const int64_t r0 = (int64_t)K * BB;
    const int mr = (m - r0) < BB ? (int)(m - r0) : BB;
    const int nw = (mr + MU - 1) / MU;  // waves with rows
    // band constants of this wave: U'a blocks as MFMA A fragments, in-micro-tile
    // vertical coefficients, the row's scale
    // U'a rows of the band above and of this band, columns of this band
    const rsrc_t rnb = make_rsrc(K > 0 ? a.Ua + (r0 - BB) * m + r0 : a.Ua,
                                 K > 0 ? ((int64_t)(BB - 1) * m + mr) * es : 0);
    const rsrc_t rbd = make_rsrc(a.Ua + r0 * m + r0, ((int64_t)(mr - 1) * m + mr) * es);
    const int colw = MU * w + cl;  // band row of this lane's MFMA output column
    T aVn[BB / 4], aVi[3 * MU / 4];
#pragma unroll
    for (int s = 0; s < BB / 4; ++s) aVn[s] = buf_load<T>(rnb, (uint32_t)((4 * s + kq) * m + colw));
#pragma unroll
    for (int s = 0; s < 3 * MU / 4; ++s)
      aVi[s] = s < 4 * w ? buf_load<T>(rbd, (uint32_t)((4 * s + kq) * m + colw)) : T(0);
    const int gr = MU * w + rr_;  // band row of this lane in the micro sweep
    const bool rowok = gr < mr;
    T cu[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = MU * w + 4 * qq + u;
      const T v = buf_load<T>(rbd, (uint32_t)((int64_t)i * m + gr));
      cu[u] = (rowok && i < gr) ? v : T(0);
    }
    // (row -1 and -2 offsets wrap past the range and read zero)
    const T cup0 = buf_load<T>(rbd, (uint32_t)((int64_t)(gr - 1) * m + gr));
    const T cup20 = buf_load<T>(rbd, (uint32_t)((int64_t)(gr - 2) * m + gr));
    const T cup = (rowok && rr_ > 0) ? cup0 : T(0);
    const T cup2 = (rowok && rr_ > 1) ? cup20 : T(0);
    const T sv0 = buf_load<T>(make_rsrc(a.s + r0, (int64_t)mr * es), (uint32_t)gr);
    const T s_r = rowok ? sv0 : T(1);
    const T rs_r = T(1) / s_r;
    if (tid < BB) {
      const T v = buf_load<T>(make_rsrc(a.s + r0, (int64_t)mr * es), (uint32_t)tid);
      sm.sc[tid] = tid < mr ? v : T(1);
    }

    const int nphase = a.Nj + nw - 1;
    int vblk = -1;  // last 64-wide block whose contribution counters wave 0 checked
    TileLoads<T> ld;
    bool pre = prefetch_tile<T>(a, K, w, -1, ld);  // ld: this phase's micro-tile loads
    for (int p = 0; p < nphase; ++p) {
      const int cdone = p - (nw - 1);  // micro-column completed by this phase
      const bool closes = cdone >= 0 && ((cdone & 3) == 3 || cdone == a.Nj - 1);
      // The trailing wave (it completes the block) reserves the block's queue slots at
      // the start of the phase, lane c for queue c; the returned bases are first needed
      // after the phase, so the atomics' latency overlaps the phase's work.
      const bool pub = w == nw - 1;
      int base = 0;
      if (pub && closes && lane < NCLS) {
        const int cnt = block_task_count(K, cdone / GOUT, a.Mb, a.Nb, lane);
        if (cnt > 0) base = atomicAdd(a.ctl + kTail + kLine * lane, cnt);
      }
      const int j = p - w;
      // (after an abort every wait inside returns at once, so the band drains quickly)
      if (w < nw && j >= 0 && j < a.Nj)
        round_micro_tile<T>(a, sm, K, w, j, vblk, pre, ld, aVn, aVi, cu, cup, cup2, s_r, rs_r);
      drain();
      // Micro-column cdone is complete once the trailing wave's stores have drained (the
      // other waves' tiles of it were drained before earlier barriers): the next band is
      // told at once, not after this phase's barrier, which waits for this band's other
      // waves.
      if (pub && cdone >= 0 && lane == 0) st_dev(a.rdone + K, cdone + 1);
      // the next micro-tile's loads, in flight across the barrier
      pre = prefetch_tile<T>(a, K, w, p, ld);
      __syncthreads();
      if (pub && closes) publish_block(a, K, cdone / GOUT, base, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM worker
// ---------------------------------------------------------------------------
// The band-update tile: C (kBM x 64) += A^T B with both operands k-major, staged through
// LDS in chunks of kKC k-rows.  Up to three chunks of loads are kept in flight in
// registers (12 eight-byte loads per thread per chunk, so together with the 32 old C
// values no wave ever has more than 63 loads outstanding, the hardware counter's limit);
// two LDS stages let the next chunk be written while the current one is multiplied.
constexpr int kKC = 16;           // k-rows per chunk
constexpr int kAheadMax = 3;      // chunks whose loads are in flight (long tasks)
constexpr int kBM = kPanel * BB;  // output rows (target side) of a task
constexpr int kSA = kBM + 16;     // LDS pitch of the staged A chunk (k-major)
constexpr int kSB = BB + 16;      // LDS pitch of the staged B chunk
constexpr int kPT = kBM + 2;      // LDS pitch of the transposed epilogue
constexpr int kStageElems = kKC * (kSA + kSB);
template <typename T>
struct GemmSmem {
  static constexpr int kElems = 2 * kStageElems > BB * kPT ? 2 * kStageElems : BB * kPT;
  T buf[kElems];
  unsigned long long desc;
  int bcast[4];
};

// G[x][y] = sum_{k<K} A[k*lda + x] B[k*ldb + y] for x < M <= kBM, y < N <= 64, K <= kKC NCH,
// both operands k-major; C[x*ldc + y] (or, with `trans`, C[y*ldc + x]) becomes G, or C + G.
// Rows x of target block x / 64 take the plain store when bit x / 64 of `first` is set
// (the target's first contribution), else read-add-write; the old C values are loaded
// while the last chunks are multiplied.  Four waves; wave w owns rows [32 w, 32 w + 32) as
// 2 x 4 MFMA tiles.  k-rows past K read as zero (exact buffer ranges); rows or columns
// past M, N read neighbouring finite data that only reaches outputs that are never
// stored.  B and C are produced by other workgroups of the same launch, so they are
// accessed at device scope.  The chunk loop is unrolled (NCH is a compile-time count), so
// every wait for a chunk's loads is exact.
template <typename T, int NCH>
__device__ inline void panel_gemm(const T* A, int64_t lda, const T* B, int64_t ldb, T* C,
                                  int64_t ldc, int M, int N, int K, bool trans, int first,
                                  GemmSmem<T>& sm) {
  typedef typename Mfma<T>::acc_t acc_t;
  constexpr int TH = kThreads;
  constexpr int NA = kKC * kBM / TH, NB = kKC * BB / TH;  // staged elements per thread
  constexpr int TM = 2, TN = 4;
  constexpr int NOLD = TM * TN * 4;
  static_assert(NA + NB == 12 && BB * kBM / TH == NOLD, "tile shape");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wi0 = 32 * w;
  const int kq = lane >> 4, cl = lane & 15;
  const int64_t es = sizeof(T);
  const rsrc_t ra = make_rsrc(A, ((int64_t)(K - 1) * lda + M) * es);
  const rsrc_t rb = make_rsrc(B, ((int64_t)(K - 1) * ldb + N) * es);
  const rsrc_t rc = trans ? make_rsrc(C, ((int64_t)(N - 1) * ldc + M) * es)
                          : make_rsrc(C, ((int64_t)(M - 1) * ldc + N) * es);
  const uint32_t va = (uint32_t)((tid / kBM) * lda + tid % kBM);
  const uint32_t vb = (uint32_t)((tid / BB) * ldb + tid % BB);
  // short tasks load the old C values first (their latency then spans the whole task)
  // and keep two chunks in flight; long tasks keep three and load C near the end
  constexpr int kAhead = NCH > 4 ? kAheadMax : 2;
  constexpr int kOld = NCH > 4 ? NCH - 1 - kAhead : -1;
  T pa[kAhead][NA], pb[kAhead][NB];
  auto fetch = [&](int c, int r) {
#pragma unroll
    for (int u = 0; u < NA; ++u)
      pa[r][u] = buf_load_s<T>(ra, va, (uint32_t)((c * kKC + u * (TH / kBM)) * lda));
#pragma unroll
    for (int u = 0; u < NB; ++u)
      pb[r][u] = buf_load_s_dev<T>(rb, vb, (uint32_t)((c * kKC + u * (TH / BB)) * ldb));
  };
  auto stage = [&](int r, int st) {
    T* as0 = sm.buf + st * kStageElems + (tid / kBM) * kSA + tid % kBM;
    T* bs0 = sm.buf + st * kStageElems + kSA * kKC + (tid / BB) * kSB + tid % BB;
#pragma unroll
    for (int u = 0; u < NA; ++u) as0[u * (TH / kBM) * kSA] = pa[r][u];
#pragma unroll
    for (int u = 0; u < NB; ++u) bs0[u * (TH / BB) * kSB] = pb[r][u];
  };
  // old C values in the layout of the epilogue that adds to them
  T old[NOLD];
  auto load_old = [&]() {
    if (!trans) {
#pragma unroll
      for (int x = 0; x < TM; ++x) {
        const bool plain = (first >> ((wi0 + 16 * x) / BB)) & 1;
#pragma unroll
        for (int y = 0; y < TN; ++y)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = wi0 + 16 * x + Mfma<T>::row(lane, e), j = 16 * y + cl;
            old[(x * TN + y) * 4 + e] =
                plain ? T(0) : buf_load_dev<T>(rc, (uint32_t)((int64_t)i * ldc + j));
          }
      }
    } else {
#pragma unroll
      for (int u = 0; u < NOLD; ++u) {
        const int idx = tid + TH * u, yj = idx / kBM, xi = idx % kBM;
        const bool plain = (first >> (xi / BB)) & 1;
        old[u] = plain ? T(0) : buf_load_dev<T>(rc, (uint32_t)((int64_t)yj * ldc + xi));
      }
    }
  };
  acc_t acc[TM][TN];
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y) acc[x][y] = acc_t{0, 0, 0, 0};
  // fp32: the fragments of k-step ks + 1 are read from LDS before the products of k-step ks
  // are issued (two register sets, held in that order by a scheduling barrier), so that the
  // reads' latency passes during the products, which take half as long as in fp64.  (In
  // fp64 the compiler's own order was faster: 22 against 24 us per 256-deep task.)
  auto multiply = [&](int st) {
    const T* as = sm.buf + st * kStageElems;
    const T* bs = as + kSA * kKC;
    T fa[2][TM], fb[2][TN];
    auto frag = [&](int ks, int b) {
#pragma unroll
      for (int x = 0; x < TM; ++x) fa[b][x] = as[(4 * ks + kq) * kSA + wi0 + 16 * x + cl];
#pragma unroll
      for (int y = 0; y < TN; ++y) fb[b][y] = bs[(4 * ks + kq) * kSB + 16 * y + cl];
    };
    frag(0, 0);
#pragma unroll
    for (int ks = 0; ks < kKC / 4; ++ks) {
      const int b = sizeof(T) == 4 ? ks & 1 : 0;
      if (sizeof(T) == 4) {
        if (ks + 1 < kKC / 4) frag(ks + 1, b ^ 1);
        __builtin_amdgcn_sched_barrier(0);
      } else if (ks > 0) {
        frag(ks, 0);
      }
#pragma unroll
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y) acc[x][y] = Mfma<T>::run(fa[b][x], fb[b][y], acc[x][y]);
    }
  };
  if (kOld < 0) load_old();
#pragma unroll
  for (int c = 0; c < kAhead && c < NCH; ++c) fetch(c, c);
  stage(0, 0);
  if (kAhead < NCH) fetch(kAhead, 0);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c + 1 < NCH) {
      stage((c + 1) % kAhead, (c + 1) & 1);
      if (c + 1 + kAhead < NCH) fetch(c + 1 + kAhead, (c + 1) % kAhead);
    }
    if (c == kOld) load_old();
    multiply(c & 1);
    __syncthreads();
  }
  if (!trans) {
#pragma unroll
    for (int x = 0; x < TM; ++x)
#pragma unroll
      for (int y = 0; y < TN; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = wi0 + 16 * x + Mfma<T>::row(lane, e), j = 16 * y + cl;
          if (i < M && j < N)
            buf_store_dev<T>(old[(x * TN + y) * 4 + e] + acc[x][y][e], rc,
                             (uint32_t)((int64_t)i * ldc + j));
        }
    return;
  }
  // transposed: the owners write G^T into LDS, then every thread updates whole C rows
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int xi = wi0 + 16 * x + Mfma<T>::row(lane, e), yj = 16 * y + cl;
        sm.buf[yj * kPT + xi] = acc[x][y][e];
      }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NOLD; ++u) {
    const int idx = tid + TH * u, yj = idx / kBM, xi = idx % kBM;
    if (xi < M && yj < N)
      buf_store_dev<T>(old[u] + sm.buf[yj * kPT + xi], rc, (uint32_t)((int64_t)yj * ldc + xi));
  }
  __syncthreads();
}

template <typename T>
// (inlined into the kernel: as a call it would take the kernel arguments through memory)
__device__ __attribute__((always_inline)) inline void gemm_worker(const SweepArgs<T>& a,
                                                                  GemmSmem<T>& sm, int cls) {
  const int64_t m = a.m, n = a.n;
  const int tid = threadIdx.x;
  for (;;) {
    __syncthreads();
    if (tid < 64) {
      // claim the next task and wait for its descriptor (whole first wave)
      int slot = 0;
      if (tid == 0) slot = aborted(a.ctl) ? a.qcap[cls] : atomicAdd(a.ctl + kHead + kLine * cls, 1);
      slot = __builtin_amdgcn_readfirstlane(slot);
      unsigned long long d = 0;
      if (slot < a.qcap[cls]) {
        for (int it = 0;; ++it) {
          d = __hip_atomic_load(a.qd[cls] + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          d = ((unsigned long long)__builtin_amdgcn_readfirstlane((int)(d >> 32)) << 32) |
              (unsigned)__builtin_amdgcn_readfirstlane((int)d);
          if (d >> 63) break;
          if ((it & 15) == 15) {
            if (aborted(a.ctl)) break;
            if (it > kSpinLimit) {
              if (tid == 0) abort_sweep(a.ctl, a.info);
              break;
            }
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      const bool go = (d >> 63) != 0;
      int first = 0;
      if (go) {
        // wait until the earlier contributions to every target tile are applied
        const bool far = (d >> 62) & 1;
        const int dir = (d >> 61) & 1;
        const int own = (d >> 45) & 0x7FFF, other = (d >> 30) & 0x7FFF;
        const int t1 = (d >> 15) & 0x7FFF, t0 = d & 0x7FFF;
        bool ok = true;
        for (int t = t0; t <= t1 && ok; ++t) {
          const int seq = push_seq(t, own, cls);
          int* cnt = dir == 0 ? a.vcnt[cls] + (int64_t)t * a.Nb + other
                              : a.hcnt[cls] + (int64_t)other * a.Nb + t;
          ok = wait_ge(cnt, seq, a.ctl, a.info);
          if (seq == 0) first |= 1 << (t - t0);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if (!ok) d = 0;
      }
      if (tid == 0) {
        sm.desc = go ? d : 0;
        sm.bcast[0] = slot;
        sm.bcast[1] = first;
      }
    }
    __syncthreads();
    const unsigned long long d = sm.desc;
    if (sm.bcast[0] >= a.qcap[cls]) return;
    if (!(d >> 63)) {
      if (aborted(a.ctl)) return;
      continue;
    }
    const bool far = (d >> 62) & 1;
    const int dir = (d >> 61) & 1;
    const int own = (d >> 45) & 0x7FFF, other = (d >> 30) & 0x7FFF;
    const int t1 = (d >> 15) & 0x7FFF, t0 = d & 0x7FFF;
    const int first = sm.bcast[1];
    const int64_t ext = dir == 0 ? m : n;  // extent along the push
    const int64_t src0 = far ? (int64_t)(own - (GOUT - 1)) * BB : (int64_t)own * BB;
    const int ks = far ? GOUT * BB : ((ext - src0) < BB ? (int)(ext - src0) : BB);
    const int64_t p0 = (int64_t)t0 * BB;
    const int64_t pend = (int64_t)(t1 + 1) * BB < ext ? (int64_t)(t1 + 1) * BB : ext;
    const int PW = (int)(pend - p0);
    // vertical: V[p0 + x][q0 + y] += sum_k U'a[src0 + k][p0 + x] R[src0 + k][q0 + y];
    // horizontal: H[q0 + y][p0 + x] += sum_k U'b[src0 + k][p0 + x] Delta^T[src0 + k][q0 + y]
    const int64_t q0 = (int64_t)other * BB;
    const int64_t qext = dir == 0 ? n : m;
    const int QW = (qext - q0) < BB ? (int)(qext - q0) : BB;
    const T* pa = dir == 0 ? a.Ua : a.Ub;
    const T* pb = dir == 0 ? a.R : a.DT;
    const int64_t ldb = dir == 0 ? n : m;
    T* pc = dir == 0 ? a.Vacc[cls] + p0 * n + q0 : a.Hacc[cls] + q0 * n + p0;
    const long long t_begin = wall_clock64();
    if (far)
      panel_gemm<T, GOUT * BB / kKC>(pa + src0 * ext + p0, ext, pb + src0 * ldb + q0, ldb, pc, n,
                                     PW, QW, ks, dir != 0, first, sm);
    else
      panel_gemm<T, BB / kKC>(pa + src0 * ext + p0, ext, pb + src0 * ldb + q0, ldb, pc, n, PW,
                              QW, ks, dir != 0, first, sm);
    drain();
    __syncthreads();
    if (tid == 0) {
      for (int t = t0; t <= t1; ++t) {
        int* cnt = dir == 0 ? a.vcnt[cls] + (int64_t)t * a.Nb + other
                            : a.hcnt[cls] + (int64_t)other * a.Nb + t;
        st_dev(cnt, push_seq(t, own, cls) + 1);
      }
      if (a.stats) {
        unsigned long long* st = a.stats + 3 * cls;
        atomicAdd(st + 0, (unsigned long long)(wall_clock64() - t_begin));
        atomicAdd(st + 1, (unsigned long long)(2 * (int64_t)PW * QW * ks));
        atomicAdd(st + 2, 1ull);
      }
    }
  }
}

template <typename T>
struct SweepSmem {
  static constexpr size_t kBand = sizeof(BandSmem<T>), kGemm = sizeof(GemmSmem<T>);
  static constexpr size_t kBytes = kBand > kGemm ? kBand : kGemm;
};

// The persistent sweep.  Workgroups draw a ticket on their XCD when they start: tickets
// 0, 1, 2 of every XCD take far, near and next band-update tasks (so every queue makes
// progress however many workgroups are resident), tickets 3 .. nbxcd + 2 own bands of
// their XCD and take far tasks once no band is left, and of the rest one in seven takes
// near tasks, one in twenty next tasks and the others far ones.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_sweep(SweepArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char smem[SweepSmem<T>::kBytes];
  __shared__ int ticket;
  if (threadIdx.x == 0) ticket = atomicAdd(a.ctl + kXTicket + kLine * xcd_id(a.nxcd), 1);
  __syncthreads();
  const int tk = ticket;
  if (tk >= 3 && tk < 3 + a.nbxcd) band_worker<T>(a, *reinterpret_cast<BandSmem<T>*>(smem));
  const int r = tk - 3 - a.nbxcd;
  const int cls = tk < 3 ? (tk == 0 ? kFar : tk == 1 ? kNear : kNext)
                  : r < 0 ? kFar
                  : r % a.near_mod == 0 ? kNear
                  : r % 20 == 5 ? kNext : kFar;
  gemm_worker<T>(a, *reinterpret_cast<GemmSmem<T>*>(smem), cls);
}

// control words, progress counters and task descriptors start at zero
__global__ __launch_bounds__(256) void k_init_sync(int* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

// When n is not a multiple of the micro-tile width, the lanes of a row's last micro-tile
// whose columns lie past n read, inside the tile's buffer range, the first columns of the
// next row.  Their values only reach outputs that are never stored, except through a
// product with a zero coefficient (the in-tile horizontal feedback multiplies every column
// of the micro-tile), where a NaN would survive.  The horizontal accumulators' first
// columns belong to column block 0, to which no contribution is ever pushed, so they would
// hold whatever the workspace held: they are cleared here, before the sweep.
template <typename T>
__global__ __launch_bounds__(256) void k_clear_lead(T* h0, T* h1, T* h2, int64_t m, int64_t n,
                                                    int cols) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m * cols) return;
  const int64_t o = (i / cols) * n + i % cols;
  h0[o] = T(0);
  h1[o] = T(0);
  h2[o] = T(0);
}

template <typename T>
__global__ __launch_bounds__(256) void k_check_scales(int64_t m, const T* __restrict__ s,
                                                      int* info) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  const T v = s[i];
  if (!(v > T(0)) || !isfinite(v)) record_info(info, 3, (int)(i + 1));
}

struct SyncLayout {
  int64_t ctl, rdone, cnt, qd[NCLS], words;  // offsets in ints; qd 8-byte aligned
  int qcap[NCLS];
};
SyncLayout sync_layout(int64_t m, int64_t n) {
  const int Mb = (int)cdiv(m, BB), Nb = (int)cdiv(n, BB);
  int64_t cap[NCLS] = {0, 0, 0};
  for (int K = 0; K < Mb; ++K)
    for (int L = 0; L < Nb; ++L)
      for (int c = 0; c < NCLS; ++c) cap[c] += block_task_count(K, L, Mb, Nb, c);
  SyncLayout s;
  s.ctl = 0;
  s.rdone = kCtlWords;
  s.cnt = s.rdone + Mb;  // vcnt of each class, then hcnt of each class
  int64_t q = (s.cnt + 2 * NCLS * (int64_t)Mb * Nb + 1) / 2 * 2;
  for (int c = 0; c < NCLS; ++c) {
    s.qd[c] = q;
    q += 2 * cap[c];
    s.qcap[c] = (int)cap[c];
  }
  s.words = q;
  return s;
}

// How many band workers each XCD gets (b) and how many consecutive bands go to one XCD
// (gs).  The sweep takes about max(pipeline, updates): the band pipeline's phases, from a
// simulation of the dealing (band K starts four phases after band K - 1 and once a band
// worker of its XCD is free; a band takes Nj + 3 phases), times a phase's duration, against
// the band updates' flops over the rate of the CUs left to them.  Both rates were measured
// on the 4096-wide layer: a phase takes 12.9 us (fp64) or 9.3 us (fp32), a CU running
// update tasks sustains 0.175 (fp64) or 0.276 (fp32) TFLOP/s, 80 % of the time busy.  The
// default (b0, gs0) keeps every band of the pipeline active at once and is kept unless
// another plan is estimated at least 10 % faster.  GPTQ2D_SWEEP_BANDS="b,gs" overrides the
// plan (a tuning knob; values are clamped to what the grid allows).
// Of the update workgroups, one in seven takes near tasks when the pipeline bounds the
// sweep (their latency is then on the critical path: fewer near workers made the
// 4096-wide layer slower); when the updates bound it, one in fourteen, which leaves more
// CUs to the far tasks (the 8192-wide and 14336 x 4096 layers were 4-6 % faster).
// GPTQ2D_SWEEP_NEAR=k overrides (k >= 1).
struct BandPlan {
  int b, gs, near_mod;
};
double pipeline_phases(int Mb, int Nj, int nx, int b, int gs) {
  std::vector<double> free_at((size_t)nx * b, 0.0);
  double prev = -(double)GOUT, end = 0.0;
  for (int K = 0; K < Mb; ++K) {
    const int x = (K / gs) % nx;
    double* f = &free_at[(size_t)x * b];
    int w = 0;
    for (int i = 1; i < b; ++i)
      if (f[i] < f[w]) w = i;
    const double st = prev + GOUT > f[w] ? prev + GOUT : f[w];
    f[w] = st + Nj + 3;
    prev = st;
    if (f[w] > end) end = f[w];
  }
  return end;
}
BandPlan plan_bands(int64_t m, int64_t n, int Mb, int Nj, int nx, int grid, int b0, int gs0,
                    bool f64) {
  const int bmax = grid / nx - NCLS;
  BandPlan best{b0, gs0, 7};
  int near_env = 0;
  if (const char* env = getenv("GPTQ2D_SWEEP_NEAR")) {
    if (sscanf(env, "%d", &near_env) != 1 || near_env < 1) near_env = 0;
  }
  if (const char* env = getenv("GPTQ2D_SWEEP_BANDS")) {
    int b = 0, gs = 0;
    if (sscanf(env, "%d,%d", &b, &gs) == 2 && b >= 1 && gs >= 1) {
      best.b = b < bmax ? b : bmax;
      best.gs = gs;
      if (near_env) best.near_mod = near_env;
      return best;
    }
  }
  const double phase = f64 ? 12.9e-6 : 9.3e-6;
  const double rate = (f64 ? 0.175e12 : 0.276e12) * 0.8;
  const double flops = 0.96 * (double)m * (double)n * (double)(m + n);
  auto est = [&](int b, int gs) {
    const double tp = pipeline_phases(Mb, Nj, nx, b, gs) * phase;
    const double tg = flops / (rate * (double)(grid - nx * b));
    return tp > tg ? tp : tg;
  };
  auto update_bound = [&](int b, int gs) {
    return flops / (rate * (double)(grid - nx * b)) > pipeline_phases(Mb, Nj, nx, b, gs) * phase;
  };
  const double t0 = est(b0, gs0);
  double tb = t0;
  for (int gs = gs0; gs >= 1; gs /= 2)
    for (int b = b0; b >= 1; --b) {
      const double t = est(b, gs);
      if (t < tb) {
        tb = t;
        best = BandPlan{b, gs, 7};
      }
    }
  if (tb > 0.9 * t0) best = BandPlan{b0, gs0, 7};
  best.near_mod = near_env ? near_env : update_bound(best.b, best.gs) ? 14 : 7;
  return best;
}

// band-update task accounting of the measurement hook (see prof.hpp)
__device__ unsigned long long g_band_stats[3 * NCLS];

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
  a.Nj = (int)cdiv(n, MU);
  a.lo = -(1 << (bits - 1));
  a.hi = (1 << (bits - 1)) - 1;
  a.bits = bits;
  a.Ua = Ua;
  a.Ub = Ub;
  a.s = scales;
  a.W = W;
  for (int c = 0; c < NCLS; ++c) {
    a.Vacc[c] = take();
    a.Hacc[c] = take();
  }
  a.R = take();
  a.DT = take();
  const SyncLayout sl = sync_layout(m, n);
  int* sync = (int*)c;
  a.ctl = sync + sl.ctl;
  a.rdone = sync + sl.rdone;
  for (int c = 0; c < NCLS; ++c) {
    a.vcnt[c] = sync + sl.cnt + (int64_t)c * a.Mb * a.Nb;
    a.hcnt[c] = sync + sl.cnt + (int64_t)(NCLS + c) * a.Mb * a.Nb;
    a.qd[c] = (unsigned long long*)(sync + sl.qd[c]);
    a.qcap[c] = sl.qcap[c];
  }
  a.codes = codes;
  a.Q = Q;
  a.info = info;
  a.stats = band_stats_device();

  int dev = 0, ncu = 0, occ = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_sweep<T>, kThreads, 0)) !=
      hipSuccess)
    return e;
  if (occ < 1) return hipErrorInvalidConfiguration;
  const int grid = ncu * occ;
  // Bands are dealt to the XCDs, and every XCD needs band workers of its own: take the
  // device's XCD count (1 when the query is not supported), capped at the slots of the
  // control area.
  int nxcd = 1;
  if (hipDeviceGetAttribute(&nxcd, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || nxcd < 1) {
    (void)hipGetLastError();
    nxcd = 1;
  }
  a.nxcd = nxcd < kMaxXcd ? nxcd : kMaxXcd;
  // Band workers: enough for the bands that are active at once (a band runs Nj + 3
  // phases, the next one starts about four phases later), at most half the grid; groups
  // of up to eight consecutive bands per XCD, one spare band worker per XCD, and a
  // workgroup per XCD left for each task queue.  On layers whose band updates outweigh the
  // pipeline, fewer band workers leave more CUs to the updates (plan_bands).
  int nbw = (a.Nj + 3) / GOUT + 2;
  if (nbw > a.Mb) nbw = a.Mb;
  if (nbw > grid / 2) nbw = grid / 2;
  if (nbw < 1) nbw = 1;
  const int nx = a.nxcd;
  const int gs0 = (a.Mb + nx - 1) / nx < 8 ? (a.Mb + nx - 1) / nx : 8;
  int b0 = (nbw + nx - 1) / nx + 1;
  if (b0 > grid / nx - NCLS) b0 = grid / nx - NCLS;
  const BandPlan bp = plan_bands(m, n, a.Mb, a.Nj, nx, grid, b0, gs0, sizeof(T) == 8);
  a.gs = bp.gs;
  a.nbxcd = bp.b;
  a.near_mod = bp.near_mod;
  if (a.nbxcd < 1) return hipErrorInvalidConfiguration;

  const bool pr = prof_on();
  const double es = (double)sizeof(T);
  prof_begin(KC_OTHER, s);
  k_check_scales<T><<<(unsigned)cdiv(m, 256), 256, 0, s>>>(m, scales, info);
  const int64_t ig = cdiv(sl.words, 256) < 4096 ? cdiv(sl.words, 256) : 4096;
  k_init_sync<<<(unsigned)ig, 256, 0, s>>>(sync, sl.words);
  if (n % MU != 0) {
    static_assert(NCLS == 3, "one accumulator per class");
    const int cols = n < MU ? (int)n : MU;
    k_clear_lead<T><<<(unsigned)cdiv(m * cols, 256), 256, 0, s>>>(a.Hacc[0], a.Hacc[1],
                                                                   a.Hacc[2], m, n, cols);
  }
  prof_end(KC_OTHER, s, 0.0, 4.0 * (double)sl.words + es * (double)m);
  // algorithmic work of the sweep: every entry takes its k vertical and l horizontal
  // feedback terms (2 flops each); HBM bytes: W, the factors and scales in, codes and
  // Q out, and R, Delta written once and read back by the band products
  const double fl = pr ? (double)m * (double)n * (double)(m + n - 2) : 0.0;
  const double by = pr ? es * (3.0 * (double)mn + (double)m * m + (double)n * n + (double)m) +
                             (double)mn : 0.0;
  prof_begin(KC_SWEEP, s);
  k_sweep<T><<<grid, kThreads, 0, s>>>(a);
  prof_end(KC_SWEEP, s, fl, by);
  return hipGetLastError();
}

}  // namespace

unsigned long long* band_stats_device() {
  if (!prof_on()) return nullptr;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_band_stats)) != hipSuccess) return nullptr;
  return (unsigned long long*)p;
}

hipError_t band_stats_collect(double* cu_ms, double* flops, int64_t* tasks) {
  unsigned long long h[3 * NCLS] = {};
  hipError_t e = hipMemcpyFromSymbol(h, HIP_SYMBOL(g_band_stats), sizeof(h), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  const unsigned long long z[3 * NCLS] = {};
  e = hipMemcpyToSymbol(HIP_SYMBOL(g_band_stats), z, sizeof(z), 0, hipMemcpyHostToDevice);
  for (int c = 0; c < NCLS; ++c) {
    cu_ms[c] = (double)h[3 * c] * 1e-5;  // 100 MHz ticks -> ms
    flops[c] = (double)h[3 * c + 1];
    tasks[c] = (int64_t)h[3 * c + 2];
  }
  return e;
}

size_t sweep_workspace(int64_t m, int64_t n, int dtype) {
  const size_t es = dtype == 0 ? sizeof(float) : sizeof(double);
  const SyncLayout sl = sync_layout(m, n);
  return (2 * NCLS + 2) * align_up((size_t)m * n * es) +
         align_up((size_t)sl.words * sizeof(int));
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
