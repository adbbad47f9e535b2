// Task-order rules of the two persistent kernels: which task a queue slot holds, which
// counters a task waits for, and which counter it sets when done.  The kernels
// (factor.hip, sweep.hip) and the host-side schedule checker of the test suite include
// this one header, so the checker exercises exactly the rules the GPU follows.  Plain C++
// (integer arithmetic only); compiled as host+device code by hipcc and as host code by a
// C++ compiler.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define G2D_HD __host__ __device__
#else
#define G2D_HD
#endif

namespace g2d {
namespace sched {

// ---------------------------------------------------------------------------
// Factor stage: the persistent Cholesky + row inverse (k_chol_persistent)
// ---------------------------------------------------------------------------
// Tiles are 64 x 64; n = tiles per edge.  The tasks of one matrix (groups go by step, the
// matrices alternating; chol_segments gives the order inside a group):
//   bulk (kind 0): tile (i, j) in step s, s + 1 <= j <= i, takes the panels
//                  bulk_lo(j, s) .. s - 1 in one task, in the steps bulk_at names;
//   crit (kind 1): the panel step of row tile i of block column s;
//   xrow (kind 2): chunk jj of tile (i, s) of X = L^-1, i = g + kInvStride jj, in order of
//                  jj and s.  Chunk 0, the last one added, covers k in [i - kInvFirst, i) and
//                  multiplies by -X_ii; chunk jj >= 1 covers kInvDepth tiles below
//                  khi = i - kInvFirst - kInvDepth (jj - 1), all clipped at s.
constexpr int kInvDepth = 16;  // tiles of k per chunk of the row inverse
constexpr int kInvFirst = 8;   // tiles of k of a row's last chunk
constexpr int kInvStride = 2;  // steps between the chunks of one row (<= kInvFirst + 1)
constexpr int kFinal = 1 << 24;  // tile counter of a final tile
// The trailing update of a tile column is deferred and applied kBulkDepth panels at a time
// (one task reads the tile once and multiplies kBulkDepth panel pairs), except in the
// kBulkNear - 1 steps before the column's own panel step, where it takes one panel per
// step (the last of them is the look-ahead, which feeds the panel chain).  The deep tasks
// of column j sit in the steps j - kBulkNear - q kBulkDepth (q >= 0), so that the last
// one ends kBulkNear - 1 steps before the panel step needs the tile, and the deep tasks of
// different columns fall in different steps: every step carries about the same work.
constexpr int kBulkDepth = 16;
constexpr int kBulkNear = 3;

// Whether tile column j takes a trailing-update task in step g (the panels 0 .. j - 2 in
// all; the panel step of column j applies panel j - 1 itself).
G2D_HD inline bool bulk_at(int j, int g) {
  if (g < 1 || g > j - 1) return false;
  return g > j - kBulkNear || (j - kBulkNear - g) % kBulkDepth == 0;
}
// First panel of column j's task in step g (bulk_at(j, g)): the task takes the panels
// bulk_lo .. g - 1, the ones after its previous task's (0 for the column's first task).
G2D_HD inline int bulk_lo(int j, int g) {
  const int prev = g > j - kBulkNear ? g - 1 : g - kBulkDepth;
  return prev >= 1 ? prev : 0;
}
// Group g lists, in this order: the look-ahead of step g (column g + 1, one panel), the
// panel steps of column g, the one-panel tasks of columns g + 2 .. g + kBulkNear - 1, the
// deep tasks of columns g + kBulkNear + q kBulkDepth, then the inverse chunks.  Sizes of the
// first four segments:
G2D_HD inline void chol_segments(int n, int g, int64_t* seg) {
  auto tiles = [&](int j) { return (int64_t)(j <= n - 1 ? n - j : 0); };  // tiles of column j
  seg[0] = g >= 1 ? tiles(g + 1) : 0;
  seg[1] = n - g;
  seg[2] = 0;
  seg[3] = 0;
  if (g == 0) return;
  for (int j = g + 2; j < g + kBulkNear; ++j) seg[2] += tiles(j);
  for (int j = g + kBulkNear; j <= n - 1; j += kBulkDepth) seg[3] += tiles(j);
}

// Tasks of the Cholesky in group g (the four segments).
G2D_HD inline int64_t chol_group_size(int n, int g) {
  int64_t seg[4];
  chol_segments(n, g, seg);
  return seg[0] + seg[1] + seg[2] + seg[3];
}
// xrow tasks of chunk jj in group g (row i = g + kInvStride jj): chunk 0 of every s < g;
// for jj >= 1 the columns s < khi = g - (kInvDepth - kInvStride) jj + kInvDepth - kInvFirst
// (a count that falls with jj).
G2D_HD inline int xrow_count(int n, int g, int jj) {
  if (g + kInvStride * jj >= n) return 0;
  if (jj == 0) return g;
  const int cnt = g - (kInvDepth - kInvStride) * jj + kInvDepth - kInvFirst;
  return cnt > 0 ? cnt : 0;
}
G2D_HD inline int64_t group_size(int n, int g) {
  int64_t c = chol_group_size(n, g) + xrow_count(n, g, 0);
  for (int jj = 1; xrow_count(n, g, jj) > 0; ++jj) c += xrow_count(n, g, jj);
  return c;
}
// chunks of the row inverse of tile (i, s), i > s
G2D_HD inline int xrow_chunks(int i, int s) {
  return 1 + (i - s > kInvFirst ? (i - s - kInvFirst + kInvDepth - 1) / kInvDepth : 0);
}

// One task: kind 0 bulk of tile (i, j) by the panels bulk_lo(j, s) .. s - 1; kind 1 the
// panel step of row tile i of block column s; kind 2 chunk j of tile (i, s) of X.
struct CholTask {
  int kind, i, s, j;
};
// Task r (0-based) of group g of a matrix with n tiles per edge (r < group_size(n, g)).
G2D_HD inline CholTask chol_decode(int n, int g, int64_t r) {
  CholTask t{-1, 0, 0, 0};
  int k = (int)r;
  int64_t seg[4];
  chol_segments(n, g, seg);
  const int64_t cg = seg[0] + seg[1] + seg[2] + seg[3];
  if (k < seg[0]) {
    t = CholTask{0, g + 1 + k, g, g + 1};
  } else if ((k -= (int)seg[0]) < seg[1]) {
    t = CholTask{1, g + k, g, 0};
  } else if ((k -= (int)seg[1]) < seg[2]) {
    int j = g + 2;
    while (k >= n - j) {
      k -= n - j;
      ++j;
    }
    t = CholTask{0, j + k, g, j};
  } else if ((k -= (int)seg[2]) < seg[3]) {
    int j = g + kBulkNear;
    while (k >= n - j) {
      k -= n - j;
      j += kBulkDepth;
    }
    t = CholTask{0, j + k, g, j};
  } else {
    k = (int)(r - cg);
    int jj = 0;
    if (k >= xrow_count(n, g, 0)) {
      k -= xrow_count(n, g, 0);
      jj = 1;
      while (jj < n && k >= xrow_count(n, g, jj)) {  // (k < the group's xrow tasks)
        k -= xrow_count(n, g, jj);
        ++jj;
      }
    }
    t = CholTask{2, g + kInvStride * jj, k, jj};
  }
  return t;
}
// Range [klo, khi) of k covered by chunk t.j of tile (t.i, t.s) (kind 2).
G2D_HD inline void xrow_range(const CholTask& t, int* klo, int* khi) {
  const int hi = t.j == 0 ? t.i : t.i - kInvFirst - kInvDepth * (t.j - 1);
  const int lo = hi - (t.j == 0 ? kInvFirst : kInvDepth);
  *khi = hi;
  *klo = lo > t.s ? lo : t.s;
}

// A counter condition: counter `idx` of array `arr` (0: tile counters of L, 1: chunk
// counters of X; both n x n, row-major by tile) must reach at least `val`.
struct CholWait {
  int arr;
  int64_t idx;
  int val;
};
// Condition q (0-based) of the conditions task t waits for before it starts, in this order;
// false when t has fewer than q + 1.  Each names exactly the tiles the task reads:
//   kind 2: L_i,khi-1 final (so every L_ik, k < khi), X_khi-1,s final (so every X_ks,
//           s <= k < khi), the tile's previous chunks, and X_ii for the last chunk;
//   kinds 0, 1: the panel tiles read are final (for kind 0 the last one, panel s - 1: a
//           row's panel tiles become final in order), and the task's own tiles carry the
//           panels before its first one (kind 0: bulk_lo(j, s); kind 1: s - 1).
// (One condition per call and no array, so that a kernel unrolling q over 0..3 keeps them
// in registers.)
G2D_HD inline bool chol_wait_at(int n, const CholTask& t, int q, CholWait* w) {
  const int64_t N = n;
  int k = 0;  // conditions listed so far
  bool found = false;
  auto put = [&](bool present, int arr, int64_t idx, int val) {
    if (!present) return;
    if (k == q) {
      *w = CholWait{arr, idx, val};
      found = true;
    }
    ++k;
  };
  if (t.kind == 2) {
    int klo, khi;
    xrow_range(t, &klo, &khi);
    const int nch = xrow_chunks(t.i, t.s);
    put(true, 0, (int64_t)t.i * N + (khi - 1), kFinal);
    if (khi - 1 == t.s)
      put(true, 0, (int64_t)t.s * N + t.s, kFinal);
    else
      put(true, 1, (int64_t)(khi - 1) * N + t.s, kFinal);
    put(t.j < nch - 1, 1, (int64_t)t.i * N + t.s, nch - 1 - t.j);
    put(t.j == 0, 0, (int64_t)t.i * N + t.i, kFinal);
  } else {
    const int r2 = t.kind == 0 ? t.j : t.s;  // the second panel row read
    put(t.s >= 1, 0, (int64_t)t.i * N + (t.s - 1), kFinal);
    put(t.s >= 1 && r2 != t.i, 0, (int64_t)r2 * N + (t.s - 1), kFinal);
    put(t.kind == 0 && bulk_lo(t.j, t.s) > 0, 0, (int64_t)t.i * N + t.j, bulk_lo(t.j, t.s));
    put(t.kind == 1 && t.s >= 2, 0, (int64_t)t.s * N + t.s, t.s - 1);
    put(t.kind == 1 && t.s >= 2 && t.i != t.s, 0, (int64_t)t.i * N + t.s, t.s - 1);
  }
  return found;
}
// All conditions of task t (at most 4) into w; returns their count.
G2D_HD inline int chol_waits(int n, const CholTask& t, CholWait* w) {
  int c = 0;
  for (int q = 0; q < 4; ++q)
    if (chol_wait_at(n, t, q, &w[c])) ++c;
  return c;
}
// The counter a finished task sets (a store, never an add): bulk tasks count the panels
// applied to their tile, a panel step marks its tile of L final, chunk jj of a tile of X
// counts the chunks added (kFinal for the last one).
G2D_HD inline CholWait chol_signal(int n, const CholTask& t) {
  const int64_t N = n;
  if (t.kind == 2)
    return CholWait{1, (int64_t)t.i * N + t.s, t.j == 0 ? kFinal : xrow_chunks(t.i, t.s) - t.j};
  if (t.kind == 0) return CholWait{0, (int64_t)t.i * N + t.j, t.s};
  return CholWait{0, (int64_t)t.i * N + t.s, kFinal};
}

// ---------------------------------------------------------------------------
// Sweep: band-update contributions (k_sweep)
// ---------------------------------------------------------------------------
constexpr int GOUT = 4;     // bands (blocks) per outer band (block)
// far pushes of outer band (block) O reach targets >= GOUT (O + 1) + FAR_OFF; with an
// offset of 2 a 256-deep task has a few phases to finish before its target needs it
constexpr int FAR_OFF = 2;
constexpr int kPanel = 2;   // target blocks per GEMM task
// Band-update contributions come in three classes, each with its own accumulators,
// contribution counters, task queue and workers:
//   near: 64 deep, from the last few bands / blocks before the target;
//   next: 256 deep, from the last outer band / block to the first kPanel targets it
//         reaches (the far contribution that is needed soonest after it is published);
//   far:  256 deep, every other contribution of whole outer bands / blocks.
// A contribution only ever waits for earlier contributions of its own class, so each
// queue is served in FIFO order, and urgent tasks never wait behind the backlog of far
// ones.
enum PushClass : int { kNear = 0, kNext = 1, kFar = 2, NCLS = 3 };

// Source index `own` (a band for vertical pushes, a column block for horizontal ones)
// pushes 64 deep to targets [own + 2, GOUT (own / GOUT) + GOUT - 1 + FAR_OFF]; the last
// band of an outer band pushes the whole outer band, 256 deep, to every target from
// GOUT (own / GOUT + 1) + FAR_OFF on (FAR_OFF >= 1).  Target T thus receives, in
// source order, the far pushes of outer bands 0 .. nfar(T) - 1 and then the near pushes
// of the bands GOUT nfar(T) .. T - 2; band T - 1 is applied by the band worker itself.
G2D_HD inline int nfar(int T) {
  return T >= GOUT + FAR_OFF ? (T - GOUT - FAR_OFF) / GOUT + 1 : 0;
}
// T is among the first kPanel targets of the far range of outer band nfar(T) - 1, whose
// push to T is then of class kNext
G2D_HD inline bool next_push(int T) {
  return T >= GOUT + FAR_OFF && (T - GOUT - FAR_OFF) % GOUT < kPanel;
}
// contributions of one class that target T receives, and a contribution's rank in them
G2D_HD inline int expected_class(int T, int cls) {
  const int nf = nfar(T), nx = next_push(T) ? 1 : 0;
  if (cls == kNear) return T >= 2 ? T - 1 - GOUT * nf : 0;
  return cls == kNext ? nx : nf - nx;
}
G2D_HD inline int push_seq(int T, int own, int cls) {
  if (cls == kNear) return own - GOUT * nfar(T);
  return cls == kNext ? 0 : own / GOUT;
}
G2D_HD inline void near_range(int own, int nt, int* t0, int* t1) {
  *t0 = own + 2;
  const int e = GOUT * (own / GOUT) + GOUT - 1 + FAR_OFF;
  *t1 = e < nt - 1 ? e : nt - 1;
}
G2D_HD inline void far_range(int own, int nt, int* t0, int* t1) {
  if (own % GOUT != GOUT - 1) {
    *t0 = 1;
    *t1 = 0;
    return;
  }
  *t0 = GOUT * (own / GOUT + 1) + FAR_OFF;
  *t1 = nt - 1;
}
G2D_HD inline int npanels(int t0, int t1) {
  return t1 >= t0 ? (t1 - t0) / kPanel + 1 : 0;
}
// The tasks a completed 64 x 64 block (K, L) publishes, in six groups g = 2 class + dir
// (dir 0: vertical, from band K to the bands below in column block L; dir 1: horizontal,
// from column block L to the blocks to its right in band K): group g covers targets
// g0[g] .. g1[g] in np[g] panels of kPanel targets.  Within a class the vertical panels
// take the class's first queue slots.
G2D_HD inline void block_groups(int K, int L, int Mb, int Nb, int* g0, int* g1, int* np) {
  for (int dir = 0; dir < 2; ++dir) {
    const int own = dir == 0 ? K : L, nt = dir == 0 ? Mb : Nb;
    int t0, t1;
    near_range(own, nt, &t0, &t1);
    g0[2 * kNear + dir] = t0;
    g1[2 * kNear + dir] = t1;
    np[2 * kNear + dir] = npanels(t0, t1);
    far_range(own, nt, &t0, &t1);
    const int nf = npanels(t0, t1);
    g0[2 * kNext + dir] = t0;
    g1[2 * kNext + dir] = t0 + kPanel - 1 < t1 ? t0 + kPanel - 1 : t1;
    np[2 * kNext + dir] = nf > 0 ? 1 : 0;
    g0[2 * kFar + dir] = t0 + kPanel;
    g1[2 * kFar + dir] = t1;
    np[2 * kFar + dir] = nf > 0 ? nf - 1 : 0;
  }
}
// Tasks of class cls that block (K, L) publishes.
G2D_HD inline int block_task_count(int K, int L, int Mb, int Nb, int cls) {
  int g0[6], g1[6], np[6];
  block_groups(K, L, Mb, Nb, g0, g1, np);
  return np[2 * cls] + np[2 * cls + 1];
}

}  // namespace sched
}  // namespace g2d
