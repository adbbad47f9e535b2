// Host-side check of the task order of the library's two persistent kernels, built from
// the same rule header the kernels use (two_sided_adaptive_amd/csrc/schedule.hpp).
//
//   factor P0 [P1]    the Cholesky + row inverse of one or two matrices with P0 (and P1)
//                     tiles per edge, in the kernel's queue order (steps in order, the
//                     matrices alternating inside a step).  Executes the queue in order and
//                     checks that every wait of every task is already met by the tasks
//                     before it, that counter stores never lower a counter, that each task
//                     appears once, and that every tile of L and X ends final.  A queue
//                     with that property drains with any number of resident workgroups:
//                     the earliest unfinished task always has its waits met.
//   qrun P0 [P1] W S  executes the factor's queue with W workgroups for S seeded random
//                     schedules and requires every schedule to drain (sim_factor).
//   run MB NB X B G WN WX WF S
//                     executes the sweep's rules on an MB x NB grid with X XCDs of B band
//                     workers (bands dealt in groups of G), WN / WX / WF near / next / far
//                     update workers, for S seeded random schedules, and requires every
//                     schedule to drain (sim_sweep).
//   sweep MB NB       the band-update contributions of an MB x NB grid of 64 x 64 blocks:
//                     per class, direction and target tile, the contributions that the
//                     blocks publish must carry the ranks 0 .. expected - 1 exactly once,
//                     in the order of their sources (so each class queue, served in FIFO
//                     order, never waits for a later task), and the band worker's wait
//                     targets (expected_class) must equal those counts.
// Prints one line per check and exits non-zero on the first violation.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <map>
#include <set>
#include <tuple>
#include <vector>

#include "schedule.hpp"

using namespace g2d::sched;

static int fail(const char* what) {
  fprintf(stderr, "VIOLATION: %s\n", what);
  return 1;
}

static int check_factor(const std::vector<int>& ns) {
  const int nmat = (int)ns.size();
  int maxn = 0;
  for (int n : ns) maxn = n > maxn ? n : maxn;
  std::vector<std::vector<int>> cnt[2];
  for (int q = 0; q < nmat; ++q) {
    cnt[q].assign(2, std::vector<int>((size_t)ns[q] * ns[q], 0));
  }
  std::set<std::tuple<int, int, int, int, int>> seen;
  int64_t tasks = 0;
  char msg[512];
  for (int g = 0; g < maxn; ++g) {
    for (int q = 0; q < nmat; ++q) {
      const int n = ns[q];
      if (g >= n) continue;
      const int64_t gsz = group_size(n, g);
      for (int64_t r = 0; r < gsz; ++r, ++tasks) {
        const CholTask t = chol_decode(n, g, r);
        if (t.kind < 0 || t.i < 0 || t.i >= n || t.s < 0 || t.s >= n) {
          snprintf(msg, sizeof msg, "factor n=%d step %d task %lld decodes out of range", n, g,
                   (long long)r);
          return fail(msg);
        }
        if (!seen.insert(std::make_tuple(q, t.kind, t.i, t.s, t.j)).second) {
          snprintf(msg, sizeof msg, "factor n=%d task (%d,%d,%d,%d) listed twice", n, t.kind,
                   t.i, t.s, t.j);
          return fail(msg);
        }
        CholWait w[4];
        const int nw = chol_waits(n, t, w);
        for (int c = 0; c < nw; ++c) {
          if (w[c].idx < 0 || w[c].idx >= (int64_t)n * n) return fail("wait index out of range");
          if (cnt[q][w[c].arr][w[c].idx] < w[c].val) {
            snprintf(msg, sizeof msg,
                     "factor matrix %d (n=%d) step %d: task kind %d (i=%d s=%d j=%d) waits for "
                     "counter %d[%lld] >= %d, which only a later task sets (now %d)",
                     q, n, g, t.kind, t.i, t.s, t.j, w[c].arr, (long long)w[c].idx, w[c].val,
                     cnt[q][w[c].arr][w[c].idx]);
            return fail(msg);
          }
        }
        // the trailing updates of a tile take the panels 0 .. s - 2 exactly once, in order:
        // a bulk task finds its tile carrying exactly the panels before its first one, and a
        // panel step finds its own tile carrying exactly the panels 0 .. s - 2
        {
          const int own = t.kind == 0 ? cnt[q][0][(size_t)t.i * n + t.j]
                                      : t.kind == 1 ? cnt[q][0][(size_t)t.i * n + t.s] : 0;
          const int want = t.kind == 0 ? bulk_lo(t.j, t.s) : t.kind == 1 ? (t.s >= 1 ? t.s - 1 : 0) : 0;
          if (t.kind != 2 && own != want) {
            snprintf(msg, sizeof msg,
                     "factor n=%d step %d: task kind %d (i=%d s=%d j=%d) finds its tile after "
                     "%d panels, expected %d", n, g, t.kind, t.i, t.s, t.j, own, want);
            return fail(msg);
          }
        }
        const CholWait sg = chol_signal(n, t);
        int& v = cnt[q][sg.arr][sg.idx];
        if (sg.val < v) {
          snprintf(msg, sizeof msg, "factor n=%d: task kind %d (i=%d s=%d j=%d) lowers a counter",
                   n, t.kind, t.i, t.s, t.j);
          return fail(msg);
        }
        v = sg.val;
      }
    }
  }
  for (int q = 0; q < nmat; ++q) {
    const int n = ns[q];
    for (int i = 0; i < n; ++i)
      for (int s = 0; s <= i; ++s) {
        if (cnt[q][0][(size_t)i * n + s] != kFinal) return fail("a tile of L never became final");
        if (s < i && cnt[q][1][(size_t)i * n + s] != kFinal)
          return fail("a tile of X never became final");
      }
  }
  printf("factor");
  for (int n : ns) printf(" %d", n);
  printf(": %lld tasks in queue order, every wait met by earlier tasks\n", (long long)tasks);
  return 0;
}

static int check_sweep(int Mb, int Nb) {
  // (class, dir, target band/block, other index) -> ranks seen, by source
  std::map<std::tuple<int, int, int, int>, std::vector<std::pair<int, int>>> got;
  int64_t total[NCLS] = {0, 0, 0};
  for (int K = 0; K < Mb; ++K)
    for (int L = 0; L < Nb; ++L) {
      int g0[6], g1[6], np[6];
      block_groups(K, L, Mb, Nb, g0, g1, np);
      for (int g = 0; g < 6; ++g) {
        const int cls = g >> 1, dir = g & 1;
        const int own = dir == 0 ? K : L, other = dir == 0 ? L : K;
        for (int k = 0; k < np[g]; ++k) {
          const int p0 = g0[g] + kPanel * k;
          const int p1 = p0 + kPanel - 1 < g1[g] ? p0 + kPanel - 1 : g1[g];
          for (int T = p0; T <= p1; ++T)
            got[std::make_tuple(cls, dir, T, other)].push_back({own, push_seq(T, own, cls)});
        }
        total[cls] += np[g];
      }
      for (int c = 0; c < NCLS; ++c)
        if (np[2 * c] + np[2 * c + 1] != block_task_count(K, L, Mb, Nb, c))
          return fail("block_task_count differs from the published groups");
    }
  char msg[512];
  for (int cls = 0; cls < NCLS; ++cls)
    for (int dir = 0; dir < 2; ++dir)
      for (int T = 0; T < (dir == 0 ? Mb : Nb); ++T)
        for (int o = 0; o < (dir == 0 ? Nb : Mb); ++o) {
          const auto it = got.find(std::make_tuple(cls, dir, T, o));
          const int exp = expected_class(T, cls);
          const int have = it == got.end() ? 0 : (int)it->second.size();
          if (have != exp) {
            snprintf(msg, sizeof msg,
                     "sweep %dx%d: class %d dir %d target %d (other %d) expects %d contributions, "
                     "%d are published", Mb, Nb, cls, dir, T, o, exp, have);
            return fail(msg);
          }
          for (int r = 0; r < have; ++r) {
            const auto& e = it->second[r];  // sources in publication order of one column
            if (e.second != r) {
              snprintf(msg, sizeof msg,
                       "sweep %dx%d: class %d dir %d target %d: source %d has rank %d, expected "
                       "%d (ranks must follow the sources' order)", Mb, Nb, cls, dir, T, e.first,
                       e.second, r);
              return fail(msg);
            }
            if (e.first >= T - 1) return fail("a contribution from the band above or later");
          }
        }
  printf("sweep %dx%d: near %lld, next %lld, far %lld tasks; ranks complete and in source order\n",
         Mb, Nb, (long long)total[0], (long long)total[1], (long long)total[2]);
  return 0;
}

// Executes the factor's queue with W workgroups: a free one claims the next task in queue
// order, a claimed task runs once every counter it waits for has its value, and each step is
// chosen at random among the enabled ones (seeded).  Fails if work remains and nothing can
// run.
static int sim_factor(const std::vector<int>& ns, int W, int seeds) {
  struct T {
    int q;
    CholTask t;
  };
  std::vector<T> order;
  int maxn = 0;
  for (int n : ns) maxn = n > maxn ? n : maxn;
  for (int g = 0; g < maxn; ++g)
    for (int q = 0; q < (int)ns.size(); ++q) {
      if (g >= ns[q]) continue;
      const int64_t gsz = group_size(ns[q], g);
      for (int64_t r = 0; r < gsz; ++r) order.push_back({q, chol_decode(ns[q], g, r)});
    }
  char msg[256];
  for (int seed = 1; seed <= seeds; ++seed) {
    uint64_t rng = 0x2545F4914F6CDD1Dull * (uint64_t)seed + 99;
    auto rnd = [&](uint64_t k) {
      rng = rng * 6364136223846793005ull + 1442695040888963407ull;
      return (uint64_t)((rng >> 33) % k);
    };
    std::vector<std::vector<int>> cnt[2];
    for (int q = 0; q < (int)ns.size(); ++q)
      cnt[q].assign(2, std::vector<int>((size_t)ns[q] * ns[q], 0));
    std::vector<int64_t> held(W, -1);
    size_t next = 0;
    int64_t done = 0;
    std::vector<std::pair<int, int>> acts;
    for (;;) {
      acts.clear();
      for (int k = 0; k < W; ++k) {
        if (held[k] < 0) {
          if (next < order.size()) acts.push_back({0, k});
          continue;
        }
        const T& e = order[held[k]];
        CholWait w[4];
        const int nw = chol_waits(ns[e.q], e.t, w);
        bool ok = true;
        for (int c = 0; c < nw && ok; ++c) ok = cnt[e.q][w[c].arr][w[c].idx] >= w[c].val;
        if (ok) acts.push_back({1, k});
      }
      if (acts.empty()) break;
      const auto a = acts[rnd(acts.size())];
      if (a.first == 0) {
        held[a.second] = (int64_t)next++;
      } else {
        const T& e = order[held[a.second]];
        const CholWait sg = chol_signal(ns[e.q], e.t);
        cnt[e.q][sg.arr][sg.idx] = sg.val;
        held[a.second] = -1;
        ++done;
      }
    }
    if (done != (int64_t)order.size()) {
      snprintf(msg, sizeof msg, "factor with %d workgroups, seed %d: stuck with %lld of %lld tasks done",
               W, seed, (long long)done, (long long)order.size());
      return fail(msg);
    }
  }
  printf("factor");
  for (int n : ns) printf(" %d", n);
  printf(" with %d workgroups: %d random schedules drained\n", W, seeds);
  return 0;
}

// Executes the sweep's dependency rules with a given number of band workers per XCD and of
// update workers per class, choosing among all enabled steps at random (seeded): a band
// completes its next 64 x 64 block once the band above has completed that block and the
// block's contribution counters of every class are complete, then publishes the block's
// tasks (class queues, first in first out); an update worker claims the next task of its
// class and applies it once every target counter equals the task's rank.  Fails if the run
// reaches a state where work remains and no step is enabled.
static int sim_sweep(int Mb, int Nb, int nx, int b, int gs, const int* W, int seeds) {
  struct Task {
    int dir, own, other, p0, p1;
  };
  char msg[512];
  for (int seed = 1; seed <= seeds; ++seed) {
    uint64_t rng = 0x9E3779B97F4A7C15ull * (uint64_t)seed + 12345;
    auto rnd = [&](uint64_t k) {
      rng = rng * 6364136223846793005ull + 1442695040888963407ull;
      return (uint64_t)((rng >> 33) % k);
    };
    std::vector<int> progress(Mb, 0);
    std::vector<std::vector<int>> xb(nx);  // bands of each XCD, in order
    for (int K = 0; K < Mb; ++K) xb[(K / gs) % nx].push_back(K);
    std::vector<size_t> xnext(nx, 0);
    std::vector<int> slot((size_t)nx * b, -1);  // band held by each band worker
    std::vector<int> cnt[2 * NCLS];             // vertical and horizontal counters per class
    for (auto& c : cnt) c.assign((size_t)Mb * Nb, 0);
    std::vector<Task> queue[NCLS];
    std::vector<size_t> head(NCLS, 0);
    std::vector<int> held[NCLS];
    for (int c = 0; c < NCLS; ++c) held[c].assign(W[c], -1);
    int64_t done_tasks = 0, steps = 0;
    int bands_done = 0;
    struct Act {
      int kind, a, b;
    };
    std::vector<Act> acts;
    for (;;) {
      acts.clear();
      for (int x = 0; x < nx; ++x)
        for (int k = 0; k < b; ++k) {
          const int K = slot[(size_t)x * b + k];
          if (K < 0) {
            if (xnext[x] < xb[x].size()) acts.push_back({0, x, k});  // claim a band
            continue;
          }
          const int L = progress[K];
          bool ok = K == 0 || progress[K - 1] > L;
          for (int c = 0; c < NCLS && ok; ++c)
            ok = cnt[2 * c][(size_t)K * Nb + L] >= expected_class(K, c) &&
                 cnt[2 * c + 1][(size_t)K * Nb + L] >= expected_class(L, c);
          if (ok) acts.push_back({1, x, k});  // complete the band's next block
        }
      for (int c = 0; c < NCLS; ++c)
        for (int k = 0; k < W[c]; ++k) {
          const int t = held[c][k];
          if (t < 0) {
            if (head[c] < queue[c].size()) acts.push_back({2, c, k});  // claim a task
            continue;
          }
          const Task& q = queue[c][t];
          bool ok = true;
          for (int T = q.p0; T <= q.p1 && ok; ++T) {
            const size_t idx = q.dir == 0 ? (size_t)T * Nb + q.other : (size_t)q.other * Nb + T;
            ok = cnt[2 * c + q.dir][idx] == push_seq(T, q.own, c);
          }
          if (ok) acts.push_back({3, c, k});  // apply the task
        }
      if (acts.empty()) break;
      const Act a = acts[rnd(acts.size())];
      ++steps;
      if (a.kind == 0) {
        slot[(size_t)a.a * b + a.b] = xb[a.a][xnext[a.a]++];
      } else if (a.kind == 1) {
        const int K = slot[(size_t)a.a * b + a.b], L = progress[K]++;
        int g0[6], g1[6], np[6];
        block_groups(K, L, Mb, Nb, g0, g1, np);
        for (int g = 0; g < 6; ++g) {
          const int cls = g >> 1, dir = g & 1;
          for (int k = 0; k < np[g]; ++k) {
            const int p0 = g0[g] + kPanel * k;
            const int p1 = p0 + kPanel - 1 < g1[g] ? p0 + kPanel - 1 : g1[g];
            queue[cls].push_back({dir, dir == 0 ? K : L, dir == 0 ? L : K, p0, p1});
          }
        }
        if (progress[K] == Nb) {
          slot[(size_t)a.a * b + a.b] = -1;
          ++bands_done;
        }
      } else if (a.kind == 2) {
        held[a.a][a.b] = (int)head[a.a]++;
      } else {
        const Task& q = queue[a.a][held[a.a][a.b]];
        for (int T = q.p0; T <= q.p1; ++T) {
          const size_t idx = q.dir == 0 ? (size_t)T * Nb + q.other : (size_t)q.other * Nb + T;
          cnt[2 * a.a + q.dir][idx] = push_seq(T, q.own, a.a) + 1;
        }
        held[a.a][a.b] = -1;
        ++done_tasks;
      }
    }
    int64_t queued = 0;
    for (int c = 0; c < NCLS; ++c) queued += (int64_t)queue[c].size();
    if (bands_done != Mb || done_tasks != queued) {
      snprintf(msg, sizeof msg,
               "sweep %dx%d, %d XCDs x %d band workers (groups of %d), update workers %d/%d/%d, "
               "seed %d: stuck after %lld steps with %d of %d bands and %lld of %lld tasks done",
               Mb, Nb, nx, b, gs, W[0], W[1], W[2], seed, (long long)steps, bands_done, Mb,
               (long long)done_tasks, (long long)queued);
      return fail(msg);
    }
  }
  printf("sweep %dx%d, %d XCDs x %d band workers (groups of %d), update workers %d/%d/%d: "
         "%d random schedules drained\n", Mb, Nb, nx, b, gs, W[0], W[1], W[2], seeds);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 3 && argv[1][0] == 'f') {
    std::vector<int> ns;
    for (int k = 2; k < argc; ++k) ns.push_back(atoi(argv[k]));
    return check_factor(ns);
  }
  if (argc == 4 && argv[1][0] == 's') return check_sweep(atoi(argv[2]), atoi(argv[3]));
  if ((argc == 5 || argc == 6) && argv[1][0] == 'q') {  // qrun P0 [P1] W SEEDS
    std::vector<int> ns;
    for (int k = 2; k < argc - 2; ++k) ns.push_back(atoi(argv[k]));
    return sim_factor(ns, atoi(argv[argc - 2]), atoi(argv[argc - 1]));
  }
  if (argc == 11 && argv[1][0] == 'r') {
    const int W[3] = {atoi(argv[7]), atoi(argv[8]), atoi(argv[9])};
    return sim_sweep(atoi(argv[2]), atoi(argv[3]), atoi(argv[4]), atoi(argv[5]), atoi(argv[6]),
                     W, atoi(argv[10]));
  }
  fprintf(stderr,
          "usage: %s factor P0 [P1] | qrun P0 [P1] WORKGROUPS SEEDS | sweep MB NB | run MB NB "
          "XCDS BANDWORKERS GROUP NEAR NEXT FAR SEEDS\n", argv[0]);
  return 2;
}
