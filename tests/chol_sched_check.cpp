// Exhaustive check of the Cholesky update schedule (chol_sched.hpp) at
// 64x64-block granularity: every block below the diagonal receives each
// earlier panel's update exactly once, before its own panel's launch; what
// a launch's workgroups write is disjoint; every update reads finished
// panels.  Usage: chol_sched_check d [d ...]; prints one line per d and
// exits non-zero on the first violation.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "chol_sched.hpp"

using namespace gq::chol_sched;

static int fail(long d, const char* what, long k, long i, long j, long p) {
  std::printf("FAIL d=%ld launch=%ld block=(%ld,%ld) panel=%ld: %s\n", d, k, i, j, p, what);
  return 1;
}

static int check(long d) {
  const long nb = (d + kW - 1) / kW;   // 64-blocks = panels
  std::vector<unsigned char> got((size_t)(nb * nb * nb), 0);
  auto G = [&](long i, long j, long p) -> unsigned char& { return got[(size_t)((i * nb + j) * nb + p)]; };
  const auto far = far_schedule(d);
  if ((long)far.size() != nb) return fail(d, "schedule length", -1, -1, -1, -1);
  long nfar = 0, peak = 0, nupd = 0, cost = 0, peak_cost = 0;
  for (long k = 0; k < nb; ++k) {
    std::vector<signed char> wr((size_t)(nb * nb), 0);   // writer of each block in this launch
    auto write = [&](long i, long j, int who) -> bool {
      signed char& w = wr[(size_t)(i * nb + j)];
      if (w != 0 && w != who) return false;
      w = (signed char)who;
      return true;
    };
    // the panel: applies panel k-1 to its own column, then factors it
    for (long i = k; i < nb; ++i) {
      if (k > 0) {
        if (G(i, k, k - 1)) return fail(d, "pre-update twice", k, i, k, k - 1);
        G(i, k, k - 1) = 1;
      }
      for (long p = 0; p < k; ++p)
        if (G(i, k, p) != 1) return fail(d, "missing update at factor time", k, i, k, p);
      if (!write(i, k, 1)) return fail(d, "panel write overlap", k, i, k, -1);
    }
    const NearRegion n = near_region(d, k);
    if (n.c1 > n.c0) {
      if (n.c0 % kW || n.a0 % kW || n.K % kW) return fail(d, "near region not block aligned", k, -1, -1, -1);
      const long p0 = n.a0 / kW, p1 = (n.a0 + n.K) / kW;
      if (p1 > k) return fail(d, "near job reads an unfinished panel", k, -1, -1, p1 - 1);
      for (long j = n.c0 / kW; j < (n.c1 + kW - 1) / kW; ++j) {
        if (j <= k) return fail(d, "near job writes the panel or left of it", k, -1, j, -1);
        for (long i = j; i < nb; ++i) {
          if (!write(i, j, 2)) return fail(d, "near write overlap", k, i, j, -1);
          for (long p = p0; p < p1; ++p) {
            if (G(i, j, p)) return fail(d, "near update twice", k, i, j, p);
            G(i, j, p) = 1;
          }
        }
      }
    }
    long cnt = 0, kcost = 0;
    for (uint32_t w : far[(size_t)k]) {
      int r, t, s, ns;
      far_unpack(w, r, t, s, ns);
      ++cnt;
      nupd += ns;
      kcost += ns == 2 ? 3 : 2;   // half single-task units (a pair costs 1.5)
      if (r < t || 2L * (s + ns - 1) + 1 >= k) return fail(d, "far task reads an unfinished panel", k, r, t, s);
      for (long i = 2L * r; i < 2L * r + 2 && i < nb; ++i)
        for (long j = 2L * t; j < 2L * t + 2 && j < nb; ++j) {
          if (j > i) continue;
          if (j <= k) return fail(d, "far task writes the panel or left of it", k, i, j, s);
          if (!write(i, j, (int)(3 + (cnt % 100)))) return fail(d, "far write overlap", k, i, j, s);
          for (long p = 2L * s; p < 2L * (s + ns); ++p) {
            if (G(i, j, p)) return fail(d, "far update twice", k, i, j, p);
            G(i, j, p) = 1;
          }
        }
    }
    nfar += cnt;
    cost += kcost;
    peak = cnt > peak ? cnt : peak;
    peak_cost = kcost > peak_cost ? kcost : peak_cost;
  }
  for (long j = 0; j < nb; ++j)
    for (long i = j; i < nb; ++i)
      for (long p = 0; p < j; ++p)
        if (G(i, j, p) != 1) return fail(d, "update missing at the end", nb, i, j, p);
  std::printf("ok d=%ld launches=%ld far_tasks=%ld far_updates=%ld peak_per_launch=%ld cost=%ld peak_cost=%ld\n",
              d, nb, nfar, nupd, peak, cost, peak_cost);
  return 0;
}

int main(int argc, char** argv) {
  for (int a = 1; a < argc; ++a)
    if (check(std::atol(argv[a]))) return 1;
  return 0;
}
