// Host-side schedule of the trailing updates of the blocked Cholesky
// (plain C++, no device code, so it can be checked on its own).
//
// The factorization runs one launch per 64-wide panel k.  Panels are paired
// into 128-wide super-panels (super-panel s = panels 2s, 2s+1, columns
// [128s, 128s+128)).  Every trailing update G[i][j] −= Σ L[i][c]·L[j][c]
// has to reach column j before the launch of j's panel, and no two
// workgroups of one launch may write the same element.  Updates come from
// three places:
//   pre-update: launch k itself first applies panel k−1 to panel k's columns;
//   near job (rank 64, beside panel k):
//     k even: panel k−1 → column block k+1 (the other half of k's super-panel),
//     k odd:  panel k−1 → the next super-panel's 128 columns;
//   far tasks: one or two consecutive finished super-panels s, s+1 → the
//     128x128 tile (row tile r, column tile t), for every t ≥ s+2 and r ≥ t
//     (rank 128 or 256; a pair costs about 1.45 single tasks on the GPU,
//     measured, for twice the work).
// Super-panel s of tile (r, t) may be applied in launches [2s+2, 2t−2]:
// super-panel s is complete from launch 2s+2 on, and launch 2t−1's near job
// writes column tile t.  A tile takes at most one task per launch.  Within
// that freedom the tasks are spread so that each launch carries about the
// same cost: launches keep most CUs free of update tiles, so the panel (a
// serial, latency-bound chain) runs on a CU of its own, and no update tile
// takes much longer than the panel beside it.  The spreading is
// earliest-deadline-first with a constant cost target per launch: tiles
// whose remaining super-panels, two per launch, exactly fill their
// remaining window are always taken (with what is released, up to two);
// then tiles in order of least slack, while the target is not reached, but
// only with two released super-panels, so optional work is always paired.
#pragma once

#include <algorithm>
#include <cstdint>
#include <vector>

#ifndef GQ_HD
#if defined(__HIPCC__)
#define GQ_HD __host__ __device__ __forceinline__
#else
#define GQ_HD inline
#endif
#endif

namespace gq {
namespace chol_sched {

constexpr int kW = 64;      // panel width
constexpr int kSW = 128;    // super-panel width = far tile size

// task word: r, t, s in 10 bits each (d < 131072), bit 30: a pair (s, s+1)
GQ_HD uint32_t far_word(int r, int t, int s, int ns = 1) {
  return (uint32_t)r | ((uint32_t)t << 10) | ((uint32_t)s << 20) | ((uint32_t)(ns - 1) << 30);
}
GQ_HD void far_unpack(uint32_t w, int& r, int& t, int& s, int& ns) {
  r = (int)(w & 1023u);
  t = (int)((w >> 10) & 1023u);
  s = (int)((w >> 20) & 1023u);
  ns = 1 + (int)((w >> 30) & 1u);
}

// The near job of launch k: columns [c0, c1) (rows from c0 down) receive
// the update of G's columns [a0, a0 + K); tile = the update tile's size.
// Empty when c1 <= c0.
struct NearRegion {
  int64_t c0 = 0, c1 = 0, a0 = 0;
  int K = 0, tile = 64;
};
inline NearRegion near_region(int64_t d, int64_t k) {
  NearRegion n;
  if (k == 0) return n;
  if (k % 2 == 0) {   // panel k−1 → column block k+1
    n.c0 = kW * (k + 1);
    n.c1 = std::min<int64_t>(kW * (k + 2), d);
    n.tile = 64;
  } else {            // panel k−1 → the next super-panel
    n.c0 = kSW * (k / 2 + 1);
    n.c1 = std::min<int64_t>(n.c0 + kSW, d);
    n.tile = 128;
  }
  if (n.c0 >= n.c1) return NearRegion{};
  n.a0 = kW * (k - 1);
  n.K = kW;
  return n;
}

// Far tasks of every launch (index = panel k), in the order they are listed
// to the launch.
inline std::vector<std::vector<uint32_t>> far_schedule(int64_t d) {
  const int np = (int)((d + kW - 1) / kW);
  const int R = (int)((d + kSW - 1) / kSW);
  std::vector<std::vector<uint32_t>> out((size_t)np);
  if (R < 3) return out;
  struct Tile { int r, t, next; };
  std::vector<Tile> tiles;
  int64_t cost = 0;   // in half single-task units: a single 2, a pair 3
  for (int t = 2; t < R; ++t)
    for (int r = t; r < R; ++r) {
      tiles.push_back({r, t, 0});
      cost += (t - 1) / 2 * 3 + (t - 1) % 2 * 2;
    }
  const int lmax = 2 * (R - 1) - 2;   // last deadline
  const int64_t target = (3 * cost + 2 * (lmax - 1) - 1) / (2 * (lmax - 1));   // ⌈1.5·cost/(lmax−1)⌉
  std::vector<std::vector<int>> bucket((size_t)np + 2);
  for (int L = 0; L < np && L <= lmax; ++L) {
    for (auto& b : bucket) b.clear();
    const int released = L / 2;   // super-panels s with 2s+2 <= L
    for (int i = 0; i < (int)tiles.size(); ++i) {
      const Tile& x = tiles[i];
      const int U = x.t - 1, avail = std::min(U, released) - x.next;
      if (avail <= 0) continue;
      const int need = (U - x.next + 1) / 2, left = 2 * x.t - 2 - L + 1;
      const int slack = left - need;   // >= 0 (see the checker)
      bucket[(size_t)std::min(std::max(slack, 0), np + 1)].push_back(i);
    }
    int64_t taken = 0;
    for (int sl = 0; sl <= np + 1; ++sl) {
      for (int i : bucket[(size_t)sl]) {
        if (sl > 0 && taken >= target) break;
        Tile& x = tiles[i];
        const int avail = std::min(x.t - 1, released) - x.next;
        if (sl > 0 && avail < 2) continue;
        const int ns = std::min(avail, 2);
        out[(size_t)L].push_back(far_word(x.r, x.t, x.next, ns));
        x.next += ns;
        taken += ns == 2 ? 3 : 2;
      }
      if (taken >= target && sl > 0) break;
    }
  }
  return out;
}

}  // namespace chol_sched
}  // namespace gq
