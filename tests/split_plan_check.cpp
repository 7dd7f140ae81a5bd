// Exhaustive check of the Hessian's token-split placement (split_plan.hpp):
// for each (d, n_tok, S) on the command line, every workgroup of the mixed
// plan maps to a distinct (tile, split); every tile gets exactly its split
// count (S+1 in the hi blocks, S elsewhere), each with the split length of
// its class, the splits cover the token range, the reduction's per-tile rule
// agrees with the blocks the workgroups used, and each XCD runs the same
// number of long and of short workgroups.  Usage: split_plan_check d n S
// [d n S ...]; prints one line per case and exits non-zero on the first
// violation.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <tuple>

#include "split_plan.hpp"

using namespace gq;

static int check(long d, long n, int S) {
  constexpr int FT = 256, FK = 32, CUS = 256;
  const long chunk = ((n + S - 1) / S + FK - 1) / FK * FK;
  const SplitPlan p = mixed_plan(d, n, S, chunk, FT, FK, CUS);
  const int nt = (int)((d + FT - 1) / FT), tiles = nt * (nt + 1) / 2;
  if (p.hi_tiles == 0) {
    std::printf("d=%ld n=%ld S=%d: uniform plan\n", d, n, S);
    return 0;
  }
  const int grid = (tiles - p.hi_tiles) * S + p.hi_tiles * (S + 1);
  if (grid % CUS != 0 || grid != 8 * (p.long_per_xcd + p.short_per_xcd)) {
    std::printf("FAIL d=%ld: grid %d is not whole rounds / XCD shares\n", d, grid);
    return 1;
  }
  std::map<std::tuple<int, int, int>, long> seen;
  for (int L = 0; L < grid; ++L) {
    int ti, tj, split;
    int64_t ch;
    mixed_unit(L, nt, tiles, p, ti, tj, split, ch);
    if (ti < 0 || tj < ti || tj >= nt) {
      std::printf("FAIL d=%ld L=%d: tile (%d,%d) outside the upper triangle\n", d, L, ti, tj);
      return 1;
    }
    if (!seen.emplace(std::make_tuple(ti, tj, split), (long)ch).second) {
      std::printf("FAIL d=%ld L=%d: (%d,%d) split %d twice\n", d, L, ti, tj, split);
      return 1;
    }
  }
  const int ng = nt / 4;
  const ReducePlan rp{S, ng, p.hi_mask, 0.0, 0.0};
  for (int ti = 0; ti < nt; ++ti)
    for (int tj = ti; tj < nt; ++tj) {
      // the reduction works on 128-tiles: all four of this 256-tile agree
      const bool hi = reduce_tile_hi(rp, 2 * ti, 2 * tj);
      if (hi != reduce_tile_hi(rp, 2 * ti + 1, 2 * tj + 1)) {
        std::printf("FAIL d=%ld: 128-tiles of (%d,%d) disagree\n", d, ti, tj);
        return 1;
      }
      const int Ss = hi ? S + 1 : S;
      const long want = hi ? p.chunk_hi : p.chunk;
      for (int s = 0; s < Ss; ++s) {
        auto it = seen.find(std::make_tuple(ti, tj, s));
        if (it == seen.end() || it->second != want) {
          std::printf("FAIL d=%ld: tile (%d,%d) split %d missing or wrong length\n", d, ti, tj, s);
          return 1;
        }
      }
      if (seen.count(std::make_tuple(ti, tj, Ss))) {
        std::printf("FAIL d=%ld: tile (%d,%d) has a split past %d\n", d, ti, tj, Ss);
        return 1;
      }
      if ((long)Ss * want < n || (long)(Ss - 1) * want >= n) {
        std::printf("FAIL d=%ld: tile (%d,%d) splits do not cover the tokens\n", d, ti, tj);
        return 1;
      }
    }
  std::printf("d=%ld n=%ld S=%d: mixed plan ok (%d workgroups, %d tiles with %d splits)\n", d, n, S,
              grid, p.hi_tiles, S + 1);
  return 0;
}

int main(int argc, char** argv) {
  for (int i = 1; i + 2 < argc; i += 3)
    if (check(std::atol(argv[i]), std::atol(argv[i + 1]), std::atoi(argv[i + 2]))) return 1;
  return 0;
}
