// Placement of the Hessian's tile products over token splits (plain C++
// that also compiles for the device, so the mapping can be replayed on the
// host; see "GPTQ: Mathematical Foundations ...", Second-Order Taylor
// Expansion and the Hessian, for the product being split: H = 2·Σ_t x_t x_tᵀ
// is a sum over tokens, so any cut of the token range into splits sums to
// the same H).
//
// Tiles are the upper-triangle 256x256 tiles (ti <= tj) of H, nt per side.
// Tile order for L2 reuse: panels are grouped in fours, blocks (I, J) with
// I <= J in row-major order, tiles inside a block row-major (upper triangle
// only on the diagonal block: 10 tiles; 16 elsewhere).
//
// Token splits: every tile's token range is cut into S splits of `chunk`
// tokens, except (mixed plan) the tiles of the blocks in `hi_mask`, cut into
// S+1 splits of `chunk_hi`: with tiles·S workgroups a few short of a whole
// number of rounds of the CUs, the extra splits fill the last round.  Each
// XCD's run (workgroup L runs on XCD L % 8) starts with its share of the
// long workgroups (the S-split tiles, split by split, in tile order) and
// ends with its share of the short ones, so the rounds stay nearly even
// (longest first).
#pragma once

#include <cstdint>

#ifndef GQ_HD
#if defined(__HIPCC__)
#define GQ_HD __host__ __device__ __forceinline__
#else
#define GQ_HD inline
#endif
#endif

namespace gq {

struct SplitPlan {
  int64_t chunk, chunk_hi;
  int S;
  int hi_tiles;              // tiles in hi blocks (0: uniform plan)
  int long_per_xcd, short_per_xcd;
  uint64_t hi_mask;          // bit b: block b (row-major upper blocks) has S+1 splits
};

// The reduction's view: split count and shift count per 128-tile.
struct ReducePlan {
  int S, ng_hi;              // ng_hi: blocks per side of the mixed plan (0: uniform)
  uint64_t hi_mask;
  double shift_lo, shift_hi;
};

// idx-th upper tile of an nt x nt grid in row-major order
GQ_HD void tile_of(int idx, int nt, int& ti, int& tj) {
  int r = 0;
  while (idx >= nt - r) { idx -= nt - r; ++r; }
  ti = r;
  tj = r + idx;
}

// r-th tile in block order (nt a multiple of 4)
GQ_HD void block_tile(int r, int nt, int& ti, int& tj) {
  const int ng = nt / 4;
  for (int I = 0; I < ng; ++I)
    for (int J = I; J < ng; ++J) {
      const int n = (I == J) ? 10 : 16;
      if (r < n) {
        int a, b;
        if (I == J) tile_of(r, 4, a, b);
        else { a = r / 4; b = r % 4; }
        ti = 4 * I + a;
        tj = 4 * J + b;
        return;
      }
      r -= n;
    }
  ti = tj = 0;   // not reached for r < nt(nt+1)/2
}

// tiles in block b (row-major upper blocks, ng per side)
GQ_HD int block_size(int b, int ng) {
  int I = 0;
  while (b >= ng - I) { b -= ng - I; ++I; }
  return b == 0 ? 10 : 16;   // the diagonal block of row I comes first
}

// the k-th tile (block order) among the blocks whose hi_mask bit equals `hi`
GQ_HD int select_tile(int k, int ng, uint64_t mask, bool hi) {
  int r = 0;
  const int nb = ng * (ng + 1) / 2;
  for (int b = 0; b < nb; ++b) {
    const int n = block_size(b, ng);
    if ((((mask >> b) & 1u) != 0) == hi) {
      if (k < n) return r + k;
      k -= n;
    }
    r += n;
  }
  return r;   // not reached for k below the selected tiles' count
}

// workgroup L of a mixed plan: its tile, split and split length
GQ_HD void mixed_unit(int L, int nt, int tiles, const SplitPlan& sp, int& ti, int& tj, int& split,
                      int64_t& chunk) {
  const int x = L & 7, p = L >> 3, ng = nt / 4;
  int r;
  if (p < sp.long_per_xcd) {
    const int idx = x * sp.long_per_xcd + p, lo_tiles = tiles - sp.hi_tiles;
    split = idx / lo_tiles;
    r = select_tile(idx % lo_tiles, ng, sp.hi_mask, false);
    chunk = sp.chunk;
  } else {
    const int idx = x * sp.short_per_xcd + (p - sp.long_per_xcd);
    split = idx / sp.hi_tiles;
    r = select_tile(idx % sp.hi_tiles, ng, sp.hi_mask, true);
    chunk = sp.chunk_hi;
  }
  block_tile(r, nt, ti, tj);
}

// whether 128-tile (ti, tj) lies in a hi block (4x4 256-tiles = 8x8 128-tiles)
GQ_HD bool reduce_tile_hi(const ReducePlan& rp, int ti, int tj) {
  if (rp.ng_hi <= 0) return false;
  const int I = ti / 8, J = tj / 8;
  const int b = I * rp.ng_hi - I * (I - 1) / 2 + (J - I);
  return ((rp.hi_mask >> b) & 1u) != 0;
}

// Tokens' worth of μμᵀ the shift MFMAs take out of one tile over `splits`
// splits of `chunk` tokens: one shift per started group of `group` tokens
// (stages of `step` tokens, groups rounded up).
inline double shift_count(int64_t n_tok, int64_t chunk, int splits, int step, int group) {
  double c = 0.0;
  for (int s = 0; s < splits; ++s) {
    const int64_t lo = s * chunk, hi = (s + 1) * chunk < n_tok ? (s + 1) * chunk : n_tok;
    const int64_t stages = (hi - lo + step - 1) / step;
    c += (double)((stages + group / step - 1) / (group / step)) * group;
  }
  return c;
}

// The mixed split plan for tiles of side `ft` on `cus` CUs: give the tiles
// of a few blocks one split more so that the workgroup count becomes a
// whole number of rounds, with the same count of long and of short
// workgroups on every XCD.  The blocks are the first `a` diagonal and the
// first `b` off-diagonal ones with 10a + 16b the missing count; returns the
// uniform plan when no such set exists (or more than 64 blocks).
inline SplitPlan mixed_plan(int64_t d, int64_t n_tok, int S, int64_t chunk, int ft, int step,
                            int cus) {
  SplitPlan u{chunk, chunk, S, 0, 0, 0, 0};
  const int nt = (int)((d + ft - 1) / ft);
  if (nt % 4 != 0 || S < 2) return u;
  const int ng = nt / 4, nb = ng * (ng + 1) / 2;
  if (nb > 64) return u;
  const int tiles = nt * (nt + 1) / 2;
  const int64_t per = (n_tok + S) / (S + 1);
  const int64_t chunk_hi = (per + step - 1) / step * step;
  if ((n_tok + chunk_hi - 1) / chunk_hi != S + 1) return u;
  const int units = tiles * S;
  const int need = (units + cus - 1) / cus * cus - units;
  if (need == 0) return u;
  for (int a = 0; a <= ng; ++a) {
    const int rest = need - 10 * a;
    if (rest < 0) break;
    if (rest % 16 != 0 || rest / 16 > ng * (ng - 1) / 2) continue;
    const int b = rest / 16;
    const int lo_units = (tiles - need) * S, hi_units = need * (S + 1);
    if (lo_units % 8 != 0 || hi_units % 8 != 0) continue;
    uint64_t mask = 0;
    int da = 0, db = 0, blk = 0;
    for (int I = 0; I < ng; ++I)
      for (int J = I; J < ng; ++J, ++blk) {
        if (I == J && da < a) { mask |= 1ull << blk; ++da; }
        if (I != J && db < b) { mask |= 1ull << blk; ++db; }
      }
    return SplitPlan{chunk, chunk_hi, S, need, lo_units / 8, hi_units / 8, mask};
  }
  return u;
}

}  // namespace gq
