// Preparation of the inverse-Hessian factor ("GPTQ: Mathematical Foundations
// ...": walkthrough steps 1-2, Hessian Damping and Numerical Regularization,
// Activation Ordering, Cholesky Decomposition and Pre-computation).
//
//   dead_i = (H_ii == 0) -> H_ii := 1;   λ = percdamp · mean(diag H)
//   π = stable descending order of diag H (identity without act-order)
//   H_d = (H + λI)[π][:, π];   U upper with H_d⁻¹ = UᵀU
//
// Route: instead of factoring H_d, inverting it and factoring the inverse
// (three O(d³) steps), H_d is factored in reversed index order.  With J the
// reversal, G = J·H_d·J = L·Lᵀ (ordinary lower Cholesky); then
// H_d = (JLJ)(JLJ)ᵀ with JLJ upper, so H_d⁻¹ = (JL⁻¹J)ᵀ(JL⁻¹J) and
// U = J·L⁻¹·J, the unique upper factor with positive diagonal.  Two O(d³)
// steps, both fp32: a blocked right-looking Cholesky with 64-wide panels
// (each diagonal block factored and inverted together, the panel below
// solved with that inverse; one launch per panel that also runs trailing
// updates on fp32 MFMA GEMM tiles: rank-64 near the panel, rank-128 tiles
// further right spread over the launches), then the rest of the triangular
// inverse by recursive
// doubling ([[A,0],[B,C]]⁻¹ has off-diagonal block −C⁻¹·B·A⁻¹, products
// skipping the zero triangles).
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <memory>
#include <vector>

#include <type_traits>

#include "common.hpp"
#include "chol_sched.hpp"
#include "gemm_dma.hpp"

namespace gq {
namespace {

constexpr int NB = kPanel;

// Dead fix, diagonal copy, damping constant.  One workgroup.
__global__ __launch_bounds__(1024) void diag_kernel(float* __restrict__ H, int64_t d,
                                                    uint8_t* __restrict__ dead_out,
                                                    float* __restrict__ diag, float percdamp,
                                                    float* __restrict__ lam, int* __restrict__ status) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 1024) {
    float h = H[i * d + i];
    const bool dead = (h == 0.f);
    if (dead) { h = 1.f; H[i * d + i] = 1.f; }
    diag[i] = h;
    if (dead_out) dead_out[i] = dead ? 1 : 0;
    acc += (double)h;
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    lam[0] = (float)((double)percdamp * part[0] / (double)d);
    status[0] = INT_MAX;   // smallest failing pivot
    status[1] = 0;         // a wave's bounded wait ran out
  }
}

// Stable descending rank sort: the position of i is
// #{j : key_j > key_i or (key_j == key_i and j < i)} (a NaN key counts as
// −inf).  Without act-order the order is the identity.  With it, workgroup
// (x, y) counts keys y·256.. against keys x·256.. from LDS and adds its
// partial counts atomically (integers: the sums do not depend on their
// order), then rank_scatter_kernel writes the order to the workspace and,
// when given, to the caller's perm_out.
__device__ __forceinline__ float rank_key(const float* diag, int j, int d) {
  const float v = j < d ? diag[j] : -INFINITY;
  return v != v ? -INFINITY : v;
}

__global__ __launch_bounds__(256) void rank_identity_kernel(int d, int* __restrict__ perm,
                                                            int* __restrict__ perm_out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < d) {
    perm[i] = i;
    if (perm_out) perm_out[i] = i;
  }
}

__global__ __launch_bounds__(256) void rank_count_kernel(const float* __restrict__ diag, int d,
                                                         int* __restrict__ cnt) {
  __shared__ __attribute__((aligned(16))) float kj[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int j0 = blockIdx.y * 256;
  kj[threadIdx.x] = rank_key(diag, j0 + threadIdx.x, d);   // keys past d: −inf, never counted
  const float ki = rank_key(diag, i, d);
  __syncthreads();
  int rank = 0;
#pragma unroll 8
  for (int k = 0; k < 256; k += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(kj + k);
#pragma unroll
    for (int u = 0; u < 4; ++u) rank += (v[u] > ki) || (v[u] == ki && j0 + k + u < i);
  }
  if (i < d && rank > 0) atomicAdd(cnt + i, rank);
}

__global__ __launch_bounds__(256) void rank_scatter_kernel(const int* __restrict__ cnt, int d,
                                                           int* __restrict__ perm,
                                                           int* __restrict__ perm_out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < d) {
    perm[cnt[i]] = i;
    if (perm_out) perm_out[cnt[i]] = i;
  }
}

__global__ __launch_bounds__(256) void zero_int_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// G[a][b] = H[π(d−1−a)][π(d−1−b)] + λ·[a == b]: the damped, permuted and
// index-reversed Hessian.  Each thread writes 4 consecutive columns of one
// row (one float4 when d is a multiple of 4); its 4 source indices are
// loaded together, then its 4 sources.
__global__ __launch_bounds__(256) void build_g_kernel(const float* __restrict__ H, int64_t d,
                                                      const int* __restrict__ perm,
                                                      const float* __restrict__ lam,
                                                      float* __restrict__ G, int ident) {
  const float l = lam[0];
  const bool vec = (d & 3) == 0;
  if (ident && vec) {   // π = identity: row d−1−a of H read backwards, a float4 at a time
    for (int64_t b0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; b0 < d;
         b0 += (int64_t)gridDim.x * 1024)
      for (int64_t a = blockIdx.y; a < d; a += gridDim.y) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(H + (d - 1 - a) * d + d - 4 - b0);
        f32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = v[3 - q] + ((a == b0 + q) ? l : 0.f);
        *reinterpret_cast<f32x4*>(G + a * d + b0) = o;
      }
    return;
  }
  for (int64_t b0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; b0 < d;
       b0 += (int64_t)gridDim.x * 1024) {
    int pb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pb[q] = b0 + q < d ? perm[d - 1 - b0 - q] : 0;
    for (int64_t a = blockIdx.y; a < d; a += gridDim.y) {
      const float* hr = H + (int64_t)perm[d - 1 - a] * d;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = b0 + q < d ? hr[pb[q]] : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] += (a == b0 + q) ? l : 0.f;
      if (vec) {
        const f32x4 o = {v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(G + a * d + b0) = o;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (b0 + q < d) G[a * d + b0 + q] = v[q];
      }
    }
  }
}

// The permuted G for rows that fit in LDS (d ≤ kRowLds): one row a per
// workgroup step.  Row π(d−1−a) of H is staged in LDS with coalesced
// loads, then every thread gathers its columns from LDS and writes them
// coalesced (a gather from memory moves one 4-byte word per access).  The
// source columns π(d−1−b) are re-read for every row (the same 4·d bytes,
// from cache): held in registers they would cost occupancy.
constexpr int kRowLds = 16384;          // floats per staged row (64 KB)
__global__ __launch_bounds__(256) void build_g_rows_kernel(const float* __restrict__ H, int d,
                                                           const int* __restrict__ perm,
                                                           const float* __restrict__ lam,
                                                           float* __restrict__ G) {
  extern __shared__ __attribute__((aligned(16))) float row[];
  const float l = lam[0];
  const int t = threadIdx.x;
  const bool vec = (d & 3) == 0;
  for (int a = blockIdx.x; a < d; a += gridDim.x) {
    const float* src = H + (int64_t)perm[d - 1 - a] * d;
    __syncthreads();   // the previous row's gathers are done
    // every load of a pass before its first LDS store
    if (vec) {
      for (int e0 = 0; e0 < d; e0 += 8192) {
        f32x4 buf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + 1024 * u + 4 * t;
          if (e < d) buf[u] = *reinterpret_cast<const f32x4*>(src + e);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + 1024 * u + 4 * t;
          if (e < d) *reinterpret_cast<f32x4*>(row + e) = buf[u];
        }
      }
    } else {
      for (int e0 = 0; e0 < d; e0 += 4096) {
        float buf[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + 256 * u + t;
          buf[u] = e < d ? src[e] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + 256 * u + t;
          if (e < d) row[e] = buf[u];
        }
      }
    }
    __syncthreads();
    float* dst = G + (int64_t)a * d;
    for (int b0 = 4 * t; b0 < d; b0 += 1024) {
      int pb[4];
      if (vec) {   // π(d−1−b0−q), q = 0..3: one aligned int4, reversed
        const int4 p4 = *reinterpret_cast<const int4*>(perm + d - 4 - b0);
        pb[0] = p4.w; pb[1] = p4.z; pb[2] = p4.y; pb[3] = p4.x;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) pb[q] = b0 + q < d ? perm[d - 1 - b0 - q] : 0;
      }
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = row[pb[q]] + ((a == b0 + q) ? l : 0.f);
      if (vec) {
        const f32x4 o = {v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(dst + b0) = o;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (b0 + q < d) dst[b0 + q] = v[q];
      }
    }
  }
}

struct PanelArgs {
  float* G; int64_t d; int k0, kb;   // G: the n x n matrix being factored (n = d here)
  float* Linv; int* status;
  int np;          // panel workgroups in the launch
  int spin_limit;  // bound on every flag wait (polls; 0 allows none)
  int64_t ld;      // row stride of G and Linv
  int piv_base;    // index of G's first column in the whole factorization
};

// A panel workgroup keeps four 64x64 blocks in LDS with float4-aligned rows
// and works on them as 16x16 tiles.  In the tile layout a lane (l16, kq) of
// a wave (l16 = lane % 16, kq = lane / 16) holds row l16, columns
// 4kq..4kq+3 of a tile: one float4 in registers, one ds_read_b128 in LDS.
constexpr int PS = NB + 4;       // LDS row stride (floats)
constexpr int PBLK = NB * PS;    // one block

__device__ __forceinline__ float* tile(float* B, int i, int j) { return B + 16 * i * PS + 16 * j; }
__device__ __forceinline__ f32x4 ld_t(const float* T, int l16, int kq) {
  return *reinterpret_cast<const f32x4*>(T + l16 * PS + 4 * kq);
}
__device__ __forceinline__ void st_t(float* T, int l16, int kq, f32x4 v) {
  *reinterpret_cast<f32x4*>(T + l16 * PS + 4 * kq) = v;
}

// acc + sign·R·Sᵀ for 16-row operands R and S of K columns, in the tile
// layout.  v_mfma_f32_16x16x4f32 takes a[x][k] = S[x][k] and b[k][y] =
// R[y][k] (lane (l16, kq) supplies row l16 of each) and leaves D[x][y] at
// lane (y, kq), rows x = 4kq + v: D = S·Rᵀ = (R·Sᵀ)ᵀ, i.e. row y of R·Sᵀ.
// Lane group kq takes k = (K/4)·kq + step, the same permutation for both
// operands, so each lane reads whole float4s.
template <int K>
__device__ __forceinline__ f32x4 mm_rs(const float* R, const float* S, f32x4 acc, float sign,
                                       int l16, int kq) {
  constexpr int NQ = K / 16;
  f32x4 rv[NQ], sv[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    rv[q] = *reinterpret_cast<const f32x4*>(R + l16 * PS + (K / 4) * kq + 4 * q);
    sv[q] = *reinterpret_cast<const f32x4*>(S + l16 * PS + (K / 4) * kq + 4 * q);
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sign * sv[q][u], rv[q][u], acc, 0, 0, 0);
  return acc;
}

// acc + sign·R·Z for 16x16 tiles, Z read by columns (a[x][k] = Z[k][x]).
__device__ __forceinline__ f32x4 mm_rz(const float* R, const float* Z, f32x4 acc, float sign,
                                       int l16, int kq) {
  const f32x4 rv = ld_t(R, l16, kq);
  float zv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) zv[u] = Z[(4 * kq + u) * PS + l16];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sign * zv[u], rv[u], acc, 0, 0, 0);
  return acc;
}

// lane J of every 16-lane row (DPP row_newbcast)
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + J, 0xf, 0xf, true));
}
// the value of 16-lane row Gr, at the same position, in all four rows (a
// permlane32 swap brings Gr's half to both halves, a permlane16 swap its row
// to both rows of each half)
template <int Gr>
__device__ __forceinline__ float grp_bcast(float v) {
  const unsigned u = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned y = (Gr < 2) ? p[0] : p[1];
  const auto q = __builtin_amdgcn_permlane16_swap(y, y, false, false);
  return __uint_as_float((Gr & 1) ? q[1] : q[0]);
}

template <int J>
__device__ __forceinline__ void f16_step(float (&a)[4], float (&r)[4], float& piv, float& inv_row,
                                         int i, int& bad) {
  constexpr int g = J >> 2, e = J & 3;
  const bool b = !(piv > 0.f) || !(piv < INFINITY);
  bad = (b && bad < 0) ? J : bad;
  // one hardware reciprocal square root on the serial chain (about 1 ulp)
  const float inv = b ? 1.f : __builtin_amdgcn_rsqf(piv);
  if constexpr (J < 15) {
    constexpr int g1 = (J + 1) >> 2, e1 = (J + 1) & 3;
    const float sa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[e]), 16 * g + J + 1));
    const float s1 =
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[e1]), 16 * g1 + J + 1));
    const float c = sa * inv;   // l[J+1][J]
    piv = fmaf(-c, c, s1);
  }
  const float col = grp_bcast<g>(a[e]);   // A[i][J]
  const float m = i > J ? -(col * (inv * inv)) : 0.f;
  inv_row = i == J ? inv : inv_row;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    a[q] = fmaf(row_bcast<J>(a[q]), m, a[q]);
    r[q] = fmaf(row_bcast<J>(r[q]), m, r[q]);
  }
}

template <int J>
__device__ __forceinline__ void f16_steps(float (&a)[4], float (&r)[4], float& piv, float& inv_row,
                                          int i, int& bad) {
  f16_step<J>(a, r, piv, inv_row, i, bad);
  if constexpr (J < 15) f16_steps<J + 1>(a, r, piv, inv_row, i, bad);
}

// Cholesky factor and inverse of a 16x16 SPD tile held by one wave in the
// tile layout (both triangles): x receives X = L⁻¹ (lower, exact zeros
// above the diagonal) in the same layout; bad the first non-positive (or
// NaN/inf) pivot's index, else −1 (such a pivot is replaced by 1 so the
// arithmetic stays finite).  Right-looking, one step per column j: with p
// the pivot and m_i = A[i][j]/p for i > j, A[i][k] −= m_i·A[j][k] (the
// rank-1 update by l = A[:, j]/√p, row j standing in for column j by
// symmetry) and R[i][k] −= m_i·R[j][k] on rows R of the identity, which
// turns R into √p-scaled rows of X; row i of X is R's row i times 1/√p of
// step i.  Row j is lane j of each 16-lane row (one DPP source operand);
// column j sits in one 16-lane row and reaches the other three by two
// permlane swaps.  The next pivot comes from two entries read before the
// step's update, so the serial chain per step is rsq, mul, fma.
__device__ __forceinline__ void factor16(const f32x4 acc, float (&x)[4], int l16, int kq,
                                         int& bad) {
  float a[4] = {acc[0], acc[1], acc[2], acc[3]};
  float r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (l16 == 4 * kq + e) ? 1.f : 0.f;
  float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[0]), 0));
  float inv_row = 0.f;
  bad = -1;
  f16_steps<0>(a, r, piv, inv_row, l16, bad);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = r[e] * inv_row;
}

constexpr int kSpinLimit = 1 << 20;   // default bound on a flag wait (never reached)

// What the routines of one panel workgroup's waves share.
struct PanelCtx {
  float *AS, *BS, *PP, *QQ;   // LDS blocks (see panel_body)
  int* fl;                    // L_{i,s} published: fl[4i + s]
  float *G, *Linv;
  int64_t d, ld, R0;
  int k0, kb, l16, kq, spin_limit;
  bool upd, rows, stalled;
};

// Bounded wait for a flag; after one expired wait a wave stops waiting and
// status[1] later marks the whole call, whose outputs are then undefined.
__device__ __forceinline__ void wait_flag(PanelCtx& c, int f) {
  for (int spin = 0; !c.stalled; ++spin) {
    if (spin >= c.spin_limit) {
      c.stalled = true;
      break;
    }
    if (__hip_atomic_load(&c.fl[f], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) break;
    __builtin_amdgcn_s_sleep(1);
  }
}
// one wave's LDS operations complete in order, so a flag stored after a
// tile vouches for it
__device__ __forceinline__ void publish(PanelCtx& c, int f) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __hip_atomic_store(&c.fl[f], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// a tile-layout value to row `row` (0..63 of the block), columns col..col+3
// of a 64-column block of G (L21) or Linv (X), within [0, kb) columns
__device__ __forceinline__ void store_row4(float* dst, bool vec, int col, int kb, f32x4 v) {
  if (vec && col + 3 < kb) {
    *reinterpret_cast<f32x4*>(dst) = v;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < kb) dst[e] = v[e];
  }
}
// L21 tile (rb, s) of this workgroup's rows
__device__ __forceinline__ void store_l21(const PanelCtx& c, f32x4 v, int rb, int s) {
  const int64_t row = c.R0 + 16 * rb + c.l16;
  const int col = 16 * s + 4 * c.kq;
  if (row < c.d) store_row4(c.G + row * c.ld + c.k0 + col, (c.ld & 3) == 0, col, c.kb, v);
}
// X tile (i, j) into Linv's diagonal block
__device__ __forceinline__ void store_x(const PanelCtx& c, f32x4 v, int i, int j) {
  const int row = 16 * i + c.l16, col = 16 * j + 4 * c.kq;
  if (row < c.kb)
    store_row4(c.Linv + (int64_t)(c.k0 + row) * c.ld + c.k0 + col, (c.ld & 3) == 0, col, c.kb, v);
}

// acc + sign·R·Sᵀ with both 16x16 operands in registers (tile layout)
__device__ __forceinline__ f32x4 mm_reg(f32x4 r, f32x4 s, f32x4 acc, float sign) {
#pragma unroll
  for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sign * s[u], r[u], acc, 0, 0, 0);
  return acc;
}

// X's off-diagonal tile (s, j), j < s: X_{s,j} = −X_s·Σ_{k=j}^{s−1} L_{s,k}·X_{k,j}
// (the off-diagonal block of the inverse of a block-lower-triangular
// matrix, one block row at a time).  Row block s >= 1 of X lives in PP's
// row block s−1; scr is a scratch tile.
__device__ __forceinline__ f32x4 x_tile(const PanelCtx& c, int s, int j, float* scr) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = j; k < s; ++k) {
    const float* Z = k == j ? tile(c.AS, j, j) : tile(c.PP, k - 1, j);   // X_{k,j}
    acc = mm_rz(tile(c.AS, s, k), Z, acc, 1.f, c.l16, c.kq);
  }
  st_t(scr, c.l16, c.kq, acc);
  return mm_rz(tile(c.AS, s, s), scr, f32x4{0.f, 0.f, 0.f, 0.f}, -1.f, c.l16, c.kq);
}

// Slab 0, waves 1-3 (h = wave − 1): the previous panel's contribution to
// A's tiles below A_00 (9 tiles) and to B's first column tile (4), K = 64
// each; tasks h, h+3, ... two at a time so their MFMA chains interleave.
__device__ __forceinline__ void pre_tasks(const PanelCtx& c, int h) {
  const int l16 = c.l16, kq = c.kq;
  for (int t0 = h; t0 < 13; t0 += 6) {
    float* C[2];
    const float* R[2];
    const float* S[2];
    bool ok[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int task = t0 + 3 * x;
      ok[x] = task < 9 || (task < 13 && c.rows);
      if (task < 9) {
        const int ti = task < 2 ? 1 : (task < 5 ? 2 : 3);
        const int tj = task < 2 ? task : (task < 5 ? task - 2 : task - 5);
        C[x] = tile(c.AS, ti, tj);
        R[x] = c.PP + 16 * ti * PS;
        S[x] = c.PP + 16 * tj * PS;
      } else {
        const int rb = task < 13 ? task - 9 : 0;
        C[x] = tile(c.BS, rb, 0);
        R[x] = c.QQ + 16 * rb * PS;
        S[x] = c.PP;
      }
    }
    f32x4 rv[2][4], sv[2][4], acc[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      acc[x] = ld_t(C[x], l16, kq);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rv[x][q] = *reinterpret_cast<const f32x4*>(R[x] + l16 * PS + 16 * kq + 4 * q);
        sv[x][q] = *reinterpret_cast<const f32x4*>(S[x] + l16 * PS + 16 * kq + 4 * q);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int x = 0; x < 2; ++x)
          acc[x] = __builtin_amdgcn_mfma_f32_16x16x4f32(-sv[x][q][u], rv[x][q][u], acc[x], 0, 0, 0);
#pragma unroll
    for (int x = 0; x < 2; ++x)
      if (ok[x]) st_t(C[x], l16, kq, acc[x]);
  }
}

// Slab PH−1 on A (wave 1): the slab's L tiles below row block PH
// (L_{i,s} = A_{i,s}·X_sᵀ, published), its update of the trailing tiles
// (i, j), PH <= j <= i, except A_PH,PH (wave 0's), and on workgroup 0 row
// block PH−1 of X.  Operands of each group are read first and the MFMA
// chains interleaved.
template <int PH>
__device__ __forceinline__ void a_helper(PanelCtx& c, bool xduty) {
  constexpr int S = PH - 1, NA = 3 - PH;
  const int l16 = c.l16, kq = c.kq;
  if constexpr (NA > 0) {
    constexpr int NO = NA * (NA + 1) / 2;
    const f32x4 xs = ld_t(tile(c.AS, S, S), l16, kq);
    f32x4 ai[NA], la[NA], co[NO], cw[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      ai[i] = ld_t(tile(c.AS, PH + 1 + i, S), l16, kq);
      cw[i] = ld_t(tile(c.AS, PH + 1 + i, PH), l16, kq);
    }
    {
      int n = 0;
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j) co[n++] = ld_t(tile(c.AS, PH + 1 + i, PH + 1 + j), l16, kq);
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) la[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NA; ++i) la[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[u], ai[i][u], la[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      st_t(tile(c.AS, PH + 1 + i, S), l16, kq, la[i]);
      publish(c, 4 * (PH + 1 + i) + S);
    }
    {
      int n = 0;
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j, ++n) co[n] = mm_reg(la[i], la[j], co[n], -1.f);
    }
    wait_flag(c, 4 * PH + S);
    const f32x4 lph = ld_t(tile(c.AS, PH, S), l16, kq);
#pragma unroll
    for (int i = 0; i < NA; ++i) cw[i] = mm_reg(la[i], lph, cw[i], -1.f);
    {
      int n = 0;
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        st_t(tile(c.AS, PH + 1 + i, PH), l16, kq, cw[i]);
#pragma unroll
        for (int j = 0; j <= i; ++j, ++n) st_t(tile(c.AS, PH + 1 + i, PH + 1 + j), l16, kq, co[n]);
      }
    }
  }
  if constexpr (S >= 1) {
    if (xduty) {
      float* xrow = c.PP + 16 * (S - 1) * PS;
#pragma unroll
      for (int j = 0; j < S; ++j) st_t(xrow + 16 * j, l16, kq, x_tile(c, S, j, xrow + 48));
    }
  }
}

// Slab PH−1 on B row tiles rb0 .. rb0+NR−1 of this workgroup's rows: the
// slab's L21 tile (LB = B_{rb,s}·X_sᵀ, to G), the previous panel's part of
// column tile PH (K = 64), then the slab's update of column tiles PH..3
// (B_{rb,j} −= LB·L_{j,s}ᵀ) as the L tiles are published.
template <int PH, int NR>
__device__ __forceinline__ void b_rows(PanelCtx& c, int rb0) {
  constexpr int S = PH - 1, NJ = 4 - PH;
  const int l16 = c.l16, kq = c.kq;
  const f32x4 xs = ld_t(tile(c.AS, S, S), l16, kq);
  f32x4 bs[NR], cc[NR][NJ], qv[NR][4], pv[4], lb[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    bs[r] = ld_t(tile(c.BS, rb0 + r, S), l16, kq);
#pragma unroll
    for (int j = 0; j < NJ; ++j) cc[r][j] = ld_t(tile(c.BS, rb0 + r, PH + j), l16, kq);
  }
  if (c.upd) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pv[q] = *reinterpret_cast<const f32x4*>(c.PP + (16 * PH + l16) * PS + 16 * kq + 4 * q);
#pragma unroll
      for (int r = 0; r < NR; ++r)
        qv[r][q] = *reinterpret_cast<const f32x4*>(c.QQ + (16 * (rb0 + r) + l16) * PS + 16 * kq + 4 * q);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) lb[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < NR; ++r) lb[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[u], bs[r][u], lb[r], 0, 0, 0);
#pragma unroll
  for (int r = 0; r < NR; ++r) store_l21(c, lb[r], rb0 + r, S);
  if (c.upd) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < NR; ++r)
          cc[r][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(-pv[q][u], qv[r][q][u], cc[r][0], 0, 0, 0);
  }
  f32x4 lj[NJ];
#pragma unroll
  for (int j = NJ - 1; j >= 0; --j) {   // the later tiles' L (wave 1) come before L_PH,s (wave 0)
    wait_flag(c, 4 * (PH + j) + S);
    lj[j] = ld_t(tile(c.AS, PH + j, S), l16, kq);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < NR; ++r)
        cc[r][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(-lj[j][u], lb[r][u], cc[r][j], 0, 0, 0);
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int j = 0; j < NJ; ++j) st_t(tile(c.BS, rb0 + r, PH + j), l16, kq, cc[r][j]);
}

// Slab PH: wave 0 computes L_{PH,PH−1} = A_{PH,PH−1}·X_{PH−1}ᵀ (published),
// applies it to A_PH,PH and factors that; waves 1-3 apply slab PH−1 (B row
// tiles 3 on wave 1 beside A, 0 and 1 on wave 2, 2 on wave 3).
template <int PH>
__device__ __forceinline__ void phase(PanelCtx& c, int w, float (&xr)[4], int& bad_j, bool xduty) {
  constexpr int S = PH - 1;
  const int l16 = c.l16, kq = c.kq;
  if (w == 0) {
    const f32x4 av = ld_t(tile(c.AS, PH, S), l16, kq);
    f32x4 cc = ld_t(tile(c.AS, PH, PH), l16, kq);
    f32x4 l = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) l = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[u], av[u], l, 0, 0, 0);
    st_t(tile(c.AS, PH, S), l16, kq, l);
    publish(c, 4 * PH + S);
    cc = mm_reg(l, l, cc, -1.f);
    int bd;
    factor16(cc, xr, l16, kq, bd);
    if (bad_j < 0 && bd >= 0) bad_j = 16 * PH + bd;
    st_t(tile(c.AS, PH, PH), l16, kq, f32x4{xr[0], xr[1], xr[2], xr[3]});
  } else if (w == 1) {
    a_helper<PH>(c, xduty);
    if (c.rows) b_rows<PH, 1>(c, 3);
  } else if (w == 2) {
    if (c.rows) b_rows<PH, 2>(c, 0);
  } else {
    if (c.rows) b_rows<PH, 1>(c, 2);
  }
  __syncthreads();
}

// One 64-wide Cholesky panel at column k0 (kb <= 64 columns, padded with
// the identity), for workgroup b of the panel's grid:
//   the previous panel's contribution to this panel's columns,
//     G[:, panel] −= L21ₚ·L21ₚ[panel rows]ᵀ (the trailing updates of the
//     previous launch skip these columns so this launch can run it),
//   L11 = chol(G11),  X = L11⁻¹,  L21 = G21·Xᵀ.
// Every workgroup factors the diagonal block itself, so no workgroup waits
// for another; workgroup b solves the 64 rows k0+kb+64b .. +63 of the panel
// in place in G, and workgroup 0 also writes X into the diagonal block of
// Linv (L11 itself is not needed later).
//
// Blocked in four 16-column slabs s.  Wave 0 runs the serial chain in
// registers: L_{s,s−1} = A_{s,s−1}·X_{s−1}ᵀ, A_ss −= L_{s,s−1}·L_{s,s−1}ᵀ,
// then the 16x16 factor of A_ss (factor16) gives X_s.  Waves 1-3 apply slab
// s−1 meanwhile: the other L tiles of the slab, its update of the trailing
// A tiles, and for this workgroup's rows the slab's L21 tile (stored to G)
// and its update of the later B tiles; they also apply the previous panel's
// contribution to B one 16-column tile ahead of its use, and (workgroup 0)
// build X's off-diagonal tiles.  One workgroup barrier per slab; inside a
// slab the L tiles are published through LDS flags, every wait bounded.  All
// products are v_mfma_f32_16x16x4f32 on 16x16 tiles.
__device__ __forceinline__ void panel_body(const PanelArgs& p, int b, float* __restrict__ smem) {
  float* AS = smem;              // G11; its tiles become X_s (diagonal) and L_{i,s} (below)
  float* BS = smem + PBLK;       // this workgroup's 64 rows of G21
  float* PP = smem + 2 * PBLK;   // the previous panel's values in the panel's rows; row block
                                 // m is free after slab m's pre-update and holds X's row m+1
  float* QQ = smem + 3 * PBLK;   // the previous panel's values in this workgroup's rows
  int* fl = reinterpret_cast<int*>(smem + 4 * PBLK);
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t d = p.d, ld = p.ld;
  const int k0 = p.k0, kb = p.kb;
  const int64_t R0 = (int64_t)k0 + kb + (int64_t)b * NB;
  const bool upd = k0 > 0;       // previous panels are full width
  const int kp = k0 - NB;
  float* G = p.G;
  {
    // all loads first, then the masks and the LDS stores.  A keeps its lower
    // triangle and, inside the diagonal tiles, the mirrored upper part (read
    // transposed).  Full-width panels of a 4-aligned G load float4: thread t
    // covers rows (t >> 4) + 16u, columns 4(t & 15) .. +3.
    if ((ld & 3) == 0 && k0 + NB <= d) {
      const int c4 = 4 * (t & 15);
      f32x4 va[4], vb[4], vp[4], vq[4];
      float vt[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = (t >> 4) + 16 * u;
        const int64_t ra = k0 + i, rb = R0 + i < d ? R0 + i : 0;
        va[u] = *reinterpret_cast<const f32x4*>(G + ra * ld + k0 + c4);
        vb[u] = *reinterpret_cast<const f32x4*>(G + rb * ld + k0 + c4);
        if (upd) {
          vp[u] = *reinterpret_cast<const f32x4*>(G + ra * ld + kp + c4);
          vq[u] = *reinterpret_cast<const f32x4*>(G + rb * ld + kp + c4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = c4 + e;
          vt[u][e] = (k > i && (k >> 4) == (i >> 4)) ? G[(int64_t)(k0 + k) * ld + k0 + i] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = (t >> 4) + 16 * u;
        const bool okb = R0 + i < d;
        f32x4 oa, ob, op, oq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = c4 + e;
          oa[e] = k <= i ? va[u][e] : vt[u][e];
          ob[e] = okb ? vb[u][e] : 0.f;
          op[e] = upd ? vp[u][e] : 0.f;
          oq[e] = (upd && okb) ? vq[u][e] : 0.f;
        }
        *reinterpret_cast<f32x4*>(AS + i * PS + c4) = oa;
        *reinterpret_cast<f32x4*>(BS + i * PS + c4) = ob;
        *reinterpret_cast<f32x4*>(PP + i * PS + c4) = op;
        *reinterpret_cast<f32x4*>(QQ + i * PS + c4) = oq;
      }
    } else {
      // ragged or unaligned panels (rare): four batches of four elements per
      // array keep the registers of this path below the float4 path's
      for (int u0 = 0; u0 < 16; u0 += 4) {
        float va[4], vb[4], vp[4], vq[4];
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          const int idx = t + 256 * (u0 + uu), i = idx >> 6, k = idx & 63;
          const bool in = i < kb && k < kb, tr = k > i && (k >> 4) == (i >> 4);
          const bool oka = in && (k <= i || tr);
          const int ai = k <= i ? i : k, ak = k <= i ? k : i;
          va[uu] = G[(int64_t)(k0 + (oka ? ai : 0)) * ld + k0 + (oka ? ak : 0)];
          const bool okb = R0 + i < d && k < kb;
          vb[uu] = G[(okb ? R0 + i : 0) * ld + (okb ? k0 + k : 0)];
          const bool okp = upd && i < kb, okq = upd && R0 + i < d;
          vp[uu] = G[(int64_t)(okp ? k0 + i : 0) * ld + (okp ? kp + k : 0)];
          vq[uu] = G[(okq ? R0 + i : 0) * ld + (okq ? kp + k : 0)];
        }
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          const int idx = t + 256 * (u0 + uu), i = idx >> 6, k = idx & 63;
          const bool in = i < kb && k < kb, tr = k > i && (k >> 4) == (i >> 4);
          AS[i * PS + k] = in ? ((k <= i || tr) ? va[uu] : 0.f) : (i == k ? 1.f : 0.f);
          BS[i * PS + k] = (R0 + i < d && k < kb) ? vb[uu] : 0.f;
          PP[i * PS + k] = (upd && i < kb) ? vp[uu] : 0.f;
          QQ[i * PS + k] = (upd && R0 + i < d) ? vq[uu] : 0.f;
        }
      }
    }
  }
  if (t < 16) fl[t] = 0;
  __syncthreads();

  PanelCtx c{AS, BS, PP, QQ, fl, G, p.Linv, d, ld, R0, k0, kb, lane & 15, lane >> 4,
             p.spin_limit, upd, R0 < d, false};
  const int l16 = c.l16, kq = c.kq;
  const bool xduty = b == 0;
  float xr[4];    // wave 0: X of the slab it factored last
  int bad_j = -1;
  // slab 0: wave 0 applies the previous panel to A_00 and factors it; the
  // other waves apply it to the rest of A and to B's first column tile
  if (w == 0) {
    f32x4 acc = ld_t(tile(AS, 0, 0), l16, kq);
    if (upd) acc = mm_rs<64>(PP, PP, acc, -1.f, l16, kq);
    factor16(acc, xr, l16, kq, bad_j);
    st_t(tile(AS, 0, 0), l16, kq, f32x4{xr[0], xr[1], xr[2], xr[3]});
  } else if (upd) {
    pre_tasks(c, w - 1);
  }
  __syncthreads();
  phase<1>(c, w, xr, bad_j, xduty);
  phase<2>(c, w, xr, bad_j, xduty);
  phase<3>(c, w, xr, bad_j, xduty);

  // slab 3's L21 tiles (one per wave); workgroup 0: X's last row block
  // (waves 1-3) and the rest of X (wave 0) to Linv
  if (c.rows) store_l21(c, mm_rs<16>(tile(BS, w, 3), tile(AS, 3, 3), f32x4{0.f, 0.f, 0.f, 0.f}, 1.f, l16, kq), w, 3);
  if (xduty) {
    if (w > 0) {
      const int j = w - 1;
      store_x(c, x_tile(c, 3, j, tile(PP, 2, j)), 3, j);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) store_x(c, ld_t(tile(AS, i, i), l16, kq), i, i);
      store_x(c, ld_t(tile(PP, 0, 0), l16, kq), 1, 0);
      store_x(c, ld_t(tile(PP, 1, 0), l16, kq), 2, 0);
      store_x(c, ld_t(tile(PP, 1, 1), l16, kq), 2, 1);
    }
  }
  if (b == 0 && w == 0 && lane == 0 && bad_j >= 0) atomicMin(p.status, p.piv_base + k0 + bad_j);
  if (lane == 0 && c.stalled) atomicOr(p.status + 1, 1);
}

// Lower-triangular tile enumeration: L -> (row by, column bx <= by).
__device__ __forceinline__ void lower_tile(int L, int& by, int& bx) {
  int y = (int)((sqrtf(8.f * (float)L + 1.f) - 1.f) * 0.5f);
  while ((y + 1) * (y + 2) / 2 <= L) ++y;
  while (y * (y + 1) / 2 > L) --y;
  by = y;
  bx = L - y * (y + 1) / 2;
}

// Without a permutation H_d = H + λI: H already holds the dead fix (its
// off-diagonal entries never change), so only the diagonal moves.
__global__ __launch_bounds__(256) void add_diag_kernel(float* __restrict__ H, int64_t d,
                                                       const float* __restrict__ lam) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < d) H[i * d + i] += lam[0];
}

// H_out[x][y] = H_d[x][y] rebuilt from G's untouched strict upper triangle
// (G = J·H_d·J, so H_d[x][y] = G[d-1-x][d-1-y]), one lower 64x64 tile of
// H_out per workgroup: the tile is read along G's rows, written directly,
// and written transposed through LDS as its mirror above the diagonal.
__global__ __launch_bounds__(256) void write_hd_kernel(float* __restrict__ H, int64_t d,
                                                       const float* __restrict__ G,
                                                       const float* __restrict__ diag,
                                                       const int* __restrict__ perm,
                                                       const float* __restrict__ lam) {
  int by, bx;
  lower_tile(blockIdx.x, by, bx);
  __shared__ float T[64][65];
  const int t = threadIdx.x;
  for (int e = t; e < 64 * 64; e += 256) {
    const int i = e >> 6, j = e & 63;
    const int64_t x = 64 * by + i, y = 64 * bx + j;
    float v = 0.f;
    if (x < d && y < d) {
      if (x == y) v = diag[perm[x]] + lam[0];
      else if (x > y) v = G[(d - 1 - x) * d + (d - 1 - y)];
      else v = G[(d - 1 - y) * d + (d - 1 - x)];   // inside a diagonal tile only
      H[x * d + y] = v;
    }
    T[i][j] = v;
  }
  if (by == bx) return;
  __syncthreads();
  for (int e = t; e < 64 * 64; e += 256) {
    const int jj = e >> 6, ii = e & 63;   // output row 64bx+jj, column 64by+ii
    const int64_t y = 64 * bx + jj, x = 64 * by + ii;
    if (x < d && y < d) H[y * d + x] = T[ii][jj];
  }
}

// Trailing-update work beside one panel (the schedule is in chol_sched.hpp).
// Near job: a product C −= A·Aᵀ over a region whose top-left corner lies on
// G's diagonal, cut into tile x tile output tiles on or below the diagonal
// and numbered column by column.
struct TileJob {
  gemm_detail::KArgs g;
  int count, nby, tile;
  int dma;   // the shapes suit the DMA tile
};
// Far tasks: 128x128 tiles of G −= Lₛ·Lₛᵀ for one super-panel s or a pair
// s, s+1 (K = 128 or 256), one packed (row tile, column tile, super-panel,
// pair) word per task, four workgroups (the tile's 64x64 quarters) per task.
constexpr int kMaxFar = 512;
struct FarJob {
  gemm_detail::KArgs g;   // A = B = C = G, K = 128; A and B move to super-panel s
  int count, dma;
  uint32_t task[kMaxFar];
};
constexpr int kRing64 = 8;    // DMA ring depths: 64 KB for 64-tiles, 64 KB for 128-tiles
constexpr int kRing128 = 4;
static_assert(gemm_detail::DTile<64, kRing64>::SMEM <= gemm_detail::GEMM_SMEM_FLOATS * 4, "");
static_assert(gemm_detail::DTile<128, kRing128>::SMEM <= gemm_detail::GEMM_SMEM_FLOATS * 4, "");

// LDS of a Cholesky launch: the panel or one update tile.  Below half of
// the CU's 160 KB, so two workgroups of a launch can share a CU (the
// register count allows two waves per SIMD).  Without the DMA path a
// 128-tile runs as four 64-tiles, whose operand buffers are smaller.
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kCholSmemFloats =
    cmax(cmax(4 * PBLK + 16, 4 * gemm_detail::Tile<64>::OPF),
         cmax(gemm_detail::DTile<64, kRing64>::SMEM, gemm_detail::DTile<128, kRing128>::SMEM) / 4);
static_assert(kCholSmemFloats * 4 <= 72 * 1024, "a Cholesky launch's LDS must allow two workgroups per CU");

template <int T>
__device__ __forceinline__ void job_tile(const gemm_detail::KArgs& g, bool dma, int bx, int by,
                                         float* smem) {
  constexpr int NS = T == 64 ? kRing64 : kRing128;
  if (dma) {
    gemm_detail::gemm_tile_dma<T, NS, false, true>(g, bx, by, 0, 1, reinterpret_cast<char*>(smem));
  } else if constexpr (T == 64) {
    gemm_detail::gemm_tile<64, false, true>(g, bx, by, 0, 1, smem);
  } else {
    for (int q = 0; q < 4; ++q) {
      if (q > 0) __syncthreads();
      gemm_detail::gemm_tile<64, false, true>(g, 2 * bx + (q & 1), 2 * by + (q >> 1), 0, 1, smem);
    }
  }
}

__device__ __forceinline__ void run_near_tile(const TileJob& j, int idx, float* smem) {
  int bx = 0;
  while (idx >= j.nby - bx) { idx -= j.nby - bx; ++bx; }
  if (j.tile == 64) job_tile<64>(j.g, j.dma, bx, bx + idx, smem);
  else job_tile<128>(j.g, j.dma, bx, bx + idx, smem);
}

// One 64x64 quarter (sub: row half sub >> 1, column half sub & 1) of far
// task idx; a diagonal task's quarter above the diagonal has nothing to do.
__device__ __forceinline__ void run_far_tile(const FarJob& f, int idx, int sub, float* smem) {
  int r, t, sp, ns;
  chol_sched::far_unpack(f.task[idx], r, t, sp, ns);
  const int by = 2 * r + (sub >> 1), bx = 2 * t + (sub & 1);
  if (bx > by) return;
  gemm_detail::KArgs g = f.g;
  g.A += (int64_t)sp * chol_sched::kSW;
  g.B += (int64_t)sp * chol_sched::kSW;
  g.K = g.k_last = ns * chol_sched::kSW;   // one or two super-panels
  job_tile<64>(g, f.dma, bx, by, smem);
}

// One step of the blocked Cholesky: workgroups [0, nP) run panel k (its
// columns first receive the previous panel's update), the rest run the
// near job's tiles and then the far tasks listed for this launch (four
// workgroups each).  The
// schedule guarantees that they all write disjoint parts of G and read
// only finished panels.  A launch with nP = 0 runs far tasks only.
__global__ __launch_bounds__(256) void chol_step_kernel(PanelArgs p, int nP, TileJob nj,
                                                        FarJob fj) {
  __shared__ __attribute__((aligned(1024))) float smem[kCholSmemFloats];
  const int L = blockIdx.x;
  if (L < nP) panel_body(p, L, smem);
  else if (L < nP + nj.count) run_near_tile(nj, L - nP, smem);
  else {
    // Workgroup L runs on XCD L % 8: in every run of 32 far workgroups the
    // four quarters of a task sit 8 apart, on one XCD, so the L rows they
    // share come through one L2 (the last, partial run keeps index order).
    const int f = L - nP - nj.count, b = f >> 5;
    if (8 * b + 8 <= fj.count) run_far_tile(fj, 8 * b + (f & 7), (f & 31) >> 3, smem);
    else run_far_tile(fj, f >> 2, f & 3, smem);
  }
}

// U[a][b] = Linv[d-1-a][d-1-b] for b >= a, 0 below the diagonal; four
// columns per thread (one reversed float4 of Linv when d is a multiple of 4).
__global__ __launch_bounds__(256) void write_u_kernel(const float* __restrict__ Linv, int64_t d,
                                                      float* __restrict__ U) {
  const bool vec = (d & 3) == 0;
  for (int64_t a = blockIdx.y; a < d; a += gridDim.y) {
    const float* lr = Linv + (d - 1 - a) * d;
    for (int64_t b0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; b0 < d;
         b0 += (int64_t)gridDim.x * 1024) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      if (vec) {
        if (b0 + 3 >= a) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(lr + d - 4 - b0);
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = b0 + q >= a ? v[3 - q] : 0.f;
        }
        *reinterpret_cast<f32x4*>(U + a * d + b0) = o;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (b0 + q < d) U[a * d + b0 + q] = b0 + q >= a ? lr[d - 1 - b0 - q] : 0.f;
      }
    }
  }
}

// Linv starts as zeros: the doubling products read whole diagonal blocks,
// whose strict upper parts must be zero.
__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

TileJob near_job(float* G, int64_t d, int64_t ld, int64_t k) {
  const chol_sched::NearRegion n = chol_sched::near_region(d, k);
  TileJob j{};
  if (n.c1 <= n.c0) return j;
  GemmArgs h{};  // G[c0:, c0:c1] −= G[c0:, a0:a0+K] · G[c0:c1, a0:a0+K]ᵀ  (lower part)
  h.M = (int)(d - n.c0); h.N = (int)(n.c1 - n.c0); h.K = n.K; h.k_last = n.K; h.batch = 1;
  h.alpha = -1.f; h.beta = 1.f;
  h.A = G + n.c0 * ld + n.a0; h.lda = ld; h.trans_a = false;
  h.B = G + n.c0 * ld + n.a0; h.ldb = ld; h.trans_b = true;
  h.C = G + n.c0 * ld + n.c0; h.ldc = ld; h.tri = 1;
  j.g = gemm_detail::make_kargs(h);
  j.dma = gemm_detail::dma_ok(j.g, false, true) ? 1 : 0;
  j.tile = n.tile;
  j.nby = (int)ceil_div(d - n.c0, n.tile);
  const int nbx = (int)ceil_div(n.c1 - n.c0, n.tile);
  j.count = nbx * j.nby - nbx * (nbx - 1) / 2;
  return j;
}

FarJob far_base(float* G, int64_t d, int64_t ld) {
  FarJob f;
  GemmArgs h{};  // tile (r, t): G[128r:, 128t:] −= G[128r:, 128s:+K] · G[128t:, 128s:+K]ᵀ
  h.M = (int)d; h.N = (int)d; h.K = chol_sched::kSW; h.k_last = chol_sched::kSW; h.batch = 1;
  h.alpha = -1.f; h.beta = 1.f;
  h.A = G; h.lda = ld; h.trans_a = false;
  h.B = G; h.ldb = ld; h.trans_b = true;
  h.C = G; h.ldc = ld; h.tri = 1;
  f.g = gemm_detail::make_kargs(h);
  // the per-task offsets of A and B (128 floats) keep the alignment
  f.dma = gemm_detail::dma_ok(f.g, false, true) ? 1 : 0;
  f.count = 0;
  return f;
}

// ---------------------------------------------------------------- leading panel in fp64
// The first 64 columns of G are eliminated in fp64.  When the activations
// share a non-zero mean, H (and G) is dominated by one large rank-1 part
// and the Schur complement left after the first columns is orders of
// magnitude smaller than the entries it comes from: an fp32 update there
// cancels to a few correct bits.  The first panel takes that part out, so
// its factor, its inverse and its update of the rest are formed in fp64
// (the L values stored back and used in the update are the fp32 ones the
// rest of the factorization reads); everything after it is well scaled and
// runs in fp32.

// Whether the leading panel needs fp64.  Its elimination cancels when G
// carries one large common part (activations sharing a channel mean make H
// close to rank one on top of the rest), and that shows in the correlations
// |G_ij|/sqrt(G_ii·G_jj) between the panel's 64 columns and the later ones:
// near 1 for a common part, about 1/sqrt(tokens) for independent zero-mean
// channels.  Their mean above kLeadCorr turns the fp64 panel on (for
// d <= 64 the panel is the whole matrix and always runs in fp64).
// lead_corr_kernel: one wave per row i >= 64 (its 64 panel entries are one
// coalesced load), kCorrBlocks partial sums in a fixed order, so the
// decision is deterministic; lead_panel_kernel adds them up.
constexpr float kLeadCorr = 0.1f;
constexpr int kCorrBlocks = 128;
__global__ __launch_bounds__(256) void lead_corr_kernel(const float* __restrict__ G, int64_t d,
                                                        double* __restrict__ part) {
  __shared__ double wsum[4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float gj = G[(int64_t)lane * d + lane];
  const float rs = gj > 0.f ? __builtin_amdgcn_rsqf(gj) : 0.f;
  double acc = 0.0;
  // two rows per iteration, both rows' loads issued before either is used
  constexpr int64_t S = (int64_t)kCorrBlocks * 4;
  for (int64_t i = NB + (int64_t)blockIdx.x * 4 + wv; i < d; i += 2 * S) {
    const bool two = i + S < d;
    const float* r0 = G + i * d;
    const float* r1 = G + (two ? i + S : i) * d;
    float v0 = fabsf(r0[lane]) * rs, v1 = fabsf(r1[lane]) * rs;
    const float g0 = r0[i], g1 = r1[two ? i + S : i];
    for (int o = 32; o > 0; o >>= 1) {
      v0 += __shfl_xor(v0, o);
      v1 += __shfl_xor(v1, o);
    }
    acc += g0 > 0.f ? (double)(v0 * __builtin_amdgcn_rsqf(g0)) : 0.0;
    if (two) acc += g1 > 0.f ? (double)(v1 * __builtin_amdgcn_rsqf(g1)) : 0.0;
  }
  if (lane == 0) wsum[wv] = acc;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// by one wave: lane l adds part[l] and part[l + 64], then a fixed tree; the
// sum is lane 0's, so every workgroup takes the same decision
__device__ __forceinline__ int lead_decide(const double* part, int64_t d, int lane) {
  if (d <= NB) return 1;
  static_assert(kCorrBlocks == 128, "two partial sums per lane");
  double v = part[lane] + part[lane + 64];
  for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o);
  return v / ((double)(d - NB) * (double)NB) > (double)kLeadCorr ? 1 : 0;
}

// The leading panel in fp64, one launch: every workgroup factors and inverts
// the 64x64 leading block itself (no workgroup waits for another), then
// workgroup b solves rows 64 + 64b .. +63 below it, L21 = G21·Xᵀ, and stores
// them rounded to fp32 in L21b [(d−64) x 64]; workgroup 0 stores X = L11⁻¹
// (rounded) in X0b [64 x 64] and reports a failed pivot (not positive or not
// finite; replaced by 1) in *status.  Blocks narrower than 64 (kb < 64) are
// padded with the identity.
//
// Lane i of every wave holds row i; wave w holds columns 16w .. 16w+15 in
// registers.  Step j of the factorization: the owner of column j scales it by
// 1/l_jj and publishes it in LDS (one barrier), and every wave updates its
// later columns, a_ik −= l_ij·l_kj.  X then comes column block by column
// block, each wave on its own 16 columns with no barrier: for k = 0..63, row
// k of the block is final once scaled by 1/l_kk, and every later row
// subtracts l_ik times it (row k reaches the other lanes through LDS: a
// wave's LDS operations complete in order).
__global__ __launch_bounds__(256) void lead_panel_kernel(const float* __restrict__ G, int64_t d,
                                                         int64_t ld, int kb, float* __restrict__ L21b,
                                                         float* __restrict__ X0b,
                                                         int* __restrict__ status,
                                                         const double* __restrict__ part,
                                                         int* __restrict__ flag) {
  // every workgroup takes the decision itself; workgroup 0 publishes it for
  // the kernels after this one
  __shared__ int on;
  if (threadIdx.x < 64) {
    const int dec = lead_decide(part, d, threadIdx.x);
    if (threadIdx.x == 0) {
      on = dec;
      if (blockIdx.x == 0) flag[0] = dec;
    }
  }
  __syncthreads();
  if (!on) return;
  __shared__ double Lc[NB][NB + 1];   // L by columns as they are published
  __shared__ double Xs[NB][NB + 1];
  __shared__ double Rs[NB][NB + 1];   // this workgroup's rows of G21
  __shared__ double dinv[NB];
  __shared__ int bad;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t r0 = NB + (int64_t)blockIdx.x * NB;
  if (t == 0) bad = INT_MAX;
  // G21 rows (every load before the stores)
  {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = t + 256 * u, rr = e >> 6, k = e & 63;
      v[u] = (r0 + rr < d && k < kb) ? G[(r0 + rr) * ld + k] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int e = t + 256 * u;
      Rs[e >> 6][e & 63] = (double)v[u];
    }
  }
  double a[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int k = 16 * w + q;
    a[q] = (lane < kb && k <= lane) ? (double)G[(int64_t)lane * ld + k] : (lane == k ? 1.0 : 0.0);
  }
  __syncthreads();
  for (int j = 0; j < NB; ++j) {
    if ((j >> 4) == w) {   // owner: column j = register j & 15
      double cj = 0.0;
#pragma unroll
      for (int q = 0; q < 16; ++q) cj = (q == (j & 15)) ? a[q] : cj;
      double piv = __shfl(cj, j);
      if (!(piv > 0.0) || !(piv < INFINITY)) {
        if (lane == 0) atomicMin(&bad, j);
        piv = 1.0;
      }
      const double ljj = sqrt(piv), inv = 1.0 / ljj;
      const double l = lane > j ? cj * inv : (lane == j ? ljj : 0.0);
      Lc[lane][j] = l;
      if (lane == 0) dinv[j] = inv;
    }
    __syncthreads();
    const double li = Lc[lane][j];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int k = 16 * w + q;
      if (k > j) a[q] = fma(-li, Lc[k][j], a[q]);
    }
  }
  // X, column block of wave w: x[q] = X[lane][16w + q]
  double x[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) x[q] = (lane == 16 * w + q) ? 1.0 : 0.0;
  for (int k = 0; k < NB; ++k) {
    const double dk = dinv[k], lik = Lc[lane][k];
    if (lane == k) {   // row k is final: publish it
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        x[q] *= dk;
        Xs[k][16 * w + q] = x[q];
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const double xk = Xs[k][16 * w + q];
      if (lane > k) x[q] = fma(-lik, xk, x[q]);
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) {
#pragma unroll
    for (int q = 0; q < 16; ++q) X0b[lane * NB + 16 * w + q] = (float)x[q];
    if (t == 0 && bad < kb) atomicMin(status, bad);
  }
  // L21 rows r0 + lane, columns 16w + q: Σ_{k <= j} G21[lane][k]·X[j][k]
  if (r0 + lane < d && r0 < d) {
    double acc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.0;
    for (int k = 0; k < NB; ++k) {
      const double g = Rs[lane][k];
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = fma(g, Xs[16 * w + q][k], acc[q]);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) L21b[(r0 - NB + lane) * NB + 16 * w + q] = (float)acc[q];
  }
}

// G22 −= L21·L21ᵀ over the lower triangle of the trailing (d−64)² block, in
// fp64 from the stored fp32 L21 (exact products), rounded once.  One 128x128
// lower tile (by >= bx) per workgroup, the two 128x64 strips of L21 staged
// in LDS as fp32 (rows padded to 65: the row groups a wave reads fall in
// distinct banks); thread t takes rows (t / 16) + 16a and columns
// (t % 16) + 16b, a, b = 0..7, and keeps its 64 sums in fp64 registers.
constexpr int LT = 128;
__global__ __launch_bounds__(256) void lead_update_kernel(float* __restrict__ G, int64_t d, int64_t ld,
                                                          const float* __restrict__ L21b,
                                                          const int* __restrict__ flag) {
  if (!flag[0]) return;
  int by = (int)((sqrtf(8.f * (float)blockIdx.x + 1.f) - 1.f) * 0.5f);
  while ((by + 1) * (by + 2) / 2 <= (int)blockIdx.x) ++by;
  while (by * (by + 1) / 2 > (int)blockIdx.x) --by;
  const int bx = (int)blockIdx.x - by * (by + 1) / 2;
  __shared__ float Ra[LT][NB + 1];
  __shared__ float Rb[LT][NB + 1];
  const int t = threadIdx.x;
  const int64_t ra0 = NB + (int64_t)by * LT, rb0 = NB + (int64_t)bx * LT;
  {
    // every load before the LDS stores: 32 floats of each strip a thread
    float va[32], vb[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int e = t + 256 * u, rr = e >> 6, k = e & 63;
      va[u] = ra0 + rr < d ? L21b[(ra0 - NB + rr) * NB + k] : 0.f;
      vb[u] = rb0 + rr < d ? L21b[(rb0 - NB + rr) * NB + k] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int e = t + 256 * u, rr = e >> 6, k = e & 63;
      Ra[rr][k] = va[u];
      Rb[rr][k] = vb[u];
    }
  }
  __syncthreads();
  const int ti = t >> 4, tj = t & 15;
  double acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
  for (int k = 0; k < NB; ++k) {
    double x[8], y[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      x[a] = (double)Ra[ti + 16 * a][k];
      y[a] = (double)Rb[tj + 16 * a][k];
    }
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[a][b] = fma(x[a], y[b], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int64_t r = ra0 + ti + 16 * a;
    if (r >= d) continue;
    float* row = G + r * ld;
    float old[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int64_t c = rb0 + tj + 16 * b;
      old[b] = (c <= r) ? row[c] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int64_t c = rb0 + tj + 16 * b;
      if (c <= r) row[c] = (float)((double)old[b] - acc[a][b]);
    }
  }
}

// Before the fp32 factorization: the leading 64 columns of G become those of
// the identity (lower part only; G's strict upper triangle is kept for the
// act-order H_d write-back), so its first panel factors to I and applies a
// zero update.  After it: the leading panel's own L21 and X = L11⁻¹ go back
// into G and Linv for the triangular inverse.
__global__ __launch_bounds__(256) void lead_identity_kernel(float* __restrict__ G, int64_t d,
                                                            const int* __restrict__ flag) {
  if (!flag[0]) return;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < d * NB; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / NB, c = e % NB;
    if (c <= r) G[r * d + c] = (r == c) ? 1.f : 0.f;
  }
}
__global__ __launch_bounds__(256) void lead_restore_kernel(float* __restrict__ G, float* __restrict__ Linv,
                                                           int64_t d, int kb,
                                                           const float* __restrict__ L21b,
                                                           const float* __restrict__ X0b,
                                                           const int* __restrict__ flag) {
  if (!flag[0]) return;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < d * NB; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / NB, c = e % NB;
    if (r >= NB) G[r * d + c] = L21b[(r - NB) * NB + c];
    else if (r < kb && c < kb) Linv[r * d + c] = X0b[r * NB + c];
  }
}

struct PrepWs {
  int* status; double* corr; float* lam; float* diag; int* perm; int* cnt; float* G; float* Linv; float* T;
};

PrepWs carve(void* ws, int64_t d) {
  char* p = static_cast<char*>(ws);
  PrepWs w;
  w.status = reinterpret_cast<int*>(p); p += 256;
  w.corr = reinterpret_cast<double*>(p); p += 1024;
  w.lam = reinterpret_cast<float*>(p); p += 256;
  w.diag = reinterpret_cast<float*>(p); p += align_up((size_t)d * 4);
  w.perm = reinterpret_cast<int*>(p); p += align_up((size_t)d * 4);
  w.cnt = reinterpret_cast<int*>(p); p += align_up((size_t)d * 4);
  w.G = reinterpret_cast<float*>(p); p += align_up((size_t)d * d * 4);
  w.Linv = reinterpret_cast<float*>(p); p += align_up((size_t)d * d * 4);
  w.T = reinterpret_cast<float*>(p);
  return w;
}

}  // namespace

size_t prepare_ws_bytes(int64_t d) {
  // T: the doubling's products (d²/2 + 64² floats); the leading panel's fp64
  // inverse (64² doubles) uses it first
  return 1536 + 3 * align_up((size_t)d * 4) + 2 * align_up((size_t)d * d * 4) +
         align_up((size_t)(d * d / 2 + 2 * NB * NB) * 4);
}

hipError_t prepare_launch(float* H, int64_t d, float percdamp, int act_order, float* U,
                          int32_t* perm_out, uint8_t* dead_mask, void* ws, int32_t** status_dev,
                          hipStream_t s) {
  PrepWs w = carve(ws, d);
  *status_dev = w.status;
  hipError_t e;
#define GQ_CHECK()                             \
  do {                                         \
    e = hipGetLastError();                     \
    if (e != hipSuccess) return e;             \
  } while (0)
  diag_kernel<<<1, 1024, 0, s>>>(H, d, dead_mask, w.diag, percdamp, w.lam, w.status);
  GQ_CHECK();
  {
    const unsigned nb = (unsigned)ceil_div(d, 256);
    if (!act_order) {
      rank_identity_kernel<<<nb, 256, 0, s>>>((int)d, w.perm, perm_out);
    } else {
      zero_int_kernel<<<nb, 256, 0, s>>>(w.cnt, (int)d);
      GQ_CHECK();
      rank_count_kernel<<<dim3(nb, nb), 256, 0, s>>>(w.diag, (int)d, w.cnt);
      GQ_CHECK();
      rank_scatter_kernel<<<nb, 256, 0, s>>>(w.cnt, (int)d, w.perm, perm_out);
    }
  }
  GQ_CHECK();
  const unsigned gy = (unsigned)std::min<int64_t>(d, 65535);
  if (act_order && d <= kRowLds)
    build_g_rows_kernel<<<(unsigned)std::min<int64_t>(d, 1024), 256, (size_t)d * 4, s>>>(
        H, (int)d, w.perm, w.lam, w.G);
  else
    build_g_kernel<<<dim3((unsigned)ceil_div(d, 1024), gy), 256, 0, s>>>(H, d, w.perm, w.lam, w.G,
                                                                        act_order ? 0 : 1);
  GQ_CHECK();
  zero_kernel<<<(unsigned)std::min<int64_t>(ceil_div(d * d, 256), 8192), 256, 0, s>>>(w.Linv, d * d);
  GQ_CHECK();

  // The leading 64 columns in fp64 (lead_panel_kernel, lead_update_kernel:
  // L21 and X of the first panel kept aside in T), then the blocked
  // right-looking Cholesky (lower) of G in fp32 with the first panel's
  // columns set to the identity (a zero update), 64-wide panels, one launch
  // per panel, trailing updates in two levels; then the first panel's L21
  // and X go back.
  const int kb0 = (int)std::min<int64_t>(NB, d);
  float* L21b = w.T;
  float* X0b = w.T + (size_t)std::max<int64_t>(d - NB, 0) * NB;
  {
    TimerScope lead_ts(kTimerLead, s);
    int* flag = w.status + 2;
    if (d > NB) {
      lead_corr_kernel<<<kCorrBlocks, 256, 0, s>>>(w.G, d, w.corr);
      GQ_CHECK();
    }
    const int64_t nb = std::max<int64_t>(1, ceil_div(d - NB, NB));
    lead_panel_kernel<<<(unsigned)nb, 256, 0, s>>>(w.G, d, d, kb0, L21b, X0b, w.status, w.corr,
                                                   flag);
    GQ_CHECK();
    if (d > NB) {
      const int64_t nt = ceil_div(d - NB, LT);
      lead_update_kernel<<<(unsigned)(nt * (nt + 1) / 2), 256, 0, s>>>(w.G, d, d, L21b, flag);
      GQ_CHECK();
    }
    lead_identity_kernel<<<(unsigned)std::min<int64_t>(ceil_div(d * NB, 256), 1024), 256, 0, s>>>(
        w.G, d, flag);
    GQ_CHECK();
  }
  std::unique_ptr<TimerScope> chol_ts(new TimerScope(kTimerChol, s));
  const std::vector<std::vector<uint32_t>> far = chol_sched::far_schedule(d);
  // GPTQ_PANEL_SPIN_LIMIT (diagnostics only) shortens the panels' bounded
  // flag waits so that the stall report can be exercised
  int spin_limit = kSpinLimit;
  if (const char* sl = std::getenv("GPTQ_PANEL_SPIN_LIMIT")) spin_limit = std::max(0, std::atoi(sl));
  FarJob fj = far_base(w.G, d, d);
  for (int64_t k = 0; k * NB < d; ++k) {
    const int64_t k0 = k * NB;
    const int kb = (int)std::min<int64_t>(NB, d - k0);
    const int64_t nr = d - (k0 + kb);
    const int nP = (int)std::max<int64_t>(1, ceil_div(nr, NB));
    PanelArgs pa{w.G, d, (int)k0, kb, w.Linv, w.status, nP, spin_limit, d, 0};
    const TileJob nj = near_job(w.G, d, d, k);
    const std::vector<uint32_t>& ft = far[(size_t)k];
    // far tasks beyond one launch's list run first, in launches of their own
    size_t done = 0;
    while (ft.size() - done > (size_t)kMaxFar) {
      fj.count = kMaxFar;
      std::copy(ft.begin() + (ptrdiff_t)done, ft.begin() + (ptrdiff_t)(done + kMaxFar), fj.task);
      chol_step_kernel<<<(unsigned)(4 * kMaxFar), 256, 0, s>>>(pa, 0, TileJob{}, fj);
      GQ_CHECK();
      done += kMaxFar;
    }
    fj.count = (int)(ft.size() - done);
    std::copy(ft.begin() + (ptrdiff_t)done, ft.end(), fj.task);
    chol_step_kernel<<<(unsigned)(nP + nj.count + 4 * fj.count), 256, 0, s>>>(pa, nP, nj, fj);
    GQ_CHECK();
  }
  lead_restore_kernel<<<(unsigned)std::min<int64_t>(ceil_div(d * NB, 256), 1024), 256, 0, s>>>(
      w.G, w.Linv, d, kb0, L21b, X0b, w.status + 2);
  GQ_CHECK();
  chol_ts.reset();
  // triangular inverse by recursive doubling on 64-aligned blocks
  TimerScope inv_ts(kTimerInverse, s);
  for (int64_t sz = NB; sz < d; sz *= 2) {
    const int64_t full = d / (2 * sz);                 // pairs with a full C block
    const int64_t rag0 = full * 2 * sz;                // start of a ragged pair, if any
    const int64_t rag_c = std::max<int64_t>(0, std::min<int64_t>(sz, d - rag0 - sz));
    for (int pass = 0; pass < 2; ++pass) {
      const int64_t batch = pass == 0 ? full : (rag_c > 0 ? 1 : 0);
      if (batch == 0) continue;
      const int64_t r0 = pass == 0 ? 0 : rag0;
      const int64_t sc = pass == 0 ? sz : rag_c;
      GemmArgs t{};  // T = B · A⁻¹
      t.M = (int)sc; t.N = (int)sz; t.K = (int)sz; t.k_last = (int)sz; t.batch = (int)batch;
      t.alpha = 1.f; t.beta = 0.f;
      t.A = w.G + (r0 + sz) * d + r0; t.lda = d; t.strideA = 2 * sz * (d + 1); t.trans_a = false;
      t.B = w.Linv + r0 * d + r0; t.ldb = d; t.strideB = 2 * sz * (d + 1); t.trans_b = false;
      t.C = w.T; t.ldc = sz; t.strideC = sz * sz; t.tri = 0;
      t.k_from_n = 1;  // A⁻¹ is lower triangular: column n needs k >= n only
      if ((e = gemm_f32(t, s)) != hipSuccess) return e;
      GemmArgs x{};  // X21 = −C⁻¹ · T
      x.M = (int)sc; x.N = (int)sz; x.K = (int)sc; x.k_last = (int)sc; x.batch = (int)batch;
      x.alpha = -1.f; x.beta = 0.f;
      x.A = w.Linv + (r0 + sz) * d + (r0 + sz); x.lda = d; x.strideA = 2 * sz * (d + 1);
      x.trans_a = false;
      x.B = w.T; x.ldb = sz; x.strideB = sz * sz; x.trans_b = false;
      x.C = w.Linv + (r0 + sz) * d + r0; x.ldc = d; x.strideC = 2 * sz * (d + 1); x.tri = 0;
      x.k_to_m = 1;  // C⁻¹ is lower triangular: row m needs k <= m only
      if ((e = gemm_f32(x, s)) != hipSuccess) return e;
    }
  }

  write_u_kernel<<<dim3((unsigned)ceil_div(d, 1024), gy), 256, 0, s>>>(w.Linv, d, U);
  GQ_CHECK();
  if (act_order) {
    const int64_t nb64 = ceil_div(d, 64);
    write_hd_kernel<<<(unsigned)(nb64 * (nb64 + 1) / 2), 256, 0, s>>>(H, d, w.G, w.diag, w.perm,
                                                                      w.lam);
  } else {
    add_diag_kernel<<<(unsigned)ceil_div(d, 256), 256, 0, s>>>(H, d, w.lam);
  }
  GQ_CHECK();
#undef GQ_CHECK
  return hipSuccess;
}

}  // namespace gq
