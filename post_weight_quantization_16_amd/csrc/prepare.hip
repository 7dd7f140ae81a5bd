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
  int spin_limit;  // bound on every flag wait (polls)
  int64_t ld;      // row stride of G and Linv
  int piv_base;    // index of G's first column in the whole factorization
};

constexpr int LS = NB + 2;       // LDS row stride: the half-waves' MFMA reads hit disjoint banks
constexpr int PXS = NB + 1;      // stride of the published x rows (strip MFMA reads of 16 rows)
constexpr int BLK = NB * LS;     // one 64x64 block in LDS (floats)
static_assert(4 * BLK + 4 * NB <= gemm_detail::GEMM_SMEM_FLOATS, "panel LDS exceeds the shared buffer");

// row / column of accumulator element e in the 32x32 tile (mi, ni)
__device__ __forceinline__ int acc_row(int mi, int lane, int e) {
  return 32 * mi + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
}

// One 64-wide Cholesky panel at column k0 (kb <= 64 columns), for workgroup
// b of the panel's grid:
//   the previous panel's contribution to this panel's columns,
//     G[:, panel] −= L21ₚ·L21ₚ[panel rows]ᵀ (the trailing updates of the
//     previous launch skip these columns so this launch can run it): the
//     diagonal block's part before the sweep, the workgroup's rows' part
//     (only the L21 solve needs it) by wave 0 after its own steps,
//   L11 = chol(G11),  X = L11⁻¹,  L21 = G21·Xᵀ.
// Every workgroup (4 waves) factors and inverts the small diagonal block
// itself, so no workgroup waits for another; workgroup b then solves the
// 64 rows k0+kb+64b .. +63 of the panel in place in G, and workgroup 0
// stores X into the diagonal block of Linv (L11 itself is not needed
// later).  The block is padded to 64 with the identity.
//
// The factor and the inverse are one right-looking sweep.  Lane i of wave w
// holds A[i][16w..16w+15] (a) and X[16w..16w+15][i] (r).  Wave w owns steps
// 16w..16w+15: step j takes the pivot from lane j, scales column j into
// l_ij = a_ij / l_jj (zeroed for i <= j), finishes x_j = r_j / l_jj,
// applies a_ik −= l_ij·l_kj and r_k −= l_kj·x_j to its next column at once
// (l_kj from lane k by readlane: that column's pivot is next), publishes l
// and x for step j in LDS, updates its remaining columns with l_kj read back
// from the published row, and raises the step's flag.  Before its own
// steps, wave w consumes steps 0 .. 16w−1 four at a time as their flags
// appear, applying the same update to its 16 columns; the last four are
// held in registers and applied to each column just before its pivot, so
// the hand-over from wave w−1 waits for one batch of reads, not for the
// whole batch's arithmetic.  The owner of a step never waits for another
// wave, so the serial chain carries no workgroup barrier; every wait is on a
// step some wave has already begun or will begin without waiting (wave 0
// waits for nothing), and is bounded.  A non-positive (or NaN/inf) pivot is
// recorded in *status (smallest index wins) and replaced by 1 so the
// arithmetic stays finite.
//
// L21's 16-column strips: X's rows 16w..16w+15 are final once wave w's
// steps are done, so wave w (w < 3) solves its strip L21[:, 16w..] =
// G21·X[16w..16w+15, :]ᵀ (v_mfma_f32_16x16x4f32, 64 rows) while the later
// waves are still sweeping, and workgroup 0's wave w stores those X rows to
// Linv from its registers.  The last strip is split over the four waves
// after the sweep.
// L21[16rb.., 16c..16c+15] for row blocks rb in [rb0, rb1) of this
// workgroup's 64 rows: G21 (BS, already reduced by the pre-update) times the
// published X rows 16c..16c+15 (PX), v_mfma_f32_16x16x4f32 (A: lane holds
// (row lane%16, k lane/16), B: (k lane/16, column lane%16), C: rows
// 4·(lane/16) + v, column lane%16), stored to G.
__device__ __forceinline__ void strip(const float* BS, const float* PX, float* G, int64_t d,
                                      int64_t ld, int64_t R0, int k0, int kb, int c, int rb0,
                                      int rb1, int lane) {
  const int m = lane & 15, kq = lane >> 4;
  for (int rb = rb0; rb < rb1; ++rb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k4 = 0; k4 < NB; k4 += 4) {
      const float av = BS[(16 * rb + m) * LS + k4 + kq];
      const float bv = PX[(16 * c + m) * PXS + k4 + kq];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
    }
    const int col = 16 * c + m;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = R0 + 16 * rb + 4 * kq + v;
      if (row < d && col < kb) G[row * ld + k0 + col] = acc[v];
    }
  }
}

// The rows' share of the pre-update, BS −= Q·Pᵀ with Q = the previous
// panel's values in this workgroup's 64 rows and P = its values in the
// panel's rows, by one wave from registers (v_mfma_f32_32x32x2f32; lanes
// 0-31 take k in [0, 32), lanes 32-63 k in [32, 64), so each lane's 32
// values of a row are contiguous).  Rows past d or kb count as zero.
__device__ __forceinline__ void rows_preupdate(const float* G, int64_t d, int64_t ld, int64_t R0,
                                               int k0, int kb, int kp, float* BS, int lane) {
  const int h = lane >> 5, l32 = lane & 31;
  const bool vec = (ld & 3) == 0;
  float qv[2][32], pv[2][32];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int64_t qr = R0 + 32 * x + l32;
    const int pr = 32 * x + l32;
    const bool qok = qr < d, pok = pr < kb;
    const float* qs = G + (qok ? qr : 0) * ld + kp + 32 * h;
    const float* ps = G + (int64_t)(k0 + (pok ? pr : 0)) * ld + kp + 32 * h;
    if (vec) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 q4 = *reinterpret_cast<const f32x4*>(qs + 4 * j);
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(ps + 4 * j);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          qv[x][4 * j + u] = qok ? q4[u] : 0.f;
          pv[x][4 * j + u] = pok ? p4[u] : 0.f;
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) {
        qv[x][kk] = qok ? qs[kk] : 0.f;
        pv[x][kk] = pok ? ps[kk] : 0.f;
      }
    }
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      f32x16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[mi][kk], pv[ni][kk], acc, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 16; ++e) BS[acc_row(mi, lane, e) * LS + 32 * ni + l32] -= acc[e];
    }
}

constexpr int kSpinLimit = 1 << 20;   // default bound on a flag wait (never reached)

__device__ __forceinline__ void panel_body(const PanelArgs& p, int b, float* __restrict__ smem) {
  float* AS = smem;              // G11 (lower, identity-padded)
  float* BS = smem + BLK;        // this workgroup's 64 rows of G21
  float* XS = smem + 2 * BLK;    // before the sweep: the previous panel's rows k0..k0+63
  // during and after the sweep: published l [64][64] in AS's place, x [64][PXS]
  // (= X by rows) in XS's place, flags [65] after it
  float* PL = smem;
  float* PX = smem + 2 * BLK;
  int* flag = reinterpret_cast<int*>(smem + 3 * BLK);
  static_assert(NB * NB <= BLK && NB * PXS <= BLK, "published steps exceed their LDS region");
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t d = p.d, ld = p.ld;
  const int k0 = p.k0, kb = p.kb;
  const int64_t R0 = (int64_t)k0 + kb + (int64_t)b * NB;
  const bool upd = k0 > 0;       // previous panels are full width
  const int kp = k0 - NB;
  float* G = p.G;

  {
    // all loads first, then the masks and the LDS stores (a select right
    // after its load, or a load-store pair per element, would wait for the
    // load at once).  Full-width panels of a 4-aligned G load float4: thread
    // t covers rows (t >> 4) + 16u, columns 4(t & 15) .. +3.
    if ((ld & 3) == 0 && k0 + NB <= d) {
      const int c4 = 4 * (t & 15);
      f32x4 va[4], vb[4], vp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = (t >> 4) + 16 * u;
        const int64_t ra = k0 + (i < kb ? i : 0), rb = R0 + i < d ? R0 + i : 0;
        va[u] = *reinterpret_cast<const f32x4*>(G + ra * ld + k0 + c4);
        vb[u] = *reinterpret_cast<const f32x4*>(G + rb * ld + k0 + c4);
        if (upd) vp[u] = *reinterpret_cast<const f32x4*>(G + ra * ld + kp + c4);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = (t >> 4) + 16 * u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = c4 + e;
          AS[i * LS + k] = (i < kb && k <= i) ? va[u][e] : (i == k ? 1.f : 0.f);
          BS[i * LS + k] = R0 + i < d ? vb[u][e] : 0.f;
          if (upd) XS[i * LS + k] = i < kb ? vp[u][e] : 0.f;
        }
      }
    } else {
      float va[16], vb[16], vp[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int idx = t + 256 * u, i = idx >> 6, k = idx & 63;
        const bool okd = i < kb && k <= i;
        va[u] = G[(int64_t)(k0 + (okd ? i : 0)) * ld + k0 + (okd ? k : 0)];
        const bool okb = R0 + i < d && k < kb;
        vb[u] = G[(okb ? R0 + i : 0) * ld + (okb ? k0 + k : 0)];
        if (upd) vp[u] = G[(int64_t)(k0 + (i < kb ? i : 0)) * ld + kp + k];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int idx = t + 256 * u, i = idx >> 6, k = idx & 63;
        AS[i * LS + k] = (i < kb && k <= i) ? va[u] : (i == k ? 1.f : 0.f);
        BS[i * LS + k] = (R0 + i < d && k < kb) ? vb[u] : 0.f;
        if (upd) XS[i * LS + k] = i < kb ? vp[u] : 0.f;
      }
    }
  }
  __syncthreads();
  // The diagonal block's pre-update, AS −= P·Pᵀ (P = XS, the previous
  // panel's values in this panel's rows), in 16x16 tiles (rb, s): rows
  // 16rb.., columns 16s.., rb >= s (v_mfma_f32_16x16x4f32, A: (row lane%16,
  // k lane/16), B: (k lane/16, column lane%16), C: rows 4·(lane/16) + v,
  // column lane%16).  Column slab 0 is shared out over the four waves so
  // wave 0 can start its steps after one barrier; every later wave updates
  // its own slab afterwards, in the time it waits for the earlier waves'
  // steps.  (What the steps publish overwrites AS and XS from their start,
  // slab 0's rows; the later slabs lie beyond every row published before
  // their wave has read them.)  The rows' pre-update (E) waits for wave 0's
  // idle time after its own steps, as only the L21 strips need it.
  auto pre_tile = [&](int rb, int sl) {
    const int m = lane & 15, kq = lane >> 4;
    // all 32 operands first: left to itself the compiler waits for each
    // pair of reads before its two MFMAs (eight LDS round trips a tile)
    float av[NB / 4], bv[NB / 4];
#pragma unroll
    for (int k = 0; k < NB / 4; ++k) {
      av[k] = XS[(16 * rb + m) * LS + 4 * k + kq];
      bv[k] = XS[(16 * sl + m) * LS + 4 * k + kq];
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NB / 4; ++k)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k], bv[k], acc, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) AS[(16 * rb + 4 * kq + v) * LS + 16 * sl + m] -= acc[v];
  };
  if (upd) pre_tile(w, 0);
  // flags: steps 0..63; at NB "E applied"; at NB+1, NB+2 "slab 1's tile in
  // row block 2 (3) done"
  if (t <= NB + 2) flag[t] = 0;
  __syncthreads();
  int bad_j = -1;
  // after one expired wait a wave stops waiting; status[1] then flags the
  // whole call, whose outputs are undefined
  bool stalled = false;
  if (upd && w > 0) {
    // wave 1 is the first to need its slab and must keep up with wave 0's
    // steps, so waves 2 and 3 take slab 1's tiles in their row blocks first
    // and release them with a flag each; then every wave updates its own slab
    if (w >= 2) {
      pre_tile(w, 1);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __hip_atomic_store(&flag[NB + w - 1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      for (int rb = w; rb < 4; ++rb) pre_tile(rb, w);
    } else {
      pre_tile(1, 1);
      for (int f = NB + 1; f <= NB + 2; ++f) {
        int spin = 0;
        while (!stalled &&
               __hip_atomic_load(&flag[f], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
          if (++spin > p.spin_limit) stalled = true;
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
  }
  float a[16], r[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    a[q] = AS[lane * LS + 16 * w + q];
    r[q] = (16 * w + q == lane) ? 1.f : 0.f;
  }

  // consume the steps of the waves before this one, four at a time: one
  // wait on the fourth step's flag covers all four (one wave publishes them
  // in order, each flag a release of the writes before it); the last four
  // stay pending (pl, px, pc) and meet each column just before its pivot
  float pl[4], px[4];
  f32x4 pc[4][4];
  auto read_batch = [&](int j0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pl[u] = PL[(j0 + u) * NB + lane];
      px[u] = PX[(j0 + u) * PXS + lane];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        pc[u][h] = *reinterpret_cast<const f32x4*>(PL + (j0 + u) * NB + 16 * w + 4 * h);
    }
  };
  for (int j0 = 0; j0 < 16 * w; j0 += 4) {
    // first look: the flag and the batch are read together, without a wait
    // between them (this wave's LDS reads complete in order, so a flag
    // found set vouches for the reads issued after it); only a flag not yet
    // set is waited for and the batch read again
    const int f = __hip_atomic_load(&flag[j0 + 3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    read_batch(j0);
    if (f == 0) {
      int spin = 0;
      while (!stalled &&
             __hip_atomic_load(&flag[j0 + 3], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
        if (++spin > p.spin_limit) stalled = true;
        __builtin_amdgcn_s_sleep(1);
      }
      read_batch(j0);
    }
    if (j0 + 4 < 16 * w) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const float c = pc[u][q >> 2][q & 3];
          a[q] = fmaf(-pl[u], c, a[q]);
          r[q] = fmaf(-c, px[u], r[q]);
        }
    }
  }
  // own steps.  The next pivot is computed from two values read before
  // this step's update, s_a = a[j+1][j] and s_1 = a[j+1][j+1] (every earlier
  // step applied): l[j+1][j] = s_a·inv and the new pivot is fma(−l, l, s_1),
  // the same operations on the same values as lane j+1's own update below,
  // so the value is identical and the serial chain per step is rsq, mul, fma.
  // The steps are instantiated with and without a pending batch, so the
  // unrolled steps carry no branch and the scheduler can move each step's
  // pivot chain ahead of the previous step's remaining updates.
  auto own_steps = [&](auto pend) {
    constexpr bool P = decltype(pend)::value;
    float piv = 0.f;
#pragma unroll
    for (int q0 = 0; q0 < 16; ++q0) {
      const int j = 16 * w + q0;
      // the pending last batch meets column 0 here and column q0 + 1 below,
      // so every column sees it exactly once, before its pivot
      if (q0 == 0) {
        if (P) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float c = pc[u][q0 >> 2][q0 & 3];
            a[q0] = fmaf(-pl[u], c, a[q0]);
            r[q0] = fmaf(-c, px[u], r[q0]);
          }
        }
        piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[q0]), j));
      }
      if (q0 + 1 < 16 && P) {   // the next column, before its pivot entry is read
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float c = pc[u][(q0 + 1) >> 2][(q0 + 1) & 3];
          a[q0 + 1] = fmaf(-pl[u], c, a[q0 + 1]);
          r[q0 + 1] = fmaf(-c, px[u], r[q0 + 1]);
        }
      }
      const bool bad = !(piv > 0.f) || !(piv < INFINITY);
      bad_j = (bad && bad_j < 0) ? j : bad_j;
      // one hardware reciprocal square root on the serial chain (about 1 ulp)
      const float inv = bad ? 1.f : __builtin_amdgcn_rsqf(piv);
      const float l = lane > j ? a[q0] * inv : 0.f;
      const float x = r[q0] * inv;
      r[q0] = x;
      if (q0 + 1 < 16) {   // the next column feeds the next pivot
        const float sa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[q0]), j + 1));
        const float s1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[q0 + 1]), j + 1));
        const float c = sa * inv;   // = l at lane j + 1
        piv = fmaf(-c, c, s1);
        a[q0 + 1] = fmaf(-l, c, a[q0 + 1]);
        r[q0 + 1] = fmaf(-c, x, r[q0 + 1]);
      }
      PL[j * NB + lane] = l;
      PX[j * PXS + lane] = x;
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __hip_atomic_store(&flag[j], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
      for (int q = q0 + 2; q < 16; ++q) {
        const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 16 * w + q));
        a[q] = fmaf(-l, c, a[q]);
        r[q] = fmaf(-c, x, r[q]);
      }
    }
  };
  if (w > 0) own_steps(std::true_type{});
  else own_steps(std::false_type{});
  const bool rows = R0 < d;
  if (upd && rows) {
    if (w == 0) {
      rows_preupdate(G, d, ld, R0, k0, kb, kp, BS, lane);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __hip_atomic_store(&flag[NB], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else if (w < 3) {
      int spin = 0;
      while (!stalled &&
             __hip_atomic_load(&flag[NB], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
        if (++spin > p.spin_limit) stalled = true;
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
  if (b == 0 && lane == 0 && bad_j >= 0) atomicMin(p.status, p.piv_base + k0 + bad_j);
  if (lane == 0 && stalled) atomicOr(p.status + 1, 1);
  if (rows && w < 3) strip(BS, PX, G, d, ld, R0, k0, kb, w, 0, 4, lane);
  __syncthreads();   // the last strip's X rows (published by wave 3) are visible
  if (rows) strip(BS, PX, G, d, ld, R0, k0, kb, 3, w, w + 1, lane);
  // X = L11⁻¹ to Linv's diagonal block, its rows spread over the panel's
  // workgroups and waves (row j by workgroup j % np)
  for (int jr = b + p.np * w; jr < kb; jr += 4 * p.np)
    if (lane < kb) p.Linv[(int64_t)(k0 + jr) * ld + k0 + lane] = PX[jr * PXS + lane];
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
// Far tasks: 128x128 tiles of G −= Lₛ·Lₛᵀ for super-panels s, one packed
// (row tile, column tile, super-panel) word per workgroup.
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

template <int T>
__device__ __forceinline__ void job_tile(const gemm_detail::KArgs& g, bool dma, int bx, int by,
                                         float* smem) {
  constexpr int NS = T == 64 ? kRing64 : kRing128;
  if (dma)
    gemm_detail::gemm_tile_dma<T, NS, false, true>(g, bx, by, 0, 1, reinterpret_cast<char*>(smem));
  else
    gemm_detail::gemm_tile<T, false, true>(g, bx, by, 0, 1, smem);
}

__device__ __forceinline__ void run_near_tile(const TileJob& j, int idx, float* smem) {
  int bx = 0;
  while (idx >= j.nby - bx) { idx -= j.nby - bx; ++bx; }
  if (j.tile == 64) job_tile<64>(j.g, j.dma, bx, bx + idx, smem);
  else job_tile<128>(j.g, j.dma, bx, bx + idx, smem);
}

__device__ __forceinline__ void run_far_tile(const FarJob& f, int idx, float* smem) {
  const uint32_t w = f.task[idx];   // chol_sched::far_word layout
  const int r = (int)(w & 1023u), t = (int)((w >> 10) & 1023u), sp = (int)((w >> 20) & 1023u);
  gemm_detail::KArgs g = f.g;
  g.A += (int64_t)sp * chol_sched::kSW;
  g.B += (int64_t)sp * chol_sched::kSW;
  job_tile<128>(g, f.dma, t, r, smem);
}

// One step of the blocked Cholesky: workgroups [0, nP) run panel k (its
// columns first receive the previous panel's update), the rest run the
// near job's tiles and then the far tasks listed for this launch.  The
// schedule guarantees that they all write disjoint parts of G and read
// only finished panels.  A launch with nP = 0 runs far tasks only.
__global__ __launch_bounds__(256) void chol_step_kernel(PanelArgs p, int nP, TileJob nj,
                                                        FarJob fj) {
  __shared__ __attribute__((aligned(1024))) float smem[gemm_detail::GEMM_SMEM_FLOATS];
  const int L = blockIdx.x;
  if (L < nP) panel_body(p, L, smem);
  else if (L < nP + nj.count) run_near_tile(nj, L - nP, smem);
  else run_far_tile(fj, L - nP - nj.count, smem);
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
  GemmArgs h{};  // tile (r, t): G[128r:, 128t:] −= G[128r:, 128s:+128] · G[128t:, 128s:+128]ᵀ
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
      chol_step_kernel<<<(unsigned)kMaxFar, 256, 0, s>>>(pa, 0, TileJob{}, fj);
      GQ_CHECK();
      done += kMaxFar;
    }
    fj.count = (int)(ft.size() - done);
    std::copy(ft.begin() + (ptrdiff_t)done, ft.end(), fj.task);
    chol_step_kernel<<<(unsigned)(nP + nj.count + fj.count), 256, 0, s>>>(pa, nP, nj, fj);
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
