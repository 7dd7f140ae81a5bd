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
// solved with that inverse; one launch per panel that also runs the previous
// panel's trailing update on fp32 MFMA GEMM tiles), then the rest of the
// triangular inverse by recursive
// doubling ([[A,0],[B,C]]⁻¹ has off-diagonal block −C⁻¹·B·A⁻¹, products
// skipping the zero triangles).
#include <algorithm>
#include <climits>

#include "common.hpp"
#include "gemm_tile.hpp"

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
    status[0] = INT_MAX;
  }
}

// Rank sort: position of i = #{j : key_j > key_i or (key_j == key_i and j < i)}.
__global__ __launch_bounds__(256) void rank_kernel(const float* __restrict__ diag, int d,
                                                   int act_order, int* __restrict__ perm) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (!act_order) {
    if (i < d) perm[i] = i;
    return;
  }
  __shared__ float kj[256];
  float ki = -INFINITY;
  if (i < d) { ki = diag[i]; if (ki != ki) ki = -INFINITY; }
  int rank = 0;
  for (int j0 = 0; j0 < d; j0 += 256) {
    __syncthreads();
    const int j = j0 + threadIdx.x;
    float v = -INFINITY;
    if (j < d) { v = diag[j]; if (v != v) v = -INFINITY; }
    kj[threadIdx.x] = v;
    __syncthreads();
    const int n = min(256, d - j0);
    for (int k = 0; k < n; ++k) {
      const float v2 = kj[k];
      rank += (v2 > ki) || (v2 == ki && j0 + k < i);
    }
  }
  if (i < d) perm[rank] = i;
}

// G[a][b] = H[π(d-1-a)][π(d-1-b)] + λ·[a == b]   (reversed, permuted, damped)
__global__ __launch_bounds__(256) void build_g_kernel(const float* __restrict__ H, int64_t d,
                                                      const int* __restrict__ perm,
                                                      const float* __restrict__ lam,
                                                      float* __restrict__ G) {
  const float l = lam[0];
  for (int64_t a = blockIdx.y; a < d; a += gridDim.y) {
    const int pa = perm[d - 1 - a];
    for (int64_t b = blockIdx.x * 256 + threadIdx.x; b < d; b += (int64_t)gridDim.x * 256) {
      float v = H[(int64_t)pa * d + perm[d - 1 - b]];
      if (a == b) v += l;
      G[a * d + b] = v;
    }
  }
}

struct PanelArgs {
  float* G; int64_t d; int k0, kb;
  float* Linv; int* status;
};

constexpr int LS = NB + 2;       // LDS row stride: the half-waves' MFMA reads hit disjoint banks
constexpr int BLK = NB * LS;     // one 64x64 block in LDS (floats)
static_assert(4 * BLK + 4 * NB <= gemm_detail::GEMM_SMEM_FLOATS, "panel LDS exceeds the shared buffer");

// acc += S1 · S2ᵀ for one 32x32 tile (rows 32mi.., columns 32ni..) of two
// 64x64 LDS blocks; v_mfma_f32_32x32x2f32 takes A(m = lane%32, k = lane/32),
// B(k, n = lane%32), so both operands are read along their rows
__device__ __forceinline__ void mfma_abt(const float* S1, const float* S2, int mi, int ni,
                                         int lane, f32x16& acc) {
#pragma unroll
  for (int kk = 0; kk < NB / 2; ++kk) {
    const int k = 2 * kk + (lane >> 5);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(S1[(32 * mi + (lane & 31)) * LS + k],
                                               S2[(32 * ni + (lane & 31)) * LS + k], acc, 0, 0, 0);
  }
}
// row / column of accumulator element e in the 32x32 tile (mi, ni)
__device__ __forceinline__ int acc_row(int mi, int lane, int e) {
  return 32 * mi + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
}

// One 64-wide Cholesky panel at column k0 (kb <= 64 columns), for workgroup
// b of the panel's grid:
//   first, the previous panel's contribution to this panel's columns,
//     G[:, panel] −= L21ₚ·L21ₚ[panel rows]ᵀ (the trailing update of the
//     previous step skips these columns so this launch can run it),
//   L11 = chol(G11),  X = L11⁻¹,  L21 = G21·Xᵀ.
// Every workgroup (4 waves) factors and inverts the small diagonal block
// itself, so no workgroup waits for another; workgroup b then solves the
// 64 rows k0+kb+64b .. +63 of the panel with one 64x64x64 fp32 MFMA product,
// in place in G, and workgroup 0 stores X into the diagonal block of Linv
// (L11 itself is not needed later).  The block is padded to 64 with the
// identity.
//
// The factor and the inverse are one right-looking sweep.  Lane i of wave w
// holds A[i][16w..16w+15] (a) and X[16w..16w+15][i] (r).  Wave w owns steps
// 16w..16w+15: step j takes the pivot from lane j, scales column j into
// l_ij = a_ij / l_jj (zeroed for i <= j), finishes x_j = r_j / l_jj, applies
// a_ik −= l_ij·l_kj and r_k −= l_kj·x_j to its own later columns (l_kj read
// from lane k with readlane) and publishes l and x for step j in LDS with a
// flag.  Before its own steps, wave w consumes steps 0 .. 16w−1 as their
// flags appear, applying the same update to its 16 columns.  The owner of a
// step never waits for another wave, so the serial chain carries no
// workgroup barrier; every wait is on a step some wave has already begun or
// will begin without waiting (wave 0 waits for nothing), and is bounded.
// A non-positive (or NaN/inf) pivot is recorded in *status (smallest index
// wins) and replaced by 1 so the arithmetic stays finite.
constexpr int kSpinLimit = 1 << 20;   // safety bound on a flag wait (never reached)

__device__ __forceinline__ void panel_body(const PanelArgs& p, int b, float* __restrict__ smem) {
  float* AS = smem;              // G11 (lower, identity-padded)
  float* BS = smem + BLK;        // this workgroup's 64 rows of G21
  float* XS = smem + 2 * BLK;    // X; before the sweep: the previous panel's rows k0..k0+63
  float* QS = smem + 3 * BLK;    // the previous panel's values in this workgroup's rows
  // during the sweep XS and QS hold the published steps: l [64][64], x [64][64], flags [64]
  float* PL = smem + 2 * BLK;
  float* PX = PL + NB * NB;
  int* flag = reinterpret_cast<int*>(PX + NB * NB);
  static_assert(2 * NB * NB + NB <= 2 * BLK, "published steps exceed their LDS region");
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t d = p.d;
  const int k0 = p.k0, kb = p.kb;
  const int64_t R0 = (int64_t)k0 + kb + (int64_t)b * NB;
  const bool upd = k0 > 0;       // previous panels are full width
  const int kp = k0 - NB;
  float* G = p.G;

  {
    // all loads first, then the LDS stores (a load-store pair per element
    // would wait a memory round trip each)
    float va[16], vb[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int idx = t + 256 * u, i = idx >> 6, k = idx & 63;
      const bool okd = i < kb && k <= i;
      va[u] = G[(int64_t)(k0 + (okd ? i : 0)) * d + k0 + (okd ? k : 0)];
      va[u] = okd ? va[u] : (i == k ? 1.f : 0.f);
      const bool okb = R0 + i < d && k < kb;
      vb[u] = G[(okb ? R0 + i : 0) * d + (okb ? k0 + k : 0)];
      vb[u] = okb ? vb[u] : 0.f;
    }
    if (upd) {
      float vp[16], vq[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int idx = t + 256 * u, i = idx >> 6, k = idx & 63;
        const bool okp = i < kb;
        vp[u] = G[(int64_t)(k0 + (okp ? i : 0)) * d + kp + k];
        vp[u] = okp ? vp[u] : 0.f;
        const bool okq = R0 + i < d;
        vq[u] = G[(okq ? R0 + i : 0) * d + kp + k];
        vq[u] = okq ? vq[u] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int idx = t + 256 * u, i = idx >> 6, k = idx & 63;
        XS[i * LS + k] = vp[u];
        QS[i * LS + k] = vq[u];
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int idx = t + 256 * u, i = idx >> 6, k = idx & 63;
      AS[i * LS + k] = va[u];
      BS[i * LS + k] = vb[u];
    }
  }
  __syncthreads();
  const int mi = w >> 1, ni = w & 1;
  if (upd) {
    f32x16 dacc, eacc;
#pragma unroll
    for (int e = 0; e < 16; ++e) { dacc[e] = 0.f; eacc[e] = 0.f; }
    mfma_abt(XS, XS, mi, ni, lane, dacc);
    mfma_abt(QS, XS, mi, ni, lane, eacc);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int o = acc_row(mi, lane, e) * LS + 32 * ni + (lane & 31);
      AS[o] -= dacc[e];
      BS[o] -= eacc[e];
    }
  }
  __syncthreads();
  float a[16], r[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    a[q] = AS[lane * LS + 16 * w + q];
    r[q] = (16 * w + q == lane) ? 1.f : 0.f;
  }
  if (t < NB) flag[t] = 0;
  __syncthreads();

  // consume the steps of the waves before this one, four at a time: one
  // wait on the fourth step's flag covers all four (one wave publishes them
  // in order, each flag a release of the writes before it)
  int bad_j = -1;
  bool stalled = false;   // after one expired wait, stop waiting (the result is flagged bad)
  for (int j0 = 0; j0 < 16 * w; j0 += 4) {
    int spin = 0;
    while (!stalled &&
           __hip_atomic_load(&flag[j0 + 3], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
      if (++spin > kSpinLimit) {
        stalled = true;
        bad_j = (bad_j < 0) ? j0 : bad_j;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    float li[4], xv[4];
    f32x4 cv[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      li[u] = PL[(j0 + u) * NB + lane];
      xv[u] = PX[(j0 + u) * NB + lane];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        cv[u][h] = *reinterpret_cast<const f32x4*>(PL + (j0 + u) * NB + 16 * w + 4 * h);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float c = cv[u][q >> 2][q & 3];
        a[q] = fmaf(-li[u], c, a[q]);
        r[q] = fmaf(-c, xv[u], r[q]);
      }
  }
  // own steps: the next column's update first (it feeds the next pivot),
  // then the publication, the remaining columns, and the step's flag
#pragma unroll
  for (int q0 = 0; q0 < 16; ++q0) {
    const int j = 16 * w + q0;
    const float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[q0]), j));
    const bool bad = !(piv > 0.f) || !(piv < INFINITY);
    bad_j = (bad && bad_j < 0) ? j : bad_j;
    // one hardware reciprocal square root on the serial chain (about 1 ulp)
    const float inv = bad ? 1.f : __builtin_amdgcn_rsqf(piv);
    const float l = lane > j ? a[q0] * inv : 0.f;
    const float x = r[q0] * inv;
    r[q0] = x;
    if (q0 + 1 < 16) {
      const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), j + 1));
      a[q0 + 1] = fmaf(-l, c, a[q0 + 1]);
      r[q0 + 1] = fmaf(-c, x, r[q0 + 1]);
    }
    PL[j * NB + lane] = l;
    PX[j * NB + lane] = x;
#pragma unroll
    for (int q = q0 + 2; q < 16; ++q) {
      const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 16 * w + q));
      a[q] = fmaf(-l, c, a[q]);
      r[q] = fmaf(-c, x, r[q]);
    }
    __hip_atomic_store(&flag[j], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 16; ++q) XS[(16 * w + q) * LS + lane] = r[q];
  __syncthreads();
  if (b == 0 && lane == 0 && bad_j >= 0) atomicMin(p.status, k0 + bad_j);
  if (b == 0) {
    for (int e = t; e < kb * kb; e += 256) {
      const int rr = e / kb, c = e % kb;
      p.Linv[(int64_t)(k0 + rr) * d + k0 + c] = XS[rr * LS + c];
    }
  }
  if (R0 >= d) return;
  // L21 block = G21 block · Xᵀ, wave w the 32x32 tile (w/2, w%2)
  f32x16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  mfma_abt(BS, XS, mi, ni, lane, acc);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = acc_row(mi, lane, e), col = 32 * ni + (lane & 31);
    if (R0 + row < d && col < kb) G[(R0 + row) * d + k0 + col] = acc[e];
  }
}

// Lower-triangular tile enumeration: L -> (row by, column bx <= by).
__device__ __forceinline__ void lower_tile(int L, int& by, int& bx) {
  int y = (int)((sqrtf(8.f * (float)L + 1.f) - 1.f) * 0.5f);
  while ((y + 1) * (y + 2) / 2 <= L) ++y;
  while (y * (y + 1) / 2 > L) --y;
  by = y;
  bx = L - y * (y + 1) / 2;
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

// One step of the blocked Cholesky: workgroups [0, nP) run panel k (its
// columns first receive the previous panel's update), the rest run the
// previous panel's trailing update of the columns beyond panel k,
// G22 −= L21ₚ·L21ₚᵀ (lower tiles only, fp32 MFMA GEMM tiles).  The two sets
// touch disjoint parts of G: the panel reads the previous panel's columns
// and writes its own, the update writes only columns right of the panel.
__global__ __launch_bounds__(256) void chol_step_kernel(PanelArgs p, int nP,
                                                        gemm_detail::KArgs tr) {
  __shared__ __attribute__((aligned(16))) float smem[gemm_detail::GEMM_SMEM_FLOATS];
  const int L = blockIdx.x;
  if (L < nP) {
    panel_body(p, L, smem);
  } else {
    int by, bx;
    lower_tile(L - nP, by, bx);
    gemm_detail::gemm_tile<128, false, true>(tr, bx, by, 0, 1, smem);
  }
}

// U[a][b] = Linv[d-1-a][d-1-b] for b >= a, 0 below the diagonal.
__global__ __launch_bounds__(256) void write_u_kernel(const float* __restrict__ Linv, int64_t d,
                                                      float* __restrict__ U) {
  for (int64_t a = blockIdx.y; a < d; a += gridDim.y)
    for (int64_t b = blockIdx.x * 256 + threadIdx.x; b < d; b += (int64_t)gridDim.x * 256)
      U[a * d + b] = (b >= a) ? Linv[(d - 1 - a) * d + (d - 1 - b)] : 0.f;
}

// Linv starts as zeros: the doubling products read whole diagonal blocks,
// whose strict upper parts must be zero.
__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

struct PrepWs {
  int* status; float* lam; float* diag; int* perm; float* G; float* Linv; float* T;
};

PrepWs carve(void* ws, int64_t d) {
  char* p = static_cast<char*>(ws);
  PrepWs w;
  w.status = reinterpret_cast<int*>(p); p += 256;
  w.lam = reinterpret_cast<float*>(p); p += 256;
  w.diag = reinterpret_cast<float*>(p); p += align_up((size_t)d * 4);
  w.perm = reinterpret_cast<int*>(p); p += align_up((size_t)d * 4);
  w.G = reinterpret_cast<float*>(p); p += align_up((size_t)d * d * 4);
  w.Linv = reinterpret_cast<float*>(p); p += align_up((size_t)d * d * 4);
  w.T = reinterpret_cast<float*>(p);
  return w;
}

}  // namespace

size_t prepare_ws_bytes(int64_t d) {
  return 512 + 2 * align_up((size_t)d * 4) + 2 * align_up((size_t)d * d * 4) +
         align_up((size_t)(d * d / 2 + NB * NB) * 4);
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
  rank_kernel<<<(unsigned)ceil_div(d, 256), 256, 0, s>>>(w.diag, (int)d, act_order, w.perm);
  GQ_CHECK();
  const unsigned gx = (unsigned)std::min<int64_t>(ceil_div(d, 256), 16);
  const unsigned gy = (unsigned)std::min<int64_t>(d, 65535);
  build_g_kernel<<<dim3(gx, gy), 256, 0, s>>>(H, d, w.perm, w.lam, w.G);
  GQ_CHECK();
  zero_kernel<<<(unsigned)std::min<int64_t>(ceil_div(d * d, 256), 8192), 256, 0, s>>>(w.Linv, d * d);
  GQ_CHECK();

  // blocked right-looking Cholesky of G (lower), 64-wide panels, one launch
  // per panel: the panel itself and, beside it, the previous panel's
  // trailing update of the columns beyond it
  for (int64_t k0 = 0; k0 < d; k0 += NB) {
    const int kb = (int)std::min<int64_t>(NB, d - k0);
    const int64_t r0 = k0 + kb, nr = d - r0;
    const int nP = (int)std::max<int64_t>(1, ceil_div(nr, NB));
    PanelArgs pa{w.G, d, (int)k0, kb, w.Linv, w.status};
    gemm_detail::KArgs tr{};
    int64_t nT = 0;
    if (k0 > 0 && nr > 0) {
      GemmArgs h{};  // G[r0:, r0:] −= L21ₚ · L21ₚᵀ  (lower triangle)
      h.M = (int)nr; h.N = (int)nr; h.K = NB; h.k_last = NB; h.batch = 1;
      h.alpha = -1.f; h.beta = 1.f;
      h.A = w.G + r0 * d + (k0 - NB); h.lda = d; h.trans_a = false;
      h.B = w.G + r0 * d + (k0 - NB); h.ldb = d; h.trans_b = true;
      h.C = w.G + r0 * d + r0; h.ldc = d; h.tri = 1;
      tr = gemm_detail::make_kargs(h);
      const int64_t nb = ceil_div(nr, 128);
      nT = nb * (nb + 1) / 2;
    }
    chol_step_kernel<<<(unsigned)(nP + nT), 256, 0, s>>>(pa, nP, tr);
    GQ_CHECK();
  }

  // triangular inverse by recursive doubling on 64-aligned blocks
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

  write_u_kernel<<<dim3(gx, gy), 256, 0, s>>>(w.Linv, d, U);
  GQ_CHECK();
  {
    const int64_t nb64 = ceil_div(d, 64);
    write_hd_kernel<<<(unsigned)(nb64 * (nb64 + 1) / 2), 256, 0, s>>>(H, d, w.G, w.diag, w.perm,
                                                                      w.lam);
  }
  GQ_CHECK();
  if (perm_out) {
    e = hipMemcpyAsync(perm_out, w.perm, (size_t)d * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
#undef GQ_CHECK
  return hipSuccess;
}

}  // namespace gq
