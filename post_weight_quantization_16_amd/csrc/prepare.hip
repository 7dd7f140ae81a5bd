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
// steps: a blocked right-looking Cholesky (64-wide panels factored in
// registers, trailing SYRK on the fp32 MFMA GEMM) and a triangular inverse:
// all 64x64 diagonal blocks inverted at once, then recursive doubling
// ([[A,0],[B,C]]⁻¹ has off-diagonal block −C⁻¹·B·A⁻¹, products skipping the
// zero triangles), both fp32.
#include <algorithm>
#include <climits>

#include "common.hpp"

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

// H_out[x][y] = H_d[x][y] rebuilt from G's untouched strict upper triangle.
__global__ __launch_bounds__(256) void write_hd_kernel(float* __restrict__ H, int64_t d,
                                                       const float* __restrict__ G,
                                                       const float* __restrict__ diag,
                                                       const int* __restrict__ perm,
                                                       const float* __restrict__ lam) {
  for (int64_t x = blockIdx.y; x < d; x += gridDim.y) {
    for (int64_t y = blockIdx.x * 256 + threadIdx.x; y < d; y += (int64_t)gridDim.x * 256) {
      float v;
      if (x == y) v = diag[perm[x]] + lam[0];
      else if (x > y) v = G[(d - 1 - x) * d + (d - 1 - y)];
      else v = G[(d - 1 - y) * d + (d - 1 - x)];
      H[x * d + y] = v;
    }
  }
}

// One Cholesky panel: factor the kb x kb diagonal block at k0 (kb <= 64) and
// solve the rows below it, L21 = G21·L11⁻ᵀ.  One wave per workgroup; every
// workgroup factors the small diagonal block itself (row i in lane i's
// registers, left-looking: step j finishes column j from row j of L, which
// is broadcast from LDS; pivots via readlane), so no
// workgroup waits for another.  G's diagonal block is only read here (other
// workgroups of the same launch read it), so workgroup 0 writes L11 to the
// diagonal block of Linv instead, where trtri_diag_kernel inverts it in place;
// workgroup b solves rows k0+kb+64b .. +63 by forward substitution in registers.
// The block is padded to 64 with the identity.  A non-positive (or NaN/inf)
// pivot is recorded in *status (smallest index wins) and replaced by 1 so the
// arithmetic stays finite.  Results leave the unrolled register arrays through
// LDS (unconditional stores) and reach memory in a bounds-checked loop: stores
// predicated inside the unrolled code would push the arrays into scratch.
__global__ __launch_bounds__(64) void potrf_trsm_kernel(float* __restrict__ G, int64_t d, int k0,
                                                        int kb, float* __restrict__ Ldiag,
                                                        int* __restrict__ status) {
  __shared__ float LM[NB][NB + 4];  // LM[i][j] = L[i][j]
  __shared__ float LT[NB][NB + 4];  // LT[j][k] = L[k][j]
  __shared__ float XO[NB][NB + 1];  // solved rows, one per lane
  const int i = threadIdx.x;
  float a[NB];
  const float* grow = G + (int64_t)(k0 + i) * d + k0;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    float v = (i == k) ? 1.f : 0.f;
    if (i < kb && k < kb && k <= i) v = grow[k];
    a[k] = v;
  }
  // left-looking: step j finishes column j; row j of L (final since step j-1)
  // is read from LM with wave-uniform loads
  int bad_j = -1;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    __syncthreads();
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int t = 0; t < j; ++t) {
      if (t & 1) s1 = fmaf(a[t], LM[j][t], s1);
      else s0 = fmaf(a[t], LM[j][t], s0);
    }
    const float v = a[j] - (s0 + s1);
    const float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
    const bool bad = !(piv > 0.f) || !(piv < INFINITY);
    if (bad && bad_j < 0) bad_j = j;
    const float ljj = bad ? 1.f : sqrtf(piv);
    a[j] = (i > j) ? v / ljj : (i == j ? ljj : 0.f);
    LM[i][j] = a[j];
    LT[j][i] = a[j];
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    if (i == 0 && bad_j >= 0) atomicMin(status, k0 + bad_j);
    for (int e = i; e < kb * kb; e += NB) {
      const int r = e / kb, c = e % kb;
      if (c <= r) Ldiag[(int64_t)(k0 + r) * d + k0 + c] = LT[c][r];
    }
  }
  const int64_t rbase = (int64_t)k0 + kb + (int64_t)blockIdx.x * NB;
  const int64_t r = rbase + i;
  const float* row = G + r * d + k0;
  float g[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) g[k] = (r < d && k < kb) ? row[k] : 0.f;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const float x = g[j] / LT[j][j];
    g[j] = x;
#pragma unroll
    for (int k = j + 1; k < NB; ++k) g[k] = fmaf(-x, LT[j][k], g[k]);
  }
#pragma unroll
  for (int k = 0; k < NB; ++k) XO[i][k] = g[k];
  __syncthreads();
  const int nrows = (int)min<int64_t>(NB, d - rbase);
  for (int e = i; e < nrows * kb; e += NB) {
    const int rr = e / kb, c = e % kb;
    G[(rbase + rr) * d + k0 + c] = XO[rr][c];
  }
}

// Inverses of all 64x64 diagonal blocks of the factor L, in place in Linv
// (where the panel kernel left the factored blocks).  One wave per block;
// lane c computes column c of L_bb⁻¹ by forward substitution
// (x_i = ([i == c] − Σ_{t<i} L_it x_t) / L_ii), reading the block's rows from
// LDS with wave-uniform loads; the result goes back through LDS.
__global__ __launch_bounds__(64) void trtri_diag_kernel(int64_t d, float* __restrict__ Linv) {
  __shared__ float L[NB][NB + 4];
  const int64_t b0 = (int64_t)blockIdx.x * NB;
  const int kb = (int)min<int64_t>(NB, d - b0);
  const int c = threadIdx.x;
  for (int t = 0; t < NB; ++t) {
    float v = (c == t) ? 1.f : 0.f;
    if (c < kb && t < kb && t <= c) v = Linv[(b0 + c) * d + b0 + t];
    L[c][t] = v;
  }
  __syncthreads();
  float x[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    float sacc = 0.f;
#pragma unroll
    for (int t = 0; t < i; ++t) sacc = fmaf(L[i][t], x[t], sacc);
    x[i] = ((i == c ? 1.f : 0.f) - sacc) / L[i][i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NB; ++i) L[i][c] = (i >= c) ? x[i] : 0.f;
  __syncthreads();
  for (int e = c; e < kb * kb; e += NB) {
    const int i = e / kb, cc = e % kb;
    Linv[(b0 + i) * d + b0 + cc] = L[i][cc];
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

  // blocked right-looking Cholesky of G (lower): per panel, one fused
  // factor+solve launch and one trailing SYRK on the fp32 MFMA GEMM
  for (int64_t k0 = 0; k0 < d; k0 += NB) {
    const int kb = (int)std::min<int64_t>(NB, d - k0);
    const int64_t r0 = k0 + kb, nr = d - r0;
    const unsigned nblk = (unsigned)std::max<int64_t>(1, ceil_div(nr, NB));
    potrf_trsm_kernel<<<nblk, NB, 0, s>>>(w.G, d, (int)k0, kb, w.Linv, w.status);
    GQ_CHECK();
    if (nr <= 0) break;
    GemmArgs h{};  // G22 −= L21 · L21ᵀ  (lower triangle)
    h.M = (int)nr; h.N = (int)nr; h.K = kb; h.k_last = kb; h.batch = 1;
    h.alpha = -1.f; h.beta = 1.f;
    h.A = w.G + r0 * d + k0; h.lda = d; h.trans_a = false;
    h.B = w.G + r0 * d + k0; h.ldb = d; h.trans_b = true;
    h.C = w.G + r0 * d + r0; h.ldc = d; h.tri = 1;
    if ((e = gemm_f32(h, s)) != hipSuccess) return e;
  }
  trtri_diag_kernel<<<(unsigned)ceil_div(d, NB), NB, 0, s>>>(d, w.Linv);
  GQ_CHECK();

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
  write_hd_kernel<<<dim3(gx, gy), 256, 0, s>>>(H, d, w.G, w.diag, w.perm, w.lam);
  GQ_CHECK();
  if (perm_out) {
    e = hipMemcpyAsync(perm_out, w.perm, (size_t)d * 4, hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return e;
  }
#undef GQ_CHECK
  return hipSuccess;
}

}  // namespace gq
