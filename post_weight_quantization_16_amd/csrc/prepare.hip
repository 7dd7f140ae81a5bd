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
// (each diagonal block factored and inverted together in one wave, the
// panel below solved with that inverse and the trailing SYRK, both on the
// fp32 MFMA GEMM), then the rest of the triangular inverse by recursive
// doubling ([[A,0],[B,C]]⁻¹ has off-diagonal block −C⁻¹·B·A⁻¹, products
// skipping the zero triangles).
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

// One Cholesky panel's diagonal block: L11 = chol(G11) and X = L11⁻¹ in a
// single right-looking sweep (one wave; the block is padded to 64 with the
// identity).  Lane i holds row i of the block being factored (a) and column i
// of the inverse being built (r).  Step j: the pivot is lane j's a[j];
// every lane scales its a[j] into l_ij and publishes it through LDS; then
// a[k] −= l_ij·l_kj (the trailing rank-1 update) and, for the inverse,
// x_j = r[j]/l_jj followed by r[k] −= l_kj·x_j (forward substitution
// carried along the same column of L).  Only X is stored, into the diagonal
// block of Linv: the rows below are then L21 = G21·Xᵀ, one GEMM, and the
// doubling inverse needs X, not L11.  A non-positive (or NaN/inf) pivot is
// recorded in *status (smallest index wins) and replaced by 1 so the
// arithmetic stays finite.
__global__ __launch_bounds__(64) void potrf_inv_kernel(const float* __restrict__ G, int64_t d,
                                                       int k0, int kb, float* __restrict__ Linv,
                                                       int* __restrict__ status) {
  __shared__ float col[2][NB];      // column j of L, double-buffered by step parity
  __shared__ float XS[NB][NB + 1];  // X staged row-major for a coalesced write
  const int i = threadIdx.x;
  float a[NB], r[NB];
  const float* grow = G + (int64_t)(k0 + i) * d + k0;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    float v = (i == k) ? 1.f : 0.f;
    if (i < kb && k < kb && k <= i) v = grow[k];
    a[k] = v;
    r[k] = (i == k) ? 1.f : 0.f;
  }
  int bad_j = -1;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const float piv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a[j]), j));
    const bool bad = !(piv > 0.f) || !(piv < INFINITY);
    bad_j = (bad && bad_j < 0) ? j : bad_j;
    const float ljj = bad ? 1.f : sqrtf(piv);
    const float inv = 1.f / ljj;
    const float l = (i > j) ? a[j] * inv : (i == j ? ljj : 0.f);
    a[j] = l;
    const float x = r[j] * inv;
    r[j] = x;
    col[j & 1][i] = l;
    __syncthreads();
#pragma unroll
    for (int k = j + 1; k < NB; ++k) {
      const float ck = col[j & 1][k];
      a[k] = fmaf(-l, ck, a[k]);
      r[k] = fmaf(-ck, x, r[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < NB; ++k) XS[k][i] = r[k];
  __syncthreads();
  if (i == 0 && bad_j >= 0) atomicMin(status, k0 + bad_j);
  for (int e = i; e < kb * kb; e += NB) {
    const int rr = e / kb, c = e % kb;
    Linv[(int64_t)(k0 + rr) * d + k0 + c] = XS[rr][c];
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

  // blocked right-looking Cholesky of G (lower), 64-wide panels: the
  // diagonal block's factor and inverse X in one workgroup, the rows below
  // as L21 = G21·Xᵀ and the trailing SYRK, both on the fp32 MFMA GEMM
  for (int64_t k0 = 0; k0 < d; k0 += NB) {
    const int kb = (int)std::min<int64_t>(NB, d - k0);
    const int64_t r0 = k0 + kb, nr = d - r0;
    potrf_inv_kernel<<<1, NB, 0, s>>>(w.G, d, (int)k0, kb, w.Linv, w.status);
    GQ_CHECK();
    if (nr <= 0) break;
    GemmArgs p{};  // L21 = G21 · Xᵀ, in place: one column of output tiles
    p.M = (int)nr; p.N = kb; p.K = kb; p.k_last = kb; p.batch = 1;  // (N <= 128), so each
    p.alpha = 1.f; p.beta = 0.f;                                      // workgroup reads all
    p.A = w.G + r0 * d + k0; p.lda = d; p.trans_a = false;           // of its rows before
    p.B = w.Linv + k0 * d + k0; p.ldb = d; p.trans_b = true;          // writing them
    p.C = w.G + r0 * d + k0; p.ldc = d; p.tri = 0;
    if ((e = gemm_f32(p, s)) != hipSuccess) return e;
    GemmArgs h{};  // G22 −= L21 · L21ᵀ  (lower triangle)
    h.M = (int)nr; h.N = (int)nr; h.K = kb; h.k_last = kb; h.batch = 1;
    h.alpha = -1.f; h.beta = 1.f;
    h.A = w.G + r0 * d + k0; h.lda = d; h.trans_a = false;
    h.B = w.G + r0 * d + k0; h.ldb = d; h.trans_b = true;
    h.C = w.G + r0 * d + r0; h.ldc = d; h.tri = 1;
    if ((e = gemm_f32(h, s)) != hipSuccess) return e;
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
