// fp32 MFMA GEMM for gfx950: the lazy block update of the GPTQ sweep and the
// trailing updates of the blocked Cholesky / triangular inverse.
//
// Tile 128x128 per workgroup of 256 threads (4 waves in a 2x2 grid, each wave
// 64x64 = 2x2 tiles of v_mfma_f32_32x32x2f32).  K advances in chunks of 16
// staged through LDS in [k][m] / [k][n] layout, so each MFMA operand is one
// float per lane read from 32 consecutive LDS words.  The next chunk is
// fetched into registers while the current one is multiplied.
#include "common.hpp"

namespace gq {
namespace {

constexpr int TM = 128, TN = 128, TK = 16;
constexpr int LDS_STRIDE = TM + 32;  // row k+1 lands 32 banks after row k

struct KArgs {
  int M, N, K, k_last;
  int k_from_n, k_to_m;
  float alpha, beta;
  const float* A; int64_t lda, strideA;
  const float* B; int64_t ldb, strideB;
  float* C; int64_t ldc, strideC;
  int tri;
  int vec_a, vec_b;
};

// Loads of one 16 x 128 operand chunk into registers (2 float4 per thread).
// "along" = the 128-wide dimension is contiguous in memory; otherwise k is.
template <bool ALONG>
__device__ __forceinline__ void load_chunk(const float* __restrict__ p, int64_t ld, int rows_valid,
                                           int k0, int kvalid, int t, bool vec, f32x4 (&r)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = t + 256 * i;
    int a, b;  // a: index along the 128-wide dim, b: k
    if (ALONG) { b = idx >> 5; a = (idx & 31) * 4; }
    else       { a = idx >> 2; b = (idx & 3) * 4; }
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (ALONG) {
      const int kk = k0 + b;
      if (kk < kvalid) {
        const float* q = p + (int64_t)kk * ld + a;
        if (vec && a + 3 < rows_valid) {
          v = *reinterpret_cast<const f32x4*>(q);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (a + j < rows_valid) ? q[j] : 0.f;
        }
      }
    } else {
      if (a < rows_valid) {
        const float* q = p + (int64_t)a * ld + k0 + b;
        if (vec && k0 + b + 3 < kvalid) {
          v = *reinterpret_cast<const f32x4*>(q);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (k0 + b + j < kvalid) ? q[j] : 0.f;
        }
      }
    }
    r[i] = v;
  }
}

template <bool ALONG>
__device__ __forceinline__ void store_chunk(float* __restrict__ s, int t, const f32x4 (&r)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = t + 256 * i;
    if (ALONG) {
      const int b = idx >> 5, a = (idx & 31) * 4;
      *reinterpret_cast<f32x4*>(s + b * LDS_STRIDE + a) = r[i];
    } else {
      const int a = idx >> 2, b = (idx & 3) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) s[(b + j) * LDS_STRIDE + a] = r[i][j];
    }
  }
}

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f32_kernel(KArgs g) {
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  if (g.tri == 1 && n0 > m0 + TM - 1) return;
  if (g.tri == 2 && n0 + TN - 1 < m0) return;
  const int z = blockIdx.z;
  const int Kz = (z == (int)gridDim.z - 1) ? g.k_last : g.K;
  const int kbeg = g.k_from_n ? (n0 / TK) * TK : 0;
  const int K = g.k_to_m ? min(Kz, m0 + TM) : Kz;
  const float* A = g.A + (int64_t)z * g.strideA;
  const float* B = g.B + (int64_t)z * g.strideB;
  float* C = g.C + (int64_t)z * g.strideC;

  __shared__ float As[TK * LDS_STRIDE];
  __shared__ float Bs[TK * LDS_STRIDE];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;

  // operand base pointers at the tile origin
  // A: op(A)(m,k). TA: stored [K x M] (m contiguous) -> ALONG; else [M x K].
  const float* Ab = TA ? A + m0 : A + (int64_t)m0 * g.lda;
  const float* Bb = TB ? B + (int64_t)n0 * g.ldb : B + n0;
  const int mvalid = g.M - m0, nvalid = g.N - n0;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  f32x4 ra[2], rb[2];
  load_chunk<TA>(Ab, g.lda, mvalid, kbeg, K, t, g.vec_a, ra);
  load_chunk<!TB>(Bb, g.ldb, nvalid, kbeg, K, t, g.vec_b, rb);
  store_chunk<TA>(As, t, ra);
  store_chunk<!TB>(Bs, t, rb);
  __syncthreads();

  for (int k0 = kbeg; k0 < K; k0 += TK) {
    const bool more = k0 + TK < K;
    if (more) {
      load_chunk<TA>(Ab, g.lda, mvalid, k0 + TK, K, t, g.vec_a, ra);
      load_chunk<!TB>(Bb, g.ldb, nvalid, k0 + TK, K, t, g.vec_b, rb);
    }
#pragma unroll
    for (int kk = 0; kk < TK / 2; ++kk) {
      const int ka = kk * 2 + (lane >> 5);
      const float a0 = As[ka * LDS_STRIDE + wm * 64 + (lane & 31)];
      const float a1 = As[ka * LDS_STRIDE + wm * 64 + 32 + (lane & 31)];
      const float b0 = Bs[ka * LDS_STRIDE + wn * 64 + (lane & 31)];
      const float b1 = Bs[ka * LDS_STRIDE + wn * 64 + 32 + (lane & 31)];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      store_chunk<TA>(As, t, ra);
      store_chunk<!TB>(Bs, t, rb);
      __syncthreads();
    }
  }

  // epilogue: lane holds rows (r/4)*8 + (lane/32)*4 + r%4, column lane%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row >= g.M || col >= g.N) continue;
        if (g.tri == 1 && col > row) continue;
        if (g.tri == 2 && col < row) continue;
        float* c = C + (int64_t)row * g.ldc + col;
        float v = g.alpha * acc[i][j][r];
        if (g.beta != 0.f) v += g.beta * *c;
        *c = v;
      }
}

}  // namespace

hipError_t gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  KArgs k;
  k.M = a.M; k.N = a.N; k.K = a.K; k.k_last = a.k_last;
  k.k_from_n = a.k_from_n; k.k_to_m = a.k_to_m;
  k.alpha = a.alpha; k.beta = a.beta;
  k.A = a.A; k.lda = a.lda; k.strideA = a.strideA;
  k.B = a.B; k.ldb = a.ldb; k.strideB = a.strideB;
  k.C = a.C; k.ldc = a.ldc; k.strideC = a.strideC;
  k.tri = a.tri;
  auto aligned = [](const float* p, int64_t ld, int64_t st) {
    return ((uintptr_t)p % 16 == 0) && (ld % 4 == 0) && (st % 4 == 0);
  };
  k.vec_a = aligned(a.A, a.lda, a.strideA);
  k.vec_b = aligned(a.B, a.ldb, a.strideB);
  dim3 grid((unsigned)ceil_div(a.N, TN), (unsigned)ceil_div(a.M, TM), (unsigned)a.batch);
  if (!a.trans_a && !a.trans_b) gemm_f32_kernel<false, false><<<grid, 256, 0, s>>>(k);
  else if (!a.trans_a && a.trans_b) gemm_f32_kernel<false, true><<<grid, 256, 0, s>>>(k);
  else if (a.trans_a && !a.trans_b) gemm_f32_kernel<true, false><<<grid, 256, 0, s>>>(k);
  else gemm_f32_kernel<true, true><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

}  // namespace gq
