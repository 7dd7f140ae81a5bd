// fp32 MFMA GEMM for gfx950: the lazy block update of the GPTQ sweep and the
// trailing updates of the triangular inverse (the tile itself is in
// gemm_tile.hpp).
#include "gemm_tile.hpp"

namespace gq {
namespace gemm_detail {
namespace {

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f32_kernel(KArgs g) {
  __shared__ __attribute__((aligned(16))) float Sm[GEMM_SMEM_FLOATS];
  gemm_tile<TA, TB>(g, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.z, Sm);
}

}  // namespace

KArgs make_kargs(const GemmArgs& a) {
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
  k.vec_c = aligned(a.C, a.ldc, a.strideC);
  return k;
}

}  // namespace gemm_detail

hipError_t gemm_f32(const GemmArgs& a, hipStream_t s) {
  using namespace gemm_detail;
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  const KArgs k = make_kargs(a);
  dim3 grid((unsigned)ceil_div(a.N, TN), (unsigned)ceil_div(a.M, TM), (unsigned)a.batch);
  if (!a.trans_a && !a.trans_b) gemm_f32_kernel<false, false><<<grid, 256, 0, s>>>(k);
  else if (!a.trans_a && a.trans_b) gemm_f32_kernel<false, true><<<grid, 256, 0, s>>>(k);
  else if (a.trans_a && !a.trans_b) gemm_f32_kernel<true, false><<<grid, 256, 0, s>>>(k);
  else gemm_f32_kernel<true, true><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

}  // namespace gq
