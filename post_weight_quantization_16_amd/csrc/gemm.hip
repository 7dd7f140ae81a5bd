// fp32 MFMA GEMM for gfx950: the lazy block updates of the GPTQ sweep and the
// products of the triangular inverse (the tile itself is in gemm_tile.hpp).
#include "gemm_dma.hpp"

namespace gq {
namespace gemm_detail {
namespace {

// blockIdx.x enumerates the nx x ny tiles.  Workgroups start in index
// order, so the order is longest-first where tiles differ in K: column-major
// from the left when column n starts its K loop at n (k_from_n), row-major
// from the bottom when row m stops at m (k_to_m), row-major otherwise.
template <int T, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f32_kernel(KArgs g, int nx, int ny) {
  __shared__ __attribute__((aligned(16))) float Sm[4 * Tile<T>::OPF];
  const int L = blockIdx.x;
  int bx, by;
  if (g.k_from_n) { bx = L / ny; by = L % ny; }
  else if (g.k_to_m) { by = ny - 1 - L / nx; bx = L % nx; }
  else { by = L / nx; bx = L % nx; }
  gemm_tile<T, TA, TB>(g, bx, by, blockIdx.z, gridDim.z, Sm);
}

// Ring depth of the DMA tile: four 16-KB stages for T = 128 (two
// workgroups per CU), six 8-KB stages for T = 64 (three per CU).
template <int T> constexpr int kRing = T == 128 ? 4 : 6;

template <int T, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_dma_kernel(KArgs g, int nx, int ny) {
  __shared__ __attribute__((aligned(1024))) char Sm[DTile<T, kRing<T>>::SMEM];
  const int L = blockIdx.x;
  int bx, by;
  if (g.k_from_n) { bx = L / ny; by = L % ny; }
  else if (g.k_to_m) { by = ny - 1 - L / nx; bx = L % nx; }
  else { by = L / nx; bx = L % nx; }
  gemm_tile_dma<T, kRing<T>, TA, TB>(g, bx, by, blockIdx.z, gridDim.z, Sm);
}

template <int T>
void launch(const KArgs& k, const GemmArgs& a, hipStream_t s) {
  const int nx = (int)ceil_div(a.N, T), ny = (int)ceil_div(a.M, T);
  dim3 grid((unsigned)(nx * ny), 1, (unsigned)a.batch);
  if (dma_ok(k, a.trans_a, a.trans_b)) {
    if (!a.trans_a && !a.trans_b) gemm_dma_kernel<T, false, false><<<grid, 256, 0, s>>>(k, nx, ny);
    else if (!a.trans_a && a.trans_b) gemm_dma_kernel<T, false, true><<<grid, 256, 0, s>>>(k, nx, ny);
    else if (a.trans_a && !a.trans_b) gemm_dma_kernel<T, true, false><<<grid, 256, 0, s>>>(k, nx, ny);
    else gemm_dma_kernel<T, true, true><<<grid, 256, 0, s>>>(k, nx, ny);
    return;
  }
  if (!a.trans_a && !a.trans_b) gemm_f32_kernel<T, false, false><<<grid, 256, 0, s>>>(k, nx, ny);
  else if (!a.trans_a && a.trans_b) gemm_f32_kernel<T, false, true><<<grid, 256, 0, s>>>(k, nx, ny);
  else if (a.trans_a && !a.trans_b) gemm_f32_kernel<T, true, false><<<grid, 256, 0, s>>>(k, nx, ny);
  else gemm_f32_kernel<T, true, true><<<grid, 256, 0, s>>>(k, nx, ny);
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
  // 128-tiles unless they would leave most CUs without a second workgroup
  // or the K loop is long (the triangular products' tiles then differ a lot
  // in length, and small tiles spread the long ones over more CUs)
  const int64_t tiles128 = ceil_div(a.M, 128) * ceil_div(a.N, 128) * a.batch;
  const bool small = tiles128 < 512 || ((a.k_from_n || a.k_to_m) && a.K >= 1024);
  if (small) launch<64>(k, a, s);
  else launch<128>(k, a, s);
  return hipGetLastError();
}

}  // namespace gq
