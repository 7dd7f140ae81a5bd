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
// workgroups per CU), eight 8-KB stages for T = 64 (two per CU: the deeper
// ring hides more of the load latency than a third workgroup did).
template <int T> constexpr int kRing = T == 128 ? 4 : 8;

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

// Triangular products (k_from_n: tile column bx runs K − bx·T of K; k_to_m:
// tile row by runs (by+1)·T): workgroup L takes a tile and its mirror image
// (bx and nx−1−bx, or by and ny−1−by) one after the other, so every
// workgroup runs about K + T, and the launch is one even round instead of a
// few long tiles that finish last (at d = 4096 the top level's two products
// 115 -> 102 us each, the next level's 53 -> 40 us).
template <int T, bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_dma_pair_kernel(KArgs g, int nx, int ny) {
  __shared__ __attribute__((aligned(1024))) char Sm[DTile<T, kRing<T>>::SMEM];
  const int L = blockIdx.x;
  int bx, by, bx2, by2;
  if (g.k_from_n) { bx = L / ny; by = L % ny; bx2 = nx - 1 - bx; by2 = by; }
  else { by = L / nx; bx = L % nx; bx2 = bx; by2 = ny - 1 - by; }
  gemm_tile_dma<T, kRing<T>, TA, TB>(g, bx, by, blockIdx.z, gridDim.z, Sm);
  if (bx2 == bx && by2 == by) return;
  __syncthreads();   // the first tile's epilogue has read its LDS before the ring refills
  gemm_tile_dma<T, kRing<T>, TA, TB>(g, bx2, by2, blockIdx.z, gridDim.z, Sm);
}

// Rectangular products whose 128-tiles fill whole rounds of the chip but
// one: the last round's tiles run as four 64-tiles each (same launch, after
// the 128-tiles), so that round takes about a quarter of a 128-tile's time
// instead of a full one.  WG L < full: 128-tile L in row-major order; then
// the remaining 128-tile positions, four 64-tile workgroups each.
constexpr int kMixRing64 = 8;
constexpr int kMixSmem = DTile<128, 4>::SMEM > DTile<64, kMixRing64>::SMEM
                             ? DTile<128, 4>::SMEM : DTile<64, kMixRing64>::SMEM;
template <bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_mixed_kernel(KArgs g, int nx, int full) {
  __shared__ __attribute__((aligned(1024))) char Sm[kMixSmem];
  const int L = blockIdx.x;
  if (L < full) {
    gemm_tile_dma<128, 4, TA, TB>(g, L % nx, L / nx, 0, 1, Sm);
  } else {
    const int j = L - full, q = full + j / 4, sub = j & 3;
    gemm_tile_dma<64, kMixRing64, TA, TB>(g, 2 * (q % nx) + (sub & 1), 2 * (q / nx) + (sub >> 1),
                                          0, 1, Sm);
  }
}

// 128-tile workgroups resident at once (two per CU)
constexpr int64_t kSlots128 = 2 * 256;

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
  const bool rect = a.batch == 1 && !a.k_from_n && !a.k_to_m && a.tri == 0;
  if (rect && tiles128 > kSlots128 && tiles128 % kSlots128 != 0 &&
      dma_ok(k, a.trans_a, a.trans_b)) {
    const int nx = (int)ceil_div(a.N, 128);
    const int64_t full = tiles128 / kSlots128 * kSlots128;
    const unsigned grid = (unsigned)(full + 4 * (tiles128 - full));
    if (!a.trans_a && !a.trans_b) gemm_mixed_kernel<false, false><<<grid, 256, 0, s>>>(k, nx, (int)full);
    else if (!a.trans_a && a.trans_b) gemm_mixed_kernel<false, true><<<grid, 256, 0, s>>>(k, nx, (int)full);
    else if (a.trans_a && !a.trans_b) gemm_mixed_kernel<true, false><<<grid, 256, 0, s>>>(k, nx, (int)full);
    else gemm_mixed_kernel<true, true><<<grid, 256, 0, s>>>(k, nx, (int)full);
    return hipGetLastError();
  }
  // paired triangular tiles once the 64-tiles fill the chip's workgroup
  // slots (two per CU); with fewer, the single tiles all run side by side
  const int64_t tiles64 = ceil_div(a.M, 64) * ceil_div(a.N, 64) * a.batch;
  if ((a.k_from_n || a.k_to_m) && tiles64 >= kSlots128 && dma_ok(k, a.trans_a, a.trans_b)) {
    const int nx = (int)ceil_div(a.N, 64), ny = (int)ceil_div(a.M, 64);
    const int gx = a.k_from_n ? (nx + 1) / 2 * ny : (ny + 1) / 2 * nx;
    dim3 grid((unsigned)gx, 1, (unsigned)a.batch);
    if (!a.trans_a && !a.trans_b) gemm_dma_pair_kernel<64, false, false><<<grid, 256, 0, s>>>(k, nx, ny);
    else if (!a.trans_a && a.trans_b) gemm_dma_pair_kernel<64, false, true><<<grid, 256, 0, s>>>(k, nx, ny);
    else if (a.trans_a && !a.trans_b) gemm_dma_pair_kernel<64, true, false><<<grid, 256, 0, s>>>(k, nx, ny);
    else gemm_dma_pair_kernel<64, true, true><<<grid, 256, 0, s>>>(k, nx, ny);
    return hipGetLastError();
  }
  const bool small = tiles128 < kSlots128 || ((a.k_from_n || a.k_to_m) && a.K >= 1024);
  if (small) launch<64>(k, a, s);
  else launch<128>(k, a, s);
  return hipGetLastError();
}

}  // namespace gq
