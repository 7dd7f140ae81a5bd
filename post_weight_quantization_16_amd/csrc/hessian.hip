// H += 2·XᵀX for token-major X [n_tok x d] ("GPTQ: Mathematical Foundations
// ...", Second-Order Taylor Expansion and the Hessian: H = 2XXᵀ with the
// page's X = d x N).
//
// Only the upper-triangle 128x128 tiles are computed (SYRK: d(d+1)N flops).
// The token axis is split S ways; each (tile, split) workgroup writes its
// fp32 partial tile, and a reduction kernel adds 2·Σ_s partial_s into both
// triangles of H in a fixed order (deterministic, exactly symmetric).
//
// bf16/fp16 path: v_mfma_f32_32x32x16_{bf16,f16}; the products are exact in
// fp32 and accumulate in fp32.  The MFMA operand layout wants 8 consecutive
// tokens of one column per lane, while X is contiguous along columns, so each
// thread loads an 8-token x 8-column block (eight 16-byte loads), transposes it
// in registers and stores eight 16-byte column runs into LDS ([col][token]
// layout, rows padded to 72 halves so both the stores and the MFMA operand
// reads are bank-conflict free).
//
// fp32 path: the generic fp32 MFMA GEMM on op(A) = Xᵀ, op(B) = X.
#include "common.hpp"

namespace gq {
namespace {

constexpr int HT = 128;        // output tile
constexpr int HK = 64;         // tokens per LDS stage
constexpr int HLD = HK + 8;    // LDS row stride in 16-bit elements

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ void tile_of(int idx, int nt, int& ti, int& tj) {
  int r = 0;
  while (idx >= nt - r) { idx -= nt - r; ++r; }
  ti = r;
  tj = r + idx;
}

// 8x8 transpose of 16-bit values: in[r] holds columns 0..7 of token row r;
// out[c] holds token rows 0..7 of column c.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {      // column pair (2p, 2p+1) lives in dword p
#pragma unroll
    for (int q = 0; q < 4; ++q) {    // token pair (2q, 2q+1)
      const uint32_t x = in[2 * q][p], y = in[2 * q + 1][p];
      out[2 * p][q] = (x & 0xFFFFu) | (y << 16);
      out[2 * p + 1][q] = (x >> 16) | (y & 0xFFFF0000u);
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void syrk16_kernel(const uint16_t* __restrict__ X, int64_t ld,
                                                     int d, int64_t n_tok, int64_t chunk, int nt,
                                                     float* __restrict__ P, int64_t dp, int vec) {
  int ti, tj;
  tile_of(blockIdx.x, nt, ti, tj);
  const int split = blockIdx.y;
  const int64_t t_begin = (int64_t)split * chunk;
  const int64_t t_end = min(n_tok, t_begin + chunk);

  __shared__ __attribute__((aligned(16))) uint16_t S[2][HT * HLD];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  // loader role: operand 0 -> column block ti, operand 1 -> column block tj
  const int op = t >> 7, u = t & 127;
  const int blk_t = u & 7, blk_c = u >> 3;
  const int col = (op ? tj : ti) * HT + blk_c * 8;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 rin[8];
  auto gload = [&](int64_t t0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t tok = t0 + blk_t * 8 + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (tok < t_end) {
        const uint16_t* p = X + tok * ld + col;
        if (vec && col + 7 < d) {
          v = *reinterpret_cast<const u32x4*>(p);
        } else {
          uint16_t e[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) e[c] = (col + c < d) ? p[c] : (uint16_t)0;
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = (uint32_t)e[2 * c] | ((uint32_t)e[2 * c + 1] << 16);
        }
      }
      rin[r] = v;
    }
  };
  auto lstore = [&]() {
    u32x4 o[8];
    transpose8x8(rin, o);
    uint16_t* base = &S[op][0];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *reinterpret_cast<u32x4*>(base + (blk_c * 8 + c) * HLD + blk_t * 8) = o[c];
  };

  gload(t_begin);
  lstore();
  __syncthreads();
  for (int64_t t0 = t_begin; t0 < t_end; t0 += HK) {
    const bool more = t0 + HK < t_end;
    if (more) gload(t0 + HK);
#pragma unroll
    for (int ks = 0; ks < HK / 16; ++ks) {
      const int koff = ks * 16 + (lane >> 5) * 8;
      if constexpr (BF16) {
        bf16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a[i] = *reinterpret_cast<const bf16x8*>(&S[0][(wm * 64 + i * 32 + (lane & 31)) * HLD + koff]);
          b[i] = *reinterpret_cast<const bf16x8*>(&S[1][(wn * 64 + i * 32 + (lane & 31)) * HLD + koff]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      } else {
        f16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a[i] = *reinterpret_cast<const f16x8*>(&S[0][(wm * 64 + i * 32 + (lane & 31)) * HLD + koff]);
          b[i] = *reinterpret_cast<const f16x8*>(&S[1][(wn * 64 + i * 32 + (lane & 31)) * HLD + koff]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
    if (more) {
      lstore();
      __syncthreads();
    }
  }

  float* Pt = P + (int64_t)split * dp * dp;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = ti * HT + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int cl = tj * HT + wn * 64 + j * 32 + (lane & 31);
        Pt[(int64_t)row * dp + cl] = acc[i][j][r];
      }
}

// H[i][j] += 2·Σ_s P_s[i][j] for i <= j, mirrored to H[j][i].
__global__ __launch_bounds__(256) void syrk_reduce_kernel(float* __restrict__ H, int d,
                                                          const float* __restrict__ P, int64_t dp,
                                                          int splits, int nt) {
  int ti, tj;
  tile_of(blockIdx.x, nt, ti, tj);
  for (int e = threadIdx.x; e < HT * HT; e += 256) {
    const int a = e / HT, b = e % HT;
    if (ti == tj && a > b) continue;
    const int i = ti * HT + a, j = tj * HT + b;
    if (i >= d || j >= d) continue;
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += P[(int64_t)s * dp * dp + (int64_t)i * dp + j];
    v *= 2.f;
    H[(int64_t)i * d + j] += v;
    if (i != j) H[(int64_t)j * d + i] += v;
  }
}

}  // namespace

int hessian_splits(int64_t d, int64_t n_tok) {
  const int64_t nt = ceil_div(d, HT);
  const int64_t tiles = nt * (nt + 1) / 2;
  int64_t s = ceil_div(2048, tiles);
  s = std::min<int64_t>(s, 32);
  s = std::min<int64_t>(s, std::max<int64_t>(1, ceil_div(n_tok, 256)));
  s = std::max<int64_t>(s, 1);
  const int64_t chunk = ceil_div(ceil_div(std::max<int64_t>(n_tok, 1), s), HK) * HK;
  return (int)ceil_div(std::max<int64_t>(n_tok, 1), chunk);
}

size_t hessian_ws_bytes(int64_t d, int64_t n_tok) {
  const int64_t dp = ceil_div(d, HT) * HT;
  return align_up((size_t)hessian_splits(d, n_tok) * dp * dp * sizeof(float));
}

hipError_t hessian_launch(float* H, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                          int64_t ld_x, void* ws, hipStream_t s) {
  if (n_tok <= 0) return hipSuccess;
  const int nt = (int)ceil_div(d, HT);
  const int64_t dp = (int64_t)nt * HT;
  const int tiles = nt * (nt + 1) / 2;
  const int splits = hessian_splits(d, n_tok);
  const int64_t chunk = ceil_div(ceil_div(n_tok, splits), HK) * HK;
  float* P = static_cast<float*>(ws);
  if (x_dtype == GPTQ_F32) {
    GemmArgs g{};
    g.M = (int)d; g.N = (int)d;
    g.K = (int)chunk; g.k_last = (int)(n_tok - (int64_t)(splits - 1) * chunk);
    g.batch = splits; g.alpha = 1.f; g.beta = 0.f;
    g.A = static_cast<const float*>(X); g.lda = ld_x; g.strideA = chunk * ld_x; g.trans_a = true;
    g.B = static_cast<const float*>(X); g.ldb = ld_x; g.strideB = chunk * ld_x; g.trans_b = false;
    g.C = P; g.ldc = dp; g.strideC = dp * dp; g.tri = 2;
    hipError_t e = gemm_f32(g, s);
    if (e != hipSuccess) return e;
  } else {
    const int vec = ((uintptr_t)X % 16 == 0) && (ld_x % 8 == 0);
    dim3 grid(tiles, splits);
    if (x_dtype == GPTQ_BF16)
      syrk16_kernel<true><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(X), ld_x, (int)d, n_tok,
                                               chunk, nt, P, dp, vec);
    else
      syrk16_kernel<false><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(X), ld_x, (int)d, n_tok,
                                                chunk, nt, P, dp, vec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  syrk_reduce_kernel<<<tiles, 256, 0, s>>>(H, (int)d, P, dp, splits, nt);
  return hipGetLastError();
}

}  // namespace gq
