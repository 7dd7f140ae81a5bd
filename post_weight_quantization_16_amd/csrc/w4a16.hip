// Inference with the exported weights: Y = A·Ŵᵀ for 16-bit activations A
// [M x K] and b-bit weights [N x K] in the dense export layout ("GPTQ:
// Mathematical Foundations ...", Inference Execution and Modern Kernel
// Architectures: the FP16xINT4 pipeline -- load packed codes, dequantize in
// registers as W = (W_int − zero)·scale, multiply, accumulate in FP32).
//
// The dequantized weight is (q − z)·s with the 16-bit scale and zero of the
// export, exact in fp32, rounded once to the activations' format (fp16 or
// bf16); products are exact in fp32 and accumulate in fp32.
//
// Codes are read in 32-code chunks: 32 codes of b bits are b whole 32-bit
// words of a row's stream (b = 2, 3, 4, 8), and every group size the
// quantizer runs is a multiple of 32 (or the whole row), so a chunk has one
// (scale, zero) unless a g_idx permutes the groups.
//   gemv_kernel  (M <= 8): HBM-bound on the weights.  A wave takes 4 weight
//                rows; lane l walks chunks l, l+64, ... of each, so a wave's
//                loads of one row are contiguous; dot products in fp32 on the
//                VALU, reduced across the wave.
//   gemm_kernel  (M > 8): 64x128 output tiles; each K step of 32 stages the
//                A tile and the dequantized W tile in LDS as 16-bit values and
//                runs v_mfma_f32_32x32x16_{f16,bf16}.
#include <utility>

#include "common.hpp"

namespace gq {
namespace {

struct WArgs {
  const uint16_t* A; int64_t M, K, lda;
  const uint32_t* q; int bits; int64_t row_words;
  const uint16_t* s16; const uint16_t* z16; int64_t ng; int64_t g;
  const int32_t* g_idx;
  int64_t N; float* C; int64_t ldc;
};

__device__ __forceinline__ float half_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
template <bool F16>
__device__ __forceinline__ float act_to_f32(uint16_t b) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, b);
  else return __uint_as_float((uint32_t)b << 16);
}
// x (exact in fp32) rounded to the activation format, as an fp32 value
template <bool F16>
__device__ __forceinline__ float round_act(float x) {
  if constexpr (F16) return (float)(_Float16)x;
  else {
    const uint32_t u = __float_as_uint(x);
    return __uint_as_float(((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16) << 16);
  }
}
template <bool F16>
__device__ __forceinline__ uint16_t round_act_bits(float x) {
  if constexpr (F16) return __builtin_bit_cast(uint16_t, (_Float16)x);
  else {
    const uint32_t u = __float_as_uint(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  }
}

// The 32 codes of chunk c of a row: BITS words (those beyond the row's end
// read as 0).  BITS and the code index are compile-time constants, so the
// words stay in registers.
template <int BITS>
__device__ __forceinline__ void load_chunk(const uint32_t* __restrict__ row, int64_t row_words,
                                           int64_t c, uint32_t (&w)[BITS]) {
  const int64_t w0 = c * BITS;
  if (w0 + BITS <= row_words) {
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = row[w0 + i];
  } else {
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = w0 + i < row_words ? row[w0 + i] : 0u;
  }
}
template <int BITS, int J>
__device__ __forceinline__ uint32_t code_of(const uint32_t (&w)[BITS]) {
  constexpr int p = J * BITS, wi = p >> 5, sh = p & 31;
  uint64_t v = w[wi];
  if constexpr (wi + 1 < BITS) v |= (uint64_t)w[wi + 1] << 32;
  return (uint32_t)(v >> sh) & ((1u << BITS) - 1u);
}
template <int BITS, int J0, int... Js>
__device__ __forceinline__ void codes8(const uint32_t (&w)[BITS], float (&out)[8],
                                       std::integer_sequence<int, Js...>) {
  ((out[Js] = (float)code_of<BITS, J0 + Js>(w)), ...);
}

// Ŵ values of codes [8·J8, 8·J8 + 8) of a chunk at column k0 of row n
// (the chunk's own scale and zero, or per column through g_idx)
template <bool F16, int BITS, int J8>
__device__ __forceinline__ void dequant8(const WArgs& a, const uint32_t (&w)[BITS], int64_t n,
                                         int64_t k0, float s, float z, float (&out)[8]) {
  codes8<BITS, 8 * J8>(w, out, std::make_integer_sequence<int, 8>{});
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float sj = s, zj = z;
    if (a.g_idx) {
      const int64_t k = k0 + 8 * J8 + j < a.K ? k0 + 8 * J8 + j : a.K - 1;
      const int64_t gi = a.g_idx[k];
      sj = half_bits_to_f32(a.s16[n * a.ng + gi]);
      zj = half_bits_to_f32(a.z16[n * a.ng + gi]);
    }
    out[j] = round_act<F16>((out[j] - zj) * sj);
  }
}

// GEMV: the workgroup stages A [MM x K] in LDS (16-bit, zero past M); every
// wave takes rows n = wave, wave + waves, ...; lane l takes the row's chunks
// l, l + 64, ...; the next row's chunk words are loaded before the current
// row's arithmetic.
constexpr int kGemvLds = 64 * 1024;    // bytes of A staged per workgroup
template <bool F16, int BITS, int MM, bool GIDX>
__global__ __launch_bounds__(256) void gemv_kernel(WArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t As[];
  const int t = threadIdx.x, lane = t & 63;
  const int64_t Kp = (a.K + 31) / 32 * 32;   // A rows padded to whole chunks
  for (int64_t e = t; e < MM * Kp; e += 256) {
    const int64_t m = e / Kp, k = e % Kp;
    As[e] = (m < a.M && k < a.K) ? a.A[m * a.lda + k] : (uint16_t)0;
  }
  __syncthreads();
  const int64_t nch = Kp / 32;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (t >> 6), nwaves = (int64_t)gridDim.x * 4;
  // chunks per lane (K <= 64·32·CPL)
  constexpr int CPL = 32;
  for (int64_t n = wave; n < a.N; n += nwaves) {
    float acc[MM];
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[m] = 0.f;
    const uint32_t* row = a.q + n * a.row_words;
    for (int64_t c = lane; c < nch; c += 64) {
      const int64_t k0 = c * 32;
      uint32_t w[BITS];
      load_chunk<BITS>(row, a.row_words, c, w);
      float s = 0.f, z = 0.f;
      if (!GIDX) {
        const int64_t gi = k0 / a.g;
        s = half_bits_to_f32(a.s16[n * a.ng + gi]);
        z = half_bits_to_f32(a.z16[n * a.ng + gi]);
      }
      float wv[4][8];
      dequant8<F16, BITS, 0>(a, w, n, k0, s, z, wv[0]);
      dequant8<F16, BITS, 1>(a, w, n, k0, s, z, wv[1]);
      dequant8<F16, BITS, 2>(a, w, n, k0, s, z, wv[2]);
      dequant8<F16, BITS, 3>(a, w, n, k0, s, z, wv[3]);
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        const uint16_t* ar = As + m * Kp + k0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = *reinterpret_cast<const uint4*>(ar + 8 * q);
          const uint32_t h4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc[m] = fmaf(act_to_f32<F16>((uint16_t)(h4[j >> 1] >> (16 * (j & 1)))), wv[q][j], acc[m]);
        }
      }
    }
    (void)CPL;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      float v = acc[m];
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0 && m < a.M) a.C[m * a.ldc + n] = v;
    }
  }
}

constexpr int BM = 64, BN = 128, BK = 32, LK = BK + 8;   // LDS row: 32 values + pad (16-bit)

template <bool F16, int BITS>
__global__ __launch_bounds__(256) void gemm_kernel(WArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LK];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[BN * LK];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;   // wave tile: rows 32·wm, columns 64·wn (two 32x32)
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const int64_t nch = (a.K + 31) / 32;
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t k0 = c * BK;
    // A tile: 64 rows x 32 values, 8 per thread
    {
      const int rr = t >> 2, kk = (t & 3) * 8;
      const int64_t m = m0 + rr;
      uint16_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = (m < a.M && k0 + kk + j < a.K) ? a.A[m * a.lda + k0 + kk + j] : (uint16_t)0;
#pragma unroll
      for (int j = 0; j < 8; ++j) As[rr * LK + kk + j] = v[j];
    }
    // W tile: 128 rows, one 32-code chunk each (threads 0..127), dequantized
    if (t < BN) {
      const int64_t n = n0 + t < a.N ? n0 + t : a.N - 1;   // rows past N: never stored
      uint32_t w[BITS];
      load_chunk<BITS>(a.q + n * a.row_words, a.row_words, c, w);
      float s = 0.f, z = 0.f;
      if (!a.g_idx) {
        const int64_t gi = k0 / a.g;
        s = half_bits_to_f32(a.s16[n * a.ng + gi]);
        z = half_bits_to_f32(a.z16[n * a.ng + gi]);
      }
      float v[4][8];
      dequant8<F16, BITS, 0>(a, w, n, k0, s, z, v[0]);
      dequant8<F16, BITS, 1>(a, w, n, k0, s, z, v[1]);
      dequant8<F16, BITS, 2>(a, w, n, k0, s, z, v[2]);
      dequant8<F16, BITS, 3>(a, w, n, k0, s, z, v[3]);
#pragma unroll
      for (int j = 0; j < 32; ++j)   // the value is exact in the format: reinterpret its bits
        Ws[t * LK + j] = k0 + j < a.K ? round_act_bits<F16>(v[j >> 3][j & 7]) : (uint16_t)0;
    }
    __syncthreads();
    // two k-steps of 16: lane holds 8 consecutive k of row / column lane % 32
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kk = ks * 16 + (lane >> 5) * 8;
      typedef __attribute__((ext_vector_type(8))) short s16x8;
      const s16x8 av = *reinterpret_cast<const s16x8*>(&As[(wm * 32 + (lane & 31)) * LK + kk]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const s16x8 bv = *reinterpret_cast<const s16x8*>(&Ws[(wn * 64 + j * 32 + (lane & 31)) * LK + kk]);
        if constexpr (F16)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                          __builtin_bit_cast(f16x8, bv), acc[j], 0, 0, 0);
        else
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                           __builtin_bit_cast(bf16x8, bv), acc[j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (m < a.M && n < a.N) a.C[m * a.ldc + n] = acc[j][r];
    }
}

}  // namespace

hipError_t w4a16_launch(const void* A, int a_dtype, int64_t M, int64_t K, int64_t lda,
                        const uint32_t* qweight, int bits, const uint16_t* s16, const uint16_t* z16,
                        const int32_t* g_idx, int64_t g, int64_t ng, int64_t N, float* C,
                        int64_t ldc, hipStream_t s) {
  WArgs a{static_cast<const uint16_t*>(A), M, K, lda, qweight, bits, ceil_div(K * bits, 32),
          s16, z16, ng, g, g_idx, N, C, ldc};
  const bool f16 = a_dtype == GPTQ_F16;
  const int mm = M <= 1 ? 1 : M <= 2 ? 2 : 4;
  const int64_t Kp = ceil_div(K, 32) * 32;
  if (M <= 4 && (int64_t)mm * Kp * 2 <= kGemvLds) {
    const unsigned grid = (unsigned)std::min<int64_t>(ceil_div(N, 4), 2048);
    const size_t lds = (size_t)mm * Kp * 2;
    const bool gx = g_idx != nullptr;
#define GQ_GEMV(F, B, MM, GX) gemv_kernel<F, B, MM, GX><<<grid, 256, lds, s>>>(a)
#define GQ_GEMV_G(F, B, MM) \
  if (gx) GQ_GEMV(F, B, MM, true); else GQ_GEMV(F, B, MM, false);
#define GQ_GEMV_M(F, B)                          \
  switch (mm) {                                  \
    case 1: GQ_GEMV_G(F, B, 1); break;           \
    case 2: GQ_GEMV_G(F, B, 2); break;           \
    default: GQ_GEMV_G(F, B, 4); break;          \
  }
#define GQ_GEMV_B(F)                             \
  switch (bits) {                                \
    case 2: GQ_GEMV_M(F, 2); break;              \
    case 3: GQ_GEMV_M(F, 3); break;              \
    case 4: GQ_GEMV_M(F, 4); break;              \
    default: GQ_GEMV_M(F, 8); break;             \
  }
    if (f16) { GQ_GEMV_B(true) } else { GQ_GEMV_B(false) }
#undef GQ_GEMV_B
#undef GQ_GEMV_M
#undef GQ_GEMV_G
#undef GQ_GEMV
  } else {
    const dim3 grid((unsigned)ceil_div(N, BN), (unsigned)ceil_div(M, BM));
#define GQ_GEMM(F)                                                         \
  switch (bits) {                                                          \
    case 2: gemm_kernel<F, 2><<<grid, 256, 0, s>>>(a); break;              \
    case 3: gemm_kernel<F, 3><<<grid, 256, 0, s>>>(a); break;              \
    case 4: gemm_kernel<F, 4><<<grid, 256, 0, s>>>(a); break;              \
    default: gemm_kernel<F, 8><<<grid, 256, 0, s>>>(a); break;             \
  }
    if (f16) { GQ_GEMM(true) } else { GQ_GEMM(false) }
#undef GQ_GEMM
  }
  return hipGetLastError();
}

}  // namespace gq
