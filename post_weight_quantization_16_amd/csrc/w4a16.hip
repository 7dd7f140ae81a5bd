// Inference with the exported weights: Y = A·Ŵᵀ for 16-bit activations A
// [M x K] and b-bit weights [N x K] in the dense export layout ("GPTQ:
// Mathematical Foundations ...", Inference Execution and Modern Kernel
// Architectures: the FP16xINT4 pipeline -- load packed codes, dequantize in
// registers as W = (W_int − zero)·scale, multiply, accumulate in FP32).
//
// The dequantized weight is (q − z)·s with the 16-bit scale and zero of the
// export, exact in fp32 (formed as fma(q, s, −z·s): q·s and z·s have at most
// 19 significant bits), rounded once to the activations' format (fp16 or
// bf16, round to nearest even, two values per v_cvt_pk); products are exact
// in fp32 and accumulate in fp32.
//
// Codes are read in 32-code chunks: 32 codes of b bits are b whole 32-bit
// words of a row's stream (b = 2, 3, 4, 8), and every group size the
// quantizer runs is a multiple of 32 (or the whole row), so a chunk has one
// (scale, zero) unless a g_idx permutes the groups.
// With fp16 activations and 4-bit codes the dequantization runs on packed
// halves: (0x6400 | code) is the half 1024 + code, so one and-or yields the
// pair (code j, code j+4) of a word, one v_pk_add_f16 subtracts 1024 + z
// (exact) and one v_pk_mul_f16 multiplies by the half scale, rounding once:
// the same value as the fp32 route.  The activations are then paired the
// same way ((a_j, a_j+4) inside each group of 8), which leaves every dot
// product and MFMA sum unchanged.
//   gemv_kernel  (M <= 4): bound by the weights' HBM traffic and the
//                dequantization.  A sits in LDS as packed 16-bit pairs,
//                staged once per workgroup (at most four per CU) while the
//                first weight words are in flight; a wave takes 2 weight rows
//                at a time, lane l their chunks l, l+64, ..., and walks its
//                row sets as one stream with the words of the next two items
//                in flight; dot products with v_dot2_f32_{f16,bf16} on packed
//                pairs, reduced across the wave at the end of each row set.
//   gemm_kernel  (M > 4): 64x64 output tiles, K in steps of 128 staged in
//                LDS as packed pairs (the W tile dequantized by all 256
//                threads, one 32-code chunk each), v_mfma_f32_32x32x16_{f16,
//                bf16}, the next two steps' global reads in flight during the
//                current one.  Few tiles (small M·N) split K over blockIdx.z
//                into fp32 partials in the caller's workspace, summed in split
//                order by reduce_kernel, so the result does not depend on
//                timing.
#include <utility>

#include "common.hpp"

namespace gq {
namespace {

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

struct WArgs {
  const uint16_t* A; int64_t M, K, lda; int vec_a;
  const uint32_t* q; int bits; int64_t row_words;
  const uint16_t* s16; const uint16_t* z16; int64_t ng; int64_t g;
  const int32_t* g_idx;
  int64_t N; float* C; int64_t ldc;
  float* P; int64_t kper;   // split-K partials [splits x M x N] (null: no split) and K per split
  uint64_t cpg_magic;       // ceil(2^32 / chunks per group), up to 2^32
};
// group of chunk c: c / (chunks per group) as a multiply-high, exact for
// c < 2^11 (K <= 65536) and at most 2^20 chunks per group
__device__ __forceinline__ int chunk_group(const WArgs& a, int c) {
  return (int)(((uint64_t)(uint32_t)c * a.cpg_magic) >> 32);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// two exact fp32 values rounded to the activation format, packed (lo = x)
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  if constexpr (F16) return __builtin_bit_cast(uint32_t, f16x2{(_Float16)x, (_Float16)y});
  else return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x, (__bf16)y});
}
template <bool F16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                           c, false);
}

// The BITS words of chunk c of a row (words beyond the row's end read as 0).
template <int BITS>
__device__ __forceinline__ void load_chunk(const uint32_t* __restrict__ row, int64_t row_words,
                                           int64_t c, uint32_t (&w)[BITS]) {
  const int64_t w0 = c * BITS;
  if (w0 + BITS <= row_words) {
    // one vector load (dwordx2/x3/x4; global loads need 4-byte alignment only)
    __builtin_memcpy(w, row + w0, sizeof(w));
  } else {
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = w0 + i < row_words ? row[w0 + i] : 0u;
  }
}
// code J of a chunk (J a compile-time constant: shifts and masks only)
template <int BITS, int J>
__device__ __forceinline__ uint32_t code_of(const uint32_t (&w)[BITS]) {
  constexpr int p = J * BITS, wi = p >> 5, sh = p & 31;
  if constexpr (sh + BITS <= 32 || wi + 1 >= BITS) return (w[wi] >> sh) & ((1u << BITS) - 1u);
  else return ((w[wi] >> sh) | (w[wi + 1] << (32 - sh))) & ((1u << BITS) - 1u);
}

// codes J0 .. J0+2·NP−1 of a chunk as NP packed pairs, one scale and zero
template <bool F16, int BITS, int J0, int... Ps>
__device__ __forceinline__ void dequant_pairs(const uint32_t (&w)[BITS], float s, float nzs,
                                              uint32_t* out, std::integer_sequence<int, Ps...>) {
  ((out[Ps] = pack2<F16>(fmaf((float)code_of<BITS, J0 + 2 * Ps>(w), s, nzs),
                         fmaf((float)code_of<BITS, J0 + 2 * Ps + 1>(w), s, nzs))), ...);
}
// the same with each column's own group through g_idx (act-order layers)
template <bool F16, int BITS, int J0, int... Ps>
__device__ __forceinline__ void dequant_pairs_gidx(const WArgs& a, const uint32_t (&w)[BITS],
                                                   int64_t n, int64_t k0, uint32_t* out,
                                                   std::integer_sequence<int, Ps...>) {
  auto val = [&](uint32_t code, int j) {
    const int64_t k = k0 + j < a.K ? k0 + j : a.K - 1;
    const int64_t gi = a.g_idx[k];
    const float s = half_bits_to_f32(a.s16[n * a.ng + gi]);
    const float z = half_bits_to_f32(a.z16[n * a.ng + gi]);
    return fmaf((float)code, s, -z * s);
  };
  ((out[Ps] = pack2<F16>(val(code_of<BITS, J0 + 2 * Ps>(w), J0 + 2 * Ps),
                         val(code_of<BITS, J0 + 2 * Ps + 1>(w), J0 + 2 * Ps + 1))), ...);
}

// fp16 activations, 4-bit codes: the chunk's 16 pairs (codes 8i+p, 8i+p+4)
// at index 4i+p, from packed-half arithmetic (see above)
template <bool F16, int BITS>
constexpr bool kHalfPairs = F16 && BITS == 4;
__device__ __forceinline__ void dequant_half4(const uint32_t (&w)[4], uint16_t s16, uint16_t z16,
                                              uint32_t* out) {
  const _Float16 z = __builtin_bit_cast(_Float16, z16);
  const _Float16 off = (_Float16)(-1024.f) - z;   // exact: z <= 15
  const f16x2 o2 = {off, off};
  const _Float16 sh = __builtin_bit_cast(_Float16, s16);
  const f16x2 s2 = {sh, sh};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f16x2 x = __builtin_bit_cast(f16x2, ((w[i] >> (4 * p)) & 0x000F000Fu) | 0x64006400u);
      out[4 * i + p] = __builtin_bit_cast(uint32_t, (x + o2) * s2);
    }
}
// four packed pairs of 8 consecutive activations (a0a1, a2a3, a4a5, a6a7)
// re-paired as (a0a4, a1a5, a2a6, a3a7)
__device__ __forceinline__ u32x4 pair_j_j4(u32x4 v) {
  return u32x4{(v[0] & 0xFFFFu) | (v[2] << 16), (v[0] >> 16) | (v[2] & 0xFFFF0000u),
               (v[1] & 0xFFFFu) | (v[3] << 16), (v[1] >> 16) | (v[3] & 0xFFFF0000u)};
}

// ---------------------------------------------------------------- GEMV
constexpr int kGemvLds = 64 * 1024;   // bytes of A staged per workgroup
constexpr int RW = 2;                 // weight rows per wave pass

template <int BITS>
struct Fetch {
  uint32_t w[RW][BITS];
  uint16_t s[RW], z[RW];
};

// the 16 pairs of chunk c of row n in the kernels' pair order
template <bool F16, int BITS, bool GIDX>
__device__ __forceinline__ void dequant_chunk(const WArgs& a, const uint32_t (&w)[BITS], uint16_t s16,
                                              uint16_t z16, int64_t n, int64_t c, uint32_t* out) {
  if constexpr (GIDX) {
    dequant_pairs_gidx<F16, BITS, 0>(a, w, n, c * 32, out, std::make_integer_sequence<int, 16>{});
  } else if constexpr (kHalfPairs<F16, BITS>) {
    dequant_half4(w, s16, z16, out);
  } else {
    const float s = half_bits_to_f32(s16), z = half_bits_to_f32(z16);
    dequant_pairs<F16, BITS, 0>(w, s, -z * s, out, std::make_integer_sequence<int, 16>{});
  }
}

template <bool F16, int BITS, int MM, bool GIDX>
__global__ __launch_bounds__(256) void gemv_kernel(WArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t Ap[];   // [MM][Kp/2] packed pairs
  constexpr bool PERM = kHalfPairs<F16, BITS> && !GIDX;
  const int t = threadIdx.x, lane = t & 63;
  const int64_t Kp = (a.K + 31) / 32 * 32;   // A rows padded to whole chunks (zeros)
  const int64_t KW = Kp / 2;
  const int64_t nch = Kp / 32;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (t >> 6), nwaves = (int64_t)gridDim.x * 4;
  auto fetch = [&](int64_t n0, int64_t c, Fetch<BITS>& f) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int64_t n = n0 + r < a.N ? n0 + r : a.N - 1;   // rows past N: never stored
      load_chunk<BITS>(a.q + n * a.row_words, a.row_words, c, f.w[r]);
      f.s[r] = 0;
      f.z[r] = 0;
      if (!GIDX) {
        const int64_t gi = chunk_group(a, (int)c);
        f.s[r] = a.s16[n * a.ng + gi];
        f.z[r] = a.z16[n * a.ng + gi];
      }
    }
  };
  // One stream per wave: item (set, j) is chunk slot j of row set `set`
  // (rows n0 = (wave + set·nwaves)·RW .., chunk c = lane + 64j); every lane
  // runs the same items (slots past the row's chunks add nothing), so the
  // wave reduction at each row set's last slot is uniform.  The words of the
  // next two items are always in flight, across row sets too; the first two
  // are issued before A is staged.  Item positions advance by additions.
  const int cps = (int)((nch + 63) / 64);
  const int64_t set_stride = nwaves * RW;
  int64_t f_n0 = wave * RW;   // the next item to fetch
  int f_j = 0;
  auto fetch_next = [&](Fetch<BITS>& f) {
    const int c = lane + 64 * f_j;
    if (f_n0 < a.N && c < nch) fetch(f_n0, c, f);
    if (++f_j == cps) { f_j = 0; f_n0 += set_stride; }
  };
  Fetch<BITS> cur, nxt;
  fetch_next(cur);
  fetch_next(nxt);
  for (int64_t e = t; e < MM * Kp / 8; e += 256) {   // 8 values (16 bytes) per item
    const int64_t m = e / (Kp / 8), k = (e % (Kp / 8)) * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (m < a.M) {
      const uint16_t* src = a.A + m * a.lda + k;
      if (a.vec_a && k + 8 <= a.K) {
        v = *reinterpret_cast<const u32x4*>(src);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = k + j < a.K ? src[j] : 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = h[2 * j] | (h[2 * j + 1] << 16);
      }
    }
    if (PERM) v = pair_j_j4(v);
    *reinterpret_cast<u32x4*>(Ap + m * KW + k / 2) = v;
  }
  __syncthreads();
  float acc[RW][MM];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[r][m] = 0.f;
  int64_t n0 = wave * RW;
  int j = 0;
  while (n0 < a.N) {
    const int c = lane + 64 * j;
    Fetch<BITS> nx2;
    fetch_next(nx2);   // two items ahead
    if (c < nch) {
      uint32_t ap[MM][16];
#pragma unroll
      for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(Ap + m * KW + c * 16 + 4 * q);
#pragma unroll
          for (int j = 0; j < 4; ++j) ap[m][4 * q + j] = v[j];
        }
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        uint32_t wp[16];
        const int64_t n = n0 + r < a.N ? n0 + r : a.N - 1;
        dequant_chunk<F16, BITS, GIDX>(a, cur.w[r], cur.s[r], cur.z[r], n, c, wp);
#pragma unroll
        for (int m = 0; m < MM; ++m)
#pragma unroll
          for (int p = 0; p < 16; ++p) acc[r][m] = dot2<F16>(ap[m][p], wp[p], acc[r][m]);
      }
    }
    cur = nxt;
    nxt = nx2;
    if (j == cps - 1) {   // the row set's last slot: reduce and store
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MM; ++m) {
          float v = acc[r][m];
          for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
          if (lane == 0 && m < a.M && n0 + r < a.N) a.C[m * a.ldc + n0 + r] = v;
          acc[r][m] = 0.f;
        }
    }
    if (++j == cps) { j = 0; n0 += set_stride; }
  }
}

// ---------------------------------------------------------------- GEMM
constexpr int TM = 64, TN = 64, TK = 128;
constexpr int LP = TK / 2 + 4;   // LDS row stride in packed pairs (pad: conflict-free reads)

template <bool F16, int BITS, bool GIDX>
__global__ __launch_bounds__(256) void gemm_kernel(WArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t As[TM * LP];
  __shared__ __attribute__((aligned(16))) uint32_t Ws[TN * LP];
  constexpr bool PERM = kHalfPairs<F16, BITS> && !GIDX;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;   // wave tile: rows 32·wm, columns 32·wn
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  const int64_t kb = (int64_t)blockIdx.z * a.kper;
  const int64_t ke = kb + a.kper < a.K ? kb + a.kper : a.K;
  // A loader: row t/4, 32 values at k offset 32·(t%4); W loader: tile row
  // t%64, chunk t/64 of the step (all 32 codes)
  const int ar = t >> 2, ak = (t & 3) * 32;
  const int wr = t & 63, wc = t >> 6;
  const int64_t am = m0 + ar;
  const int nch = (int)((a.K + 31) / 32);
  const int64_t wnr = n0 + wr < a.N ? n0 + wr : a.N - 1;   // rows past N: never stored
  const uint32_t* wrow = a.q + wnr * a.row_words;
  struct Stage {
    u32x4 av[4];
    uint32_t w[BITS];
    uint16_t s, z;
  };
  auto fetch = [&](int64_t k0, Stage& st) {
    const int64_t k = k0 + ak;
    if (am < a.M && a.vec_a && k + 32 <= a.K) {
      const uint16_t* src = a.A + am * a.lda + k;
#pragma unroll
      for (int q = 0; q < 4; ++q) st.av[q] = *reinterpret_cast<const u32x4*>(src + 8 * q);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t kk = k + 8 * q + j;
          h[j] = (am < a.M && kk < a.K) ? a.A[am * a.lda + kk] : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) st.av[q][j] = h[2 * j] | (h[2 * j + 1] << 16);
      }
    }
    const int c = (int)(k0 >> 5) + wc;
    load_chunk<BITS>(wrow, a.row_words, c, st.w);
    st.s = 0;
    st.z = 0;
    if (!GIDX) {
      const int64_t gi = chunk_group(a, c < nch ? c : nch - 1);
      st.s = a.s16[wnr * a.ng + gi];
      st.z = a.z16[wnr * a.ng + gi];
    }
  };
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // three stages: the current one and the next two in flight
  Stage cur, nxt, nx2;
  if (kb < ke) fetch(kb, cur);
  if (kb + TK < ke) fetch(kb + TK, nxt);
  for (int64_t k0 = kb; k0 < ke; k0 += TK) {
    const bool more = k0 + TK < ke;
    if (k0 + 2 * TK < ke) fetch(k0 + 2 * TK, nx2);
    // this step's tiles into LDS: A as loaded; W dequantized (codes past K
    // pair with zero activations, so their values do not matter)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(As + ar * LP + ak / 2 + 4 * q) = PERM ? pair_j_j4(cur.av[q]) : cur.av[q];
    uint32_t wp[16];
    dequant_chunk<F16, BITS, GIDX>(a, cur.w, cur.s, cur.z, wnr, k0 / 32 + wc, wp);
    uint32_t* wd = Ws + wr * LP + 16 * wc;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(wd + 4 * q) = u32x4{wp[4 * q], wp[4 * q + 1], wp[4 * q + 2], wp[4 * q + 3]};
    __syncthreads();
    // eight k-steps of 16: lane holds 8 k (one group of 8) of row / column lane % 32
#pragma unroll
    for (int ks = 0; ks < TK / 16; ++ks) {
      const int kk = ks * 8 + (lane >> 5) * 4;   // in pairs
      const u32x4 av = *reinterpret_cast<const u32x4*>(As + (wm * 32 + (lane & 31)) * LP + kk);
      const u32x4 bv = *reinterpret_cast<const u32x4*>(Ws + (wn * 32 + (lane & 31)) * LP + kk);
      if constexpr (F16)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                     __builtin_bit_cast(f16x8, bv), acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      cur = nxt;
      nxt = nx2;
    }
  }
  float* out = a.P ? a.P + (int64_t)blockIdx.z * a.M * a.N : a.C;
  const int64_t ldo = a.P ? a.N : a.ldc;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t m = m0 + wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
    const int64_t n = n0 + wn * 32 + (lane & 31);
    if (m < a.M && n < a.N) out[m * ldo + n] = acc[r];
  }
}

// C = Σ_s P[s] in split order
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ P, int splits,
                                                     int64_t M, int64_t N, float* __restrict__ C,
                                                     int64_t ldc) {
  const int64_t MN = M * N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < MN; e += (int64_t)gridDim.x * 256) {
    float v = P[e];
    for (int s = 1; s < splits; ++s) v += P[s * MN + e];
    C[(e / N) * ldc + e % N] = v;
  }
}

// K splits for the GEMM: enough (tile, split) workgroups for two per CU
int gemm_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ceil_div(M, TM) * ceil_div(N, TN);
  const int64_t steps = ceil_div(K, TK);
  int64_t s = std::min<int64_t>(ceil_div(512, tiles), std::min<int64_t>(steps, 16));
  if (s < 2) return 1;
  const int64_t kper = ceil_div(steps, s) * TK;
  return (int)ceil_div(K, kper);
}

}  // namespace

size_t w4a16_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 4) return 256;
  const int s = gemm_splits(M, N, K);
  return s > 1 ? align_up((size_t)s * M * N * 4) : 256;
}

hipError_t w4a16_launch(const void* A, int a_dtype, int64_t M, int64_t K, int64_t lda,
                        const uint32_t* qweight, int bits, const uint16_t* s16, const uint16_t* z16,
                        const int32_t* g_idx, int64_t g, int64_t ng, int64_t N, float* C,
                        int64_t ldc, void* ws, size_t ws_bytes, hipStream_t s) {
  const int vec_a = ((uintptr_t)A % 16 == 0) && (lda % 8 == 0);
  const uint64_t cpg = g >= K ? (1u << 20) : (uint64_t)(g / 32);   // one group: all in group 0
  const uint64_t magic = ((uint64_t)1 << 32) / cpg + (((uint64_t)1 << 32) % cpg != 0);
  WArgs a{static_cast<const uint16_t*>(A), M, K, lda, vec_a, qweight, bits, ceil_div(K * bits, 32),
          s16, z16, ng, g, g_idx, N, C, ldc, nullptr, K, magic};
  const bool f16 = a_dtype == GPTQ_F16;
  const bool gx = g_idx != nullptr;
  const int mm = M <= 1 ? 1 : M <= 2 ? 2 : 4;
  const int64_t Kp = ceil_div(K, 32) * 32;
  if (M <= 4 && (int64_t)mm * Kp * 2 <= kGemvLds) {
    // at most four workgroups per CU: each stages A once and loops over rows
    const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(ceil_div(N, 4 * RW), 1024));
    const size_t lds = (size_t)mm * Kp * 2;
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
    return hipGetLastError();
  }
  int splits = gemm_splits(M, N, K);
  if (splits > 1 && (!ws || ws_bytes < w4a16_ws_bytes(M, N, K))) splits = 1;
  if (splits > 1) {
    a.P = static_cast<float*>(ws);
    a.kper = ceil_div(ceil_div(K, TK), splits) * TK;
    splits = (int)ceil_div(K, a.kper);
  }
  const dim3 grid((unsigned)ceil_div(N, TN), (unsigned)ceil_div(M, TM), (unsigned)splits);
#define GQ_GEMM_G(F, B) \
  if (gx) gemm_kernel<F, B, true><<<grid, 256, 0, s>>>(a); else gemm_kernel<F, B, false><<<grid, 256, 0, s>>>(a);
#define GQ_GEMM(F)                                \
  switch (bits) {                                 \
    case 2: GQ_GEMM_G(F, 2); break;               \
    case 3: GQ_GEMM_G(F, 3); break;               \
    case 4: GQ_GEMM_G(F, 4); break;               \
    default: GQ_GEMM_G(F, 8); break;              \
  }
  if (f16) { GQ_GEMM(true) } else { GQ_GEMM(false) }
#undef GQ_GEMM
#undef GQ_GEMM_G
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const unsigned gr = (unsigned)std::min<int64_t>(ceil_div(M * N, 256), 4096);
  reduce_kernel<<<gr, 256, 0, s>>>(a.P, splits, M, N, C, ldc);
  return hipGetLastError();
}

}  // namespace gq
