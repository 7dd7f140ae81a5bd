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
//                staged once per workgroup (16 waves per CU) while the
//                first weight words are in flight; a wave takes 2 weight rows
//                at a time, lane l their chunks l, l+64, ..., and walks its
//                row sets as one stream with the words of the next two items
//                in flight; dot products with v_dot2_f32_{f16,bf16} on packed
//                pairs, reduced across the wave at the end of each row set.
//   gemm_kernel  (M > 4): (32·MT) x 128 output tiles, each lane dequantizing
//                the codes of its own MFMA B operands into registers (every
//                weight once per row tile), A staged in LDS per step of 64,
//                v_mfma_f32_32x32x16_{f16,bf16}, the next three steps' codes
//                and A values in flight.  Few tiles split K over blockIdx.z into fp32
//                partials in the caller's workspace, summed in split order by
//                reduce_kernel, so the result does not depend on timing.
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
  uint32_t q_bytes;         // bytes of the weight words (< 2^32)
  uint32_t a_bytes;         // bytes of A from its first element to the last row's K-th value
};
// Buffer resources (byte-addressed, stride 0): reads past num_records return
// 0 without a branch, so the loads of the kernels' loops are straight-line
// and the compiler can keep every prefetch in flight (divergent load paths
// make it wait for all outstanding loads where they join).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
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

// The BITS words of chunk c of row n (words past the row's end belong to
// the next row, or read 0 past the buffer: they only ever pair with zero
// activations).
template <int BITS>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t rs, int64_t row_words, int64_t n,
                                           int64_t c, uint32_t (&w)[BITS]) {
  const uint32_t off = (uint32_t)((n * row_words + c * BITS) * 4);
  if constexpr (BITS == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (BITS == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(rs, off, 0, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  } else if constexpr (BITS == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    const auto u = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) { w[i] = v[i]; w[4 + i] = u[i]; }
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

// Workgroup barrier for LDS data only: the LDS writes before it are visible
// after it, and global loads in flight stay in flight (__syncthreads() would
// also wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// f(integral_constant<int, I>) for I = B .. E−1, in order
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------- GEMV
constexpr int kGemvLds = 64 * 1024;   // bytes of A staged per workgroup
constexpr int RW = 2;                 // weight rows per wave pass
constexpr int GPD = 3;                // ring slots (items loaded GPD−1 ahead)

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

// threads per GEMV workgroup: four A rows take up to 64 KB of LDS, two
// workgroups per CU, so they run eight waves each
constexpr int gemv_threads(int MM) { return MM == 4 ? 512 : 256; }

template <bool F16, int BITS, int MM, bool GIDX>
__global__ __launch_bounds__(gemv_threads(MM)) void gemv_kernel(WArgs a) {
  constexpr int GT = gemv_threads(MM), GW = GT / 64;
  extern __shared__ __attribute__((aligned(16))) uint32_t Ap[];   // [MM][Kp/2] packed pairs
  constexpr bool PERM = kHalfPairs<F16, BITS> && !GIDX;
  const int t = threadIdx.x, lane = t & 63;
  const int64_t Kp = (a.K + 31) / 32 * 32;   // A rows padded to whole chunks (zeros)
  const int64_t KW = Kp / 2;
  const int64_t nch = Kp / 32;
  // the wave index as a scalar: the item loop below is uniform per wave
  const int64_t wave = (int64_t)blockIdx.x * GW + __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * GW;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q, a.q_bytes);
  // rows past N and chunks past the row are fetched from the last row and
  // chunk (in bounds, never used), so every fetch is the same straight-line
  // code
  auto fetch = [&](int64_t n0, int64_t c, Fetch<BITS>& f) {
    const int64_t cc = c < nch ? c : nch - 1;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int64_t n = n0 + r < a.N ? n0 + r : a.N - 1;   // rows past N: never stored
      load_chunk<BITS>(qrs, a.row_words, n, cc, f.w[r]);
      f.s[r] = 0;
      f.z[r] = 0;
      if (!GIDX) {
        const int64_t gi = chunk_group(a, (int)cc);
        f.s[r] = a.s16[n * a.ng + gi];
        f.z[r] = a.z16[n * a.ng + gi];
      }
    }
  };
  // One stream per wave: item (set, j) is chunk slot j of row set `set`
  // (rows n0 = (wave + set·nwaves)·RW .., chunk c = lane + 64j); every lane
  // runs the same items (slots past the row's chunks add nothing), so the
  // wave reduction at each row set's last slot is uniform.  The words of the
  // items are loaded into a ring of GPD slots, GPD−1 items ahead, across row
  // sets too; the first ones are issued before A is staged.  Item positions
  // advance by additions.
  const int cps = (int)((nch + 63) / 64);
  const int64_t set_stride = nwaves * RW;
  const int64_t nsets = (a.N + RW - 1) / RW;
  const int64_t items = wave < nsets ? ((nsets - 1 - wave) / nwaves + 1) * cps : 0;
  int64_t f_n0 = wave * RW;   // the next item to fetch
  int f_j = 0;
  auto fetch_next = [&](Fetch<BITS>& f) {
    fetch(f_n0 < a.N ? f_n0 : a.N - 1, lane + 64 * f_j, f);
    if (++f_j == cps) { f_j = 0; f_n0 += set_stride; }
  };
  // A into LDS, 16 bytes (8 values) per thread and item, four items per
  // thread at a time, straight-line: rows past M read 0 (past the buffer),
  // values past K are masked to 0; 4-byte aligned rows load as one dwordx4,
  // others as eight 16-bit loads.  The first items of the weight stream are
  // issued behind the first batch of A, so they stay in flight while it is
  // written.
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(a.A, a.a_bytes);
  const int ipr = (int)(Kp / 8), nitems_a = MM * ipr;   // 16-byte items per row, in all
  Fetch<BITS> ring[GPD];
  auto stage_a = [&](int e0, auto first, auto vec) {
    u32x4 v[4];
    int ke[4], me[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + t + GT * i;
      me[i] = (int)((uint32_t)e / (uint32_t)ipr);
      ke[i] = (e - me[i] * ipr) * 8;
      const uint32_t off = e < nitems_a && me[i] < a.M ? (uint32_t)((me[i] * a.lda + ke[i]) * 2) : a.a_bytes;
      if constexpr (decltype(vec)::value) {
        v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, off, 0, 0));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v[i][j] = __builtin_amdgcn_raw_buffer_load_b16(ars, off + 4 * j, 0, 0) |
                    ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(ars, off + 4 * j + 2, 0, 0) << 16);
      }
    }
    if constexpr (decltype(first)::value) {
#pragma unroll
      for (int p = 0; p < GPD - 1; ++p) fetch_next(ring[p]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + t + GT * i;
      if (e < nitems_a) {
        const int64_t left = a.K - ke[i];   // values of this item inside K
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t keep = left >= 2 * j + 2 ? 0xFFFFFFFFu : (left == 2 * j + 1 ? 0xFFFFu : 0u);
          v[i][j] &= keep;
        }
        *reinterpret_cast<u32x4*>(Ap + me[i] * KW + ke[i] / 2) = PERM ? pair_j_j4(v[i]) : v[i];
      }
    }
  };
  auto stage_all = [&](auto vec) {
    stage_a(0, std::true_type{}, vec);
    for (int e0 = 4 * GT; e0 < nitems_a; e0 += 4 * GT) stage_a(e0, std::false_type{}, vec);
  };
  if (a.vec_a) stage_all(std::true_type{}); else stage_all(std::false_type{});
  lds_barrier();
  float acc[RW][MM];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MM; ++m) acc[r][m] = 0.f;
  int64_t n0 = wave * RW;
  int j = 0;
  auto item = [&](auto pc) {
    constexpr int p = decltype(pc)::value;
    // the slot of the previous item (already used) takes the item GPD−1 ahead
    fetch_next(ring[(p + GPD - 1) % GPD]);
    const int c = lane + 64 * j;
    const bool valid = c < nch;
    const int ca = valid ? c : (int)nch - 1;
    uint32_t ap[MM][16];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(Ap + m * KW + ca * 16 + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) ap[m][4 * q + i] = v[i];
      }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      uint32_t wp[16];
      const int64_t n = n0 + r < a.N ? n0 + r : a.N - 1;
      dequant_chunk<F16, BITS, GIDX>(a, ring[p].w[r], ring[p].s[r], ring[p].z[r], n, ca, wp);
#pragma unroll
      for (int m = 0; m < MM; ++m) {
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ps = dot2<F16>(ap[m][i], wp[i], ps);
        acc[r][m] += valid ? ps : 0.f;
      }
    }
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
  };
  static_assert(GPD == 3, "the loop below is unrolled for GPD = 3");
  int64_t it = 0;
  for (; it + GPD <= items; it += GPD) {
    item(std::integral_constant<int, 0>{});
    item(std::integral_constant<int, 1>{});
    item(std::integral_constant<int, 2>{});
  }
  if (it < items) item(std::integral_constant<int, 0>{});
  if (it + 1 < items) item(std::integral_constant<int, 1>{});
}

// ---------------------------------------------------------------- GEMM

// A workgroup computes a BM x 128 output tile (BM = 32·MT rows, MT <= 4; four
// waves of 32 columns each) over its K range in steps of 64.  Each lane
// dequantizes exactly the codes its own MFMA B operands need, straight into
// registers: lane (n, h) (n = lane % 32, h = lane / 32) takes the 32-code
// chunk h of the step for column n, and K-substep s (of four, 16 deep each)
// reads its pairs 4s..4s+3, so the 64 codes of the step meet the A values
// in the same permuted K order on both sides (MFMA sums over k in any
// order).  Every weight is dequantized once per row tile, by one lane.  The
// A tile (BM x 64 as packed pairs, re-paired like the weights) is staged in
// LDS, double-buffered, one barrier per step; the codes and A values of the
// next PD−1 steps are in flight while the current step is dequantized.
constexpr int TKS = 64;          // K per step
constexpr int LPA = TKS / 2 + 4; // LDS row stride of A in packed pairs (conflict-free b128 reads)
constexpr int TNW = 32;          // columns per wave
constexpr int TN = 4 * TNW;      // columns per workgroup
constexpr int PD = 4;            // steps in flight (even: the A buffers alternate with the step)
static_assert(PD % 2 == 0, "");

template <bool F16, int BITS, int MT, bool GIDX, bool VA>
__global__ __launch_bounds__(256) void gemm_kernel(WArgs a) {
  constexpr int BM = 32 * MT;
  __shared__ __attribute__((aligned(16))) uint32_t As[2][BM * LPA];
  constexpr bool PERM = kHalfPairs<F16, BITS> && !GIDX;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * TN;
  const int64_t kb = (int64_t)blockIdx.z * a.kper;
  const int64_t ke = kb + a.kper < a.K ? kb + a.kper : a.K;
  const int nch = (int)((a.K + 31) / 32);
  const int64_t ncol = n0 + wv * TNW + l32;
  const int64_t wn = ncol < a.N ? ncol : a.N - 1;   // columns past N: never stored
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q, a.q_bytes);
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(a.A, a.a_bytes);
  // A loader: unit u = t + 256i (i < MT) is row u / 8, values 8(u % 8) .. +7
  // of the step; rows past M read 0 (past the buffer); dword loads need
  // 4-byte aligned rows (VA), else eight 16-bit loads.  The ring holds the
  // raw loads: nothing touches them until the step's A goes to LDS, so the
  // loads stay in flight meanwhile.
  auto load_a = [&](int64_t k0, u32x4 (&av)[MT]) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int u = t + 256 * i, row = u >> 3, q8 = (u & 7) * 8;
      const int64_t m = m0 + row, k = k0 + q8;
      const uint32_t off = m < a.M ? (uint32_t)((m * a.lda + k) * 2) : a.a_bytes;
      if constexpr (VA) {
        av[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, off, 0, 0));
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          av[i][j] = __builtin_amdgcn_raw_buffer_load_b16(ars, off + 4 * j, 0, 0) |
                     ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(ars, off + 4 * j + 2, 0, 0) << 16);
      }
    }
  };
  // values past K are masked to 0 (they would meet codes that do not belong
  // to the row), then the pairs are re-paired like the weights
  auto store_a = [&](const u32x4 (&av)[MT], int64_t k0, uint32_t* buf) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int u = t + 256 * i, row = u >> 3, q8 = (u & 7) * 8;
      const int64_t left = a.K - (k0 + q8);   // values of this group of 8 inside K
      u32x4 v = av[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t keep = left >= 2 * j + 2 ? 0xFFFFFFFFu : (left == 2 * j + 1 ? 0xFFFFu : 0u);
        v[j] &= keep;
      }
      *reinterpret_cast<u32x4*>(buf + row * LPA + q8 / 2) = PERM ? pair_j_j4(v) : v;
    }
  };
  struct Stage {
    uint32_t w[BITS];
    uint16_t s, z;
  };
  auto fetch = [&](int64_t k0, Stage& st) {
    const int c0 = (int)(k0 >> 5) + h, c = c0 < nch ? c0 : nch - 1;
    load_chunk<BITS>(qrs, a.row_words, wn, c, st.w);
    st.s = 0;
    st.z = 0;
    if (!GIDX) {
      const int64_t gi = chunk_group(a, c);
      st.s = a.s16[wn * a.ng + gi];
      st.z = a.z16[wn * a.ng + gi];
    }
  };
  f32x16 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  // a ring of PD steps in flight: codes and A values of steps i+1 .. i+PD−1
  // are loading while step i computes.  The loop is unrolled by PD so every
  // ring slot is a fixed set of registers, and its body is straight-line:
  // the refill of a slot is never skipped, it re-reads the last step (from
  // cache) once no step is left to load.
  Stage st[PD];
  u32x4 av[PD][MT];
  const int64_t nsteps = ke > kb ? (ke - kb + TKS - 1) / TKS : 0;
  const int64_t klast = kb + (nsteps - 1) * TKS;
  if (nsteps > 0) {
#pragma unroll
    for (int p = 0; p < PD - 1; ++p) {
      const int64_t kf = kb + p * TKS < klast ? kb + p * TKS : klast;
      fetch(kf, st[p]);
      load_a(kf, av[p]);
    }
    store_a(av[0], kb, As[0]);
    lds_barrier();
  }
  auto step = [&](auto pc, int64_t i) {
    constexpr int p = decltype(pc)::value;
    const int64_t k0 = kb + i * TKS;
    // the slot of step i−1 (dequantized and its A stored) takes step i+PD−1
    {
      constexpr int q = (p + PD - 1) % PD;
      const int64_t kf = k0 + (PD - 1) * TKS < klast ? k0 + (PD - 1) * TKS : klast;
      fetch(kf, st[q]);
      load_a(kf, av[q]);
    }
    // step i+1's A into the other buffer (read by no wave since the last
    // barrier; after the last step nothing reads it)
    store_a(av[(p + 1) % PD], k0 + TKS, As[(p + 1) & 1]);
    // this lane's 32 codes of the step (codes past K pair with zero
    // activations, so their values do not matter)
    uint32_t wp[16];
    dequant_chunk<F16, BITS, GIDX>(a, st[p].w, st[p].s, st[p].z, wn, k0 / 32 + h, wp);
    const uint32_t* ab = As[p & 1];   // step i's buffer (i ≡ p mod PD, PD even)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 bv = {wp[4 * s], wp[4 * s + 1], wp[4 * s + 2], wp[4 * s + 3]};
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const u32x4 avv = *reinterpret_cast<const u32x4*>(ab + (32 * mi + l32) * LPA + 16 * h + 4 * s);
        if constexpr (F16)
          acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8, avv), __builtin_bit_cast(f16x8, bv), acc[mi], 0, 0, 0);
        else
          acc[mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, avv), __builtin_bit_cast(bf16x8, bv), acc[mi], 0, 0, 0);
      }
    }
    lds_barrier();
    // keeps the next step's work (masking A values, dequantizing codes) from
    // being scheduled up into this one, where it would wait for loads that
    // are meant to stay in flight
    __builtin_amdgcn_sched_barrier(0);
  };
  int64_t i0 = 0;
  for (; i0 + PD <= nsteps; i0 += PD)
    static_for<0, PD>([&](auto pc) { step(pc, i0 + decltype(pc)::value); });
  static_for<0, PD - 1>([&](auto pc) {
    if (i0 + decltype(pc)::value < nsteps) step(pc, i0 + decltype(pc)::value);
  });
  float* out = a.P ? a.P + (int64_t)blockIdx.z * a.M * a.N : a.C;
  const int64_t ldo = a.P ? a.N : a.ldc;
  if (ncol < a.N) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + 32 * i + (r >> 2) * 8 + h * 4 + (r & 3);
        if (m < a.M) out[m * ldo + ncol] = acc[i][r];
      }
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

constexpr int gemm_mt(int64_t M) { return M <= 32 ? 1 : M <= 128 ? 2 : 4; }

// K splits for the GEMM: about 256 (tile, split) workgroups, at most eight
// splits and at least eight steps of K per split
int gemm_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ceil_div(M, 32 * gemm_mt(M)) * ceil_div(N, TN);
  const int64_t steps = ceil_div(K, TKS);
  const int64_t s = std::min<int64_t>(ceil_div(256, tiles), std::min<int64_t>(8, steps / 8));
  if (s < 2) return 1;
  const int64_t kper = ceil_div(steps, s) * TKS;
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
  const int vec_a = ((uintptr_t)A % 4 == 0) && (lda % 2 == 0);   // dword loads of A
  const uint64_t cpg = g >= K ? (1u << 20) : (uint64_t)(g / 32);   // one group: all in group 0
  const uint64_t magic = ((uint64_t)1 << 32) / cpg + (((uint64_t)1 << 32) % cpg != 0);
  const int64_t row_words = ceil_div(K * bits, 32);
  const int64_t q_bytes = N * row_words * 4, a_bytes = ((M - 1) * lda + K) * 2;
  if (q_bytes >= ((int64_t)1 << 32) || a_bytes >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
  WArgs a{static_cast<const uint16_t*>(A), M, K, lda, vec_a, qweight, bits, row_words,
          s16, z16, ng, g, g_idx, N, C, ldc, nullptr, K, magic, (uint32_t)q_bytes, (uint32_t)a_bytes};
  const bool va = vec_a;
  const bool f16 = a_dtype == GPTQ_F16;
  const bool gx = g_idx != nullptr;
  const int mm = M <= 1 ? 1 : M <= 2 ? 2 : 4;
  const int64_t Kp = ceil_div(K, 32) * 32;
  if (M <= 4 && (int64_t)mm * Kp * 2 <= kGemvLds) {
    // 4096 waves (sixteen per CU): each workgroup stages A once and its
    // waves loop over rows
    const int gw = gemv_threads(mm) / 64;
    const unsigned grid =
        (unsigned)std::max<int64_t>(1, std::min<int64_t>(ceil_div(N, gw * RW), 4096 / gw));
    const size_t lds = (size_t)mm * Kp * 2;
#define GQ_GEMV(F, B, MM, GX) gemv_kernel<F, B, MM, GX><<<grid, gemv_threads(MM), lds, s>>>(a)
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
    a.kper = ceil_div(ceil_div(K, TKS), splits) * TKS;
    splits = (int)ceil_div(K, a.kper);
  }
  const int mt = gemm_mt(M);
  const dim3 grid((unsigned)ceil_div(N, TN), (unsigned)ceil_div(M, 32 * mt), (unsigned)splits);
#define GQ_GEMM_V(F, B, MT, GX) \
  if (va) gemm_kernel<F, B, MT, GX, true><<<grid, 256, 0, s>>>(a); else gemm_kernel<F, B, MT, GX, false><<<grid, 256, 0, s>>>(a);
#define GQ_GEMM_K(F, B, MT) \
  if (gx) { GQ_GEMM_V(F, B, MT, true) } else { GQ_GEMM_V(F, B, MT, false) }
#define GQ_GEMM_G(F, B)                        \
  switch (mt) {                                \
    case 1: GQ_GEMM_K(F, B, 1); break;         \
    case 2: GQ_GEMM_K(F, B, 2); break;         \
    default: GQ_GEMM_K(F, B, 4); break;        \
  }
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
#undef GQ_GEMM_K
#undef GQ_GEMM_V
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const unsigned gr = (unsigned)std::min<int64_t>(ceil_div(M * N, 256), 4096);
  reduce_kernel<<<gr, 256, 0, s>>>(a.P, splits, M, N, C, ldc);
  return hipGetLastError();
}

}  // namespace gq
