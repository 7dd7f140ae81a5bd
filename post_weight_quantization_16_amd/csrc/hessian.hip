// H += 2·XᵀX for token-major X [n_tok x d] ("GPTQ: Mathematical Foundations
// ...", Second-Order Taylor Expansion and the Hessian: H = 2XXᵀ with the
// page's X = d x N).
//
// Only upper-triangle tiles are computed (SYRK: d(d+1)N flops).  The token
// axis is split S >= 1 ways; each (tile, split) workgroup writes an fp32
// partial tile and a reduction adds 2·Σ_s partial_s into H's upper triangle
// in a fixed order.  A final
// LDS-tiled transpose copies the upper triangle into the lower one, so H is
// exactly symmetric and the result is deterministic.
//
// bf16/fp16 inputs: v_mfma_f32_32x32x16_{bf16,f16}; the products are exact in
// fp32 and accumulate in fp32.
//
// Shifted accumulation.  An fp32 sum of n terms that share a sign loses
// about u·sqrt(n) of its value, and activations with a non-zero channel mean
// make every entry of XᵀX such a sum (the entries grow like N·μ_iμ_j).  Each
// workgroup therefore keeps its accumulators near zero: every 512 tokens it
// adds, with one more MFMA per accumulator tile, the product of the constant
// operands 32·μ_i and −μ_j over its 16 k-slots, i.e. −512·μ_iμ_j, where μ is
// the per-channel mean of the call's first tokens rounded to the input's
// 16-bit format (0 where that mean is not significant).  These products are
// exact in fp32, and the reduction adds the exact total 512·c·μ_iμ_j back in
// fp64 (c = number of such MFMAs over all splits).  The result is the same
// sum with its rounding errors taken relative to the centred partial sums;
// for zero-mean channels μ = 0 and nothing changes.  The split partials are
// summed in fp64 as well, so H leaves the reduction rounded once to fp32.
//
// The MFMA operand wants 8 consecutive tokens of
// one column per lane while X is contiguous along columns:
//   fast path (d, ld multiples of 8, X 16-byte aligned): 256x256 tiles, X kept
//     in natural layout in LDS and read with LDS transpose loads;
//   generic path: 128x128 tiles; each thread loads an 8-token x 8-column block,
//     transposes it in registers and stores [col][token] runs into LDS.
// fp32 inputs: the generic fp32 MFMA GEMM on op(A) = Xᵀ, op(B) = X.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.hpp"
#include "split_plan.hpp"

namespace gq {
namespace {

constexpr int HT = 128;        // output tile
constexpr int HK = 64;         // tokens per LDS stage
constexpr int HLD = HK + 8;    // LDS row stride in 16-bit elements
constexpr int kShiftTok = 512;        // tokens between two shift MFMAs
constexpr int kShiftSample = 1024;    // tokens the shift μ is estimated from

typedef __attribute__((ext_vector_type(8))) short s16x8;

// The shift operands of one lane: 8 k-slots holding the same 16-bit value.
__device__ __forceinline__ s16x8 splat16(uint16_t v) {
  const short x = (short)v;
  return s16x8{x, x, x, x, x, x, x, x};
}
// 32·μ and −μ as 16-bit patterns (exact: a power-of-two scale and a sign
// flip of a value whose magnitude the shift kernel keeps in range)
template <bool BF16>
__device__ __forceinline__ uint16_t times32(uint16_t m) {
  if (m == 0) return 0;
  return (uint16_t)(m + (BF16 ? (5u << 7) : (5u << 10)));   // exponent + 5
}
__device__ __forceinline__ uint16_t negate16(uint16_t m) { return m ? (uint16_t)(m ^ 0x8000u) : 0; }

template <bool BF16>
__device__ __forceinline__ float half_to_f32(uint16_t b) {
  if constexpr (BF16) return __uint_as_float((uint32_t)b << 16);
  else return (float)__builtin_bit_cast(_Float16, b);
}
template <bool BF16>
__device__ __forceinline__ uint16_t f32_to_half_rne(float f) {
  if constexpr (BF16) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  } else {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
}

// μ_c for c < dp: the mean of column c over the first n0 tokens, rounded to
// the 16-bit input format, or 0 when it is not significant (|mean| at most
// 4·std/√n0: a zero-mean channel keeps the plain accumulation) or when
// c >= d.  Workgroup: 16 columns (2 groups of 8 adjacent columns, 16-byte
// loads) x 128 token lanes, so d/16 workgroups share the reads; the lanes'
// sums are combined in a fixed order, so μ is deterministic.  The magnitude is kept below 2^10 so that 32·μ and
// the shift products stay finite in either 16-bit format.
template <bool BF16>
__global__ __launch_bounds__(256) void shift_mean_kernel(const uint16_t* __restrict__ X, int64_t ld,
                                                         int d, int dp, int n0, int vec,
                                                         uint16_t* __restrict__ mu) {
  constexpr int TL = 128, CW = 16;   // token lanes, columns per workgroup
  __shared__ float S1[TL][CW + 1], S2[TL][CW + 1];
  const int t = threadIdx.x, cg = t & 1, tl = t >> 1;
  const int c0 = blockIdx.x * CW + cg * 8;
  float s1[8], s2[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) { s1[q] = 0.f; s2[q] = 0.f; }
  for (int r0 = tl; r0 < n0; r0 += TL * 4) {
    uint16_t e[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + TL * u;
      const uint16_t* p = X + (int64_t)r * ld + c0;
      if (r < n0 && vec && c0 + 7 < d) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) e[u][q] = (uint16_t)(w4[q >> 1] >> (16 * (q & 1)));
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) e[u][q] = (r < n0 && c0 + q < d) ? p[q] : (uint16_t)0;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float x = half_to_f32<BF16>(e[u][q]);
        s1[q] += x;
        s2[q] = fmaf(x, x, s2[q]);
      }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) { S1[tl][cg * 8 + q] = s1[q]; S2[tl][cg * 8 + q] = s2[q]; }
  __syncthreads();
  if (t < CW) {
    const int c = blockIdx.x * CW + t;
    double a = 0.0, b = 0.0;
    for (int l = 0; l < TL; ++l) { a += S1[l][t]; b += S2[l][t]; }
    uint16_t m = 0;
    if (c < d && n0 > 1) {
      const double mean = a / n0;
      const double var = fmax(b / n0 - mean * mean, 0.0);
      // normal numbers only (32·μ is formed by the exponent), below 2^10
      if (fabs(mean) > 4.0 * sqrt(var / n0) && fabs(mean) < 1024.0 && fabs(mean) >= 1.0 / 8192)
        m = f32_to_half_rne<BF16>((float)mean);
    }
    if (c < dp) mu[c] = m;
  }
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;


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
__global__ __launch_bounds__(256) void syrk16_generic_kernel(const uint16_t* __restrict__ X, int64_t ld,
                                                     int d, int64_t n_tok, int64_t chunk, int nt,
                                                     float* __restrict__ P, int64_t dp, int vec,
                                                     const uint16_t* __restrict__ mu) {
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

  // shift operands: 32·μ of this lane's A rows, −μ of its B columns
  uint16_t sa[2], sb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    sa[i] = times32<BF16>(mu[ti * HT + wm * 64 + i * 32 + (lane & 31)]);
    sb[i] = negate16(mu[tj * HT + wn * 64 + i * 32 + (lane & 31)]);
  }
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
    if (((t0 - t_begin) / HK) % (kShiftTok / HK) == kShiftTok / HK - 1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (BF16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, splat16(sa[i])), __builtin_bit_cast(bf16x8, splat16(sb[j])),
                acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, splat16(sa[i])), __builtin_bit_cast(f16x8, splat16(sb[j])),
                acc[i][j], 0, 0, 0);
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

// ---------------------------------------------------------------- fast path
// 256x256 output tiles, 4 waves each owning a 128x128 block (4x4 tiles of
// v_mfma_f32_32x32x16).  X stays in its natural [token][column] layout in
// LDS: stages of 32 tokens, rows of 512 bytes whose 16-byte chunks are
// XOR-swizzled by (row & 3) << 2, in a ring of four stage buffers.  Stages
// go from memory straight into LDS (global_load_lds_dwordx4: no registers,
// no LDS store instructions), three stages ahead, each wave copying 8 KB of
// every stage; a wave waits for its own copies of the stage it is about to
// read (s_waitcnt vmcnt), then one barrier makes everyone's copies visible
// and frees the buffer read in the previous stage for the next copy.  The
// swizzle is applied on the global side (a lane fetches the chunk its LDS
// slot will hold); lanes whose token or column is out of range fetch a
// zeroed 16-byte chunk instead.  The copies are written as inline asm
// because the compiler, not seeing which buffer a copy writes, would wait
// for all of them before every LDS read.  MFMA operands (8 consecutive
// tokens of one column per lane) come from two ds_read_b64_tr_b16 each: in
// every group of 16 lanes, lane i receives element i%4 of the 8-byte piece
// addressed by lane 4r + i/4 (r = 0..3), so lanes addressing 4 rows x 16
// columns get one column each; with the swizzle a half-wave's 4 rows x 64
// bytes hit 64 distinct banks.
// Work placement: workgroup L runs on XCD L % 8; see block_tile.
// Requires d % 8 == 0, ld % 8 == 0 and a 16-byte aligned X.
constexpr int FT = 256;                 // output tile
constexpr int FK = 32;                  // tokens per stage
constexpr int FROW = FT * 2;            // bytes per LDS row (one token)
constexpr int FOP = FK * FROW;          // bytes per operand per stage (16 KB)
constexpr int FSTAGE = 2 * FOP;         // bytes per stage (32 KB)
constexpr int NBUF = 4;                 // stage buffers in the LDS ring (128 KB)
constexpr int kPre = 1;                 // MFMAs of the second batch issued before the barrier
// s_waitcnt immediates (vmcnt is split over bits [3:0] and [15:14];
// expcnt/lgkmcnt not waited): in the loop, 2 stages of copies (8
// instructions each) may stay pending; before it, one
constexpr int kWaitCount = 8 * (NBUF - 2);
constexpr int kWaitStage = ((kWaitCount >> 4) << 14) | (kWaitCount & 15) | 0x70 | 0xF00;
constexpr int kWaitFirstCount = 8 * (NBUF - 3);   // before the loop: stages 0 and 1 done
constexpr int kWaitFirst = ((kWaitFirstCount >> 4) << 14) | (kWaitFirstCount & 15) | 0x70 | 0xF00;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int fswz(int row) { return (row & 3) << 2; }



__device__ __forceinline__ void fast_tile(int L, int nt, int tiles, const SplitPlan& sp, int& ti,
                                          int& tj, int& split, int64_t& chunk) {
  const int grid = (int)gridDim.x;
  chunk = sp.chunk;
  if (sp.hi_tiles > 0) {
    mixed_unit(L, nt, tiles, sp, ti, tj, split, chunk);
  } else if (nt % 4 == 0 && grid % 8 == 0) {
    const int u = (L & 7) * (grid / 8) + (L >> 3);
    split = u / tiles;
    block_tile(u % tiles, nt, ti, tj);
  } else {
    split = L / tiles;
    tile_of(L % tiles, nt, ti, tj);
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void syrk256_kernel(const uint16_t* __restrict__ X, int64_t ld,
                                                       int d, int64_t n_tok, SplitPlan plan, int nt,
                                                       float* __restrict__ P, int64_t dp,
                                                       const uint16_t* __restrict__ zero16,
                                                       const uint16_t* __restrict__ mu) {
  const int tiles = nt * (nt + 1) / 2;
  int ti, tj, split;
  int64_t chunk;
  fast_tile(blockIdx.x, nt, tiles, plan, ti, tj, split, chunk);
  const int64_t t_begin = (int64_t)split * chunk;
  const int64_t t_end = min(n_tok, t_begin + chunk);
  // stages of FK tokens, rounded up to whole shift groups of kShiftTok
  // tokens (stages past the data copy the zero chunk and add nothing)
  constexpr int kGroup = kShiftTok / FK;
  const int nstage = (int)((t_end - t_begin + kShiftTok - 1) / kShiftTok) * kGroup;
  __shared__ __attribute__((aligned(1024))) char S[NBUF * FSTAGE];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // DMA plan: wave w's instruction i fills LDS bytes [(8w+i) KB, +1 KB) of a
  // stage: operand (8w+i)/16, token rows 2((8w+i)%16) + lane/32, 16-byte slot
  // lane%32 which holds chunk slot ^ swizzle(row).
  constexpr int NI = FSTAGE / (4 * 1024);   // copy instructions per wave per stage (8)
  const char* pbase[NI];   // this lane's source for stage 0 (zero chunk if the column is out)
  int rrow[NI];
  bool colok[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int seg = w * NI + i;
    const int op = seg / (FOP / 1024);
    const int r = ((seg % (FOP / 1024)) << 1) + (lane >> 5);
    const int ch = (lane & 31) ^ fswz(r);
    const int col = (op ? tj : ti) * FT + ch * 8;
    colok[i] = col < d;
    rrow[i] = r;
    pbase[i] = colok[i] ? reinterpret_cast<const char*>(X) + (t_begin + r) * ld * 2 + (int64_t)col * 2
                        : reinterpret_cast<const char*>(zero16);
  }
  const unsigned sbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)S;
  const int nrows = (int)(t_end - t_begin);
  // copy instruction i of stage st (the wave's 1 KB piece i of the stage)
  auto dma_one = [&](int st, int i) {
    const int rem = min(max(nrows - st * FK, 0), FK);   // valid token rows of the stage
    const int64_t soff = (int64_t)st * FK * ld * 2;
    const unsigned lb = sbase + (unsigned)((st % NBUF) * FSTAGE) + (unsigned)(w * NI + i) * 1024u;
    const bool ok = colok[i] && rrow[i] < rem;
    const char* a = ok ? pbase[i] + soff : reinterpret_cast<const char*>(zero16);
    // global_load_lds_dwordx4: 16 bytes per lane from address a to LDS
    // M0 + 16·lane.  It has no register result; the stage's wait
    // (s_waitcnt vmcnt) is what orders it before the reads.
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(lb), "v"(a) : "memory");
  };
  auto dma = [&](int st) {
#pragma unroll
    for (int i = 0; i < NI; ++i) dma_one(st, i);
  };
  const int g = lane >> 4, j16 = lane & 15;
  const int rsub = 8 * (g >> 1) + (j16 >> 2);
  const int csub = 16 * (g & 1) + 4 * (j16 & 3);
  // Operand pieces of one 16-token step: piece n = 2f + h is half h (tokens
  // 4h.. of each 8) of fragment f, f = 0..3 the A fragments, 4..7 the B
  // fragments.  They are read in the order the MFMAs first need them.
  constexpr int kOrder[8] = {0, 4, 5, 6, 7, 1, 2, 3};
  auto rd = [&](const char* stage, int ks, int n) {
    const int f = kOrder[n >> 1], h = n & 1;
    const char* base = stage + (f < 4 ? 0 : FOP);
    const int col = (f < 4 ? wm : wn) * 128 + (f & 3) * 32 + csub;
    const int row = ks * 16 + 4 * h + rsub;
    const int off = row * FROW + (((col >> 3) ^ fswz(row)) << 4) + ((col & 7) << 1);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
  };
  // slot of fragment f in the piece array
  constexpr int kSlot[8] = {0, 5, 6, 7, 1, 2, 3, 4};
  auto mm = [&](int n, const s16x4 (&p)[16]) {
    const int fi = n >> 2, fj = n & 3;
    const int sa = kSlot[fi], sb = kSlot[4 + fj];
    const s16x8 a = __builtin_shufflevector(p[2 * sa], p[2 * sa + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    const s16x8 b = __builtin_shufflevector(p[2 * sb], p[2 * sb + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    if constexpr (BF16)
      acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc[fi][fj], 0, 0, 0);
    else
      acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
          __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc[fi][fj], 0, 0, 0);
  };
  static_assert(FK == 32, "a stage is two 16-token MFMA steps");
  auto stage_ptr = [&](int st) { return (const char*)S + (st % NBUF) * FSTAGE; };
  // shift operands (see the top of this file): 32·μ of this lane's A rows
  // and −μ of its B columns, packed two per register
  uint32_t sh[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
    sh[f] = (uint32_t)times32<BF16>(mu[ti * FT + wm * 128 + f * 32 + (lane & 31)]) |
            ((uint32_t)negate16(mu[tj * FT + wn * 128 + f * 32 + (lane & 31)]) << 16);
  auto shift = [&]() {
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int fj = 0; fj < 4; ++fj) {
        const s16x8 a = splat16((uint16_t)(sh[fi] & 0xFFFFu));
        const s16x8 b = splat16((uint16_t)(sh[fj] >> 16));
        if constexpr (BF16)
          acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc[fi][fj], 0, 0, 0);
        else
          acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc[fi][fj], 0, 0, 0);
      }
  };
  for (int s0 = 0; s0 < NBUF - 1; ++s0) dma(s0);
  // Each stage is two batches of 16 MFMAs.  Batch A multiplies the pieces of
  // the stage's first step (p0) while reading those of its second step (p1)
  // and issuing the copies of stage st+3; batch B multiplies p1 while
  // reading the next stage's first step into p0.  One MFMA and one LDS read
  // alternate (scheduling barriers keep the order), so the reads run under
  // the MFMAs.  Between the batches each wave waits for its copies of stage
  // st+1 (the copies of the two stages after it stay in flight) and for its
  // LDS reads, and the barrier makes stage st+1 visible and frees the buffer
  // of stage st (read completely by now) for the next copy.
  // On a diagonal tile only the upper triangle is read by the reduction, so
  // the wave below the diagonal (wm = 1, wn = 0) multiplies nothing: it
  // copies its share of every stage and takes part in the barriers.
  const bool idle = ti == tj && wm > wn;
  __builtin_amdgcn_s_waitcnt(kWaitFirst);
  __builtin_amdgcn_s_barrier();
  if (idle) {
    for (int st = 0; st < nstage; ++st) {
      dma(st + NBUF - 1);
      __builtin_amdgcn_s_waitcnt(kWaitStage & ~0xF00);
      __builtin_amdgcn_s_barrier();
    }
  } else {
    s16x4 p0[16], p1[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) p0[n] = rd(stage_ptr(0), 0, n);
    // one shift per group of 16 stages (512 tokens); the group is unrolled
    // so the shift MFMAs share the stages' basic block (a shift behind a
    // branch made the compiler move the accumulators out of their registers)
    for (int g0 = 0; g0 < nstage; g0 += kGroup) {
#pragma unroll
    for (int st16 = 0; st16 < kGroup; ++st16) {
      const int st = g0 + st16;
      const char* cur = stage_ptr(st);
      const char* nxt = stage_ptr(st + 1);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        mm(n, p0);
        p1[n] = rd(cur, 1, n);
        if (n & 1) dma_one(st + NBUF - 1, n >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int n = 0; n < kPre; ++n) {
        mm(n, p1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // lgkmcnt(0) as well: every wave's reads of this stage's buffer are
      // complete before the barrier after which it is copied over again
      __builtin_amdgcn_s_waitcnt(kWaitStage & ~0xF00);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        if (n + kPre < 16) mm(n + kPre, p1);
        p0[n] = rd(nxt, 0, n);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    shift();
    __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no DMA may outlive the workgroup
  if (idle) return;
  float* Pt = P + (int64_t)split * dp * dp;
#pragma unroll
  for (int fi = 0; fi < 4; ++fi)
#pragma unroll
    for (int fj = 0; fj < 4; ++fj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = ti * FT + wm * 128 + fi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int cl = tj * FT + wn * 128 + fj * 32 + (lane & 31);
        Pt[(int64_t)row * dp + cl] = acc[fi][fj][r];
      }
}

// The 256-byte zero chunk of the workspace (a fill kernel, not a memset, so
// a captured graph replays it correctly).
__global__ __launch_bounds__(64) void zero_chunk_kernel(uint32_t* __restrict__ z) {
  z[threadIdx.x] = 0u;
}

// H[i][j] += 2·(Σ_s P_s[i][j] + c·μ_iμ_j) over the upper triangle, and the
// mirrored H[j][i] = H[i][j], one 32-row strip of a 128x128 upper tile
// (ti <= tj) per workgroup (four per tile, so the strips fill the CUs with
// a short last round).  c·μ_iμ_j restores what the shift MFMAs took out (c
// tokens' worth, mu = null when no shift was applied).  The sum is formed
// in fp64 in a fixed order (deterministic) and rounded once.  Each thread
// owns 4 float4 runs of the strip and issues the loads of four splits
// before adding them, and all of its H reads before any H write (reads
// after a write through the same pointer would each wait a memory round
// trip); the finished strip goes through LDS to be written transposed, so
// both writes are coalesced.
constexpr int RS = 32;   // strip rows

// H = 0 (d² floats), for a Hessian set from no tokens.
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ H, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    H[i] = 0.f;
}
template <bool BF16>
__global__ __launch_bounds__(256) void reduce_mirror_kernel(float* __restrict__ H, int d,
                                                            const float* __restrict__ P,
                                                            int64_t dp, ReducePlan rp, int nt,
                                                            int vec_h,
                                                            const uint16_t* __restrict__ mu,
                                                            int acc_h) {
  int ti, tj;
  tile_of(blockIdx.x >> 2, nt, ti, tj);
  const bool hi = reduce_tile_hi(rp, ti, tj);
  const int splits = hi ? rp.S + 1 : rp.S;
  const double shift_tok = hi ? rp.shift_hi : rp.shift_lo;
  const int r0 = (blockIdx.x & 3) * RS;   // the strip's first row inside the tile
  __shared__ float T[RS][HT + 1];
  __shared__ double mr[RS], mc[HT];
  const int t = threadIdx.x;
  constexpr int NR = RS * HT / (256 * 4);   // float4 runs per thread (4)
  const int64_t pstride = dp * dp;
  const float* src = P + (int64_t)(ti * HT + r0) * dp + tj * HT;   // always inside the partials
  if (mu) {
    if (t < RS) mr[t] = shift_tok * (double)half_to_f32<BF16>(mu[ti * HT + r0 + t]);
    if (t < HT) mc[t] = (double)half_to_f32<BF16>(mu[tj * HT + t]);
  }
  typedef __attribute__((ext_vector_type(4))) double f64x4;
  f64x4 acc[NR];
#pragma unroll
  for (int it = 0; it < NR; ++it) acc[it] = f64x4{0.0, 0.0, 0.0, 0.0};
  constexpr int SG = 4;   // splits whose loads are in flight together
  for (int sp0 = 0; sp0 < splits; sp0 += SG) {
    f32x4 v[SG][NR];
#pragma unroll
    for (int u = 0; u < SG; ++u)
#pragma unroll
      for (int it = 0; it < NR; ++it) {
        const int e = t + 256 * it, a = e >> 5, b4 = (e & 31) * 4;
        const int sp = sp0 + u < splits ? sp0 + u : sp0;
        v[u][it] = *reinterpret_cast<const f32x4*>(src + sp * pstride + (int64_t)a * dp + b4);
      }
    // splits in index order (the loads of a missing split are not added)
#pragma unroll
    for (int u = 0; u < SG; ++u)
      if (sp0 + u < splits)
#pragma unroll
        for (int it = 0; it < NR; ++it)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[it][q] += (double)v[u][it][q];
  }
  if (mu) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < NR; ++it) {
      const int e = t + 256 * it, a = e >> 5, b4 = (e & 31) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[it][q] = fma(mr[a], mc[b4 + q], acc[it][q]);
    }
  }
  const int i0 = ti * HT + r0;   // the strip's first row of H
  const bool full = vec_h && ti < tj && (tj + 1) * HT <= d;
  if (full) {
    f32x4 h[NR];
#pragma unroll
    for (int it = 0; it < NR; ++it) {
      const int e = t + 256 * it, a = e >> 5, b4 = (e & 31) * 4;
      h[it] = acc_h ? *reinterpret_cast<const f32x4*>(H + (int64_t)(i0 + a) * d + tj * HT + b4)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int it = 0; it < NR; ++it) {
      const int e = t + 256 * it, a = e >> 5, b4 = (e & 31) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) h[it][q] = (float)fma(2.0, acc[it][q], (double)h[it][q]);
      *reinterpret_cast<f32x4*>(H + (int64_t)(i0 + a) * d + tj * HT + b4) = h[it];
#pragma unroll
      for (int q = 0; q < 4; ++q) T[a][b4 + q] = h[it][q];
    }
  } else {
    for (int it = 0; it < NR; ++it) {
      const int e = t + 256 * it, a = e >> 5, b4 = (e & 31) * 4;
      const int i = i0 + a;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int jq = tj * HT + b4 + q;
        float v = 0.f;
        if (i < d && jq < d && jq >= i) {
          v = (float)fma(2.0, acc[it][q], acc_h ? (double)H[(int64_t)i * d + jq] : 0.0);
          H[(int64_t)i * d + jq] = v;
        }
        T[a][b4 + q] = v;
      }
    }
  }
  __syncthreads();
  // lower triangle: row tj*HT + bb, columns i0 + aa (contiguous in aa)
  for (int e = t; e < RS * HT; e += 256) {
    const int bb = e / RS, aa = e % RS;
    const int r = tj * HT + bb, c = i0 + aa;
    if (r < d && c < d && c < r) H[(int64_t)r * d + c] = T[aa][bb];
  }
}

}  // namespace

namespace {

constexpr int kCUs = 256;  // MI355X compute units (one fast-path workgroup each)

// Splits for the generic 128-tile kernel and the fp32 path.
int generic_splits(int64_t d, int64_t n_tok) {
  const int64_t nt = ceil_div(d, HT);
  const int64_t tiles = nt * (nt + 1) / 2;
  int64_t s = ceil_div(2048, tiles);
  s = std::min<int64_t>(s, 32);
  s = std::min<int64_t>(s, std::max<int64_t>(1, ceil_div(n_tok, 256)));
  s = std::max<int64_t>(s, 1);
  const int64_t chunk = ceil_div(ceil_div(std::max<int64_t>(n_tok, 1), s), HK) * HK;
  return (int)ceil_div(std::max<int64_t>(n_tok, 1), chunk);
}

// Splits for the 256-tile kernel: minimise the modelled time of
// ceil(tiles·S / CUs) rounds of 1/S of a tile's work, plus writing and
// reading S partial Hessians.
int fast_splits(int64_t d, int64_t n_tok) {
  const int64_t nt = ceil_div(d, FT);
  const double tiles = (double)(nt * (nt + 1) / 2);
  const double dp = (double)(nt * FT);
  const double t_tile = 2.0 * FT * FT * (double)n_tok / (1.5e15 / kCUs);
  const double t_byte = 1.0 / 8e12;
  int best = 1;
  double best_t = 1e300;
  for (int S = 1; S <= 32; ++S) {
    if (S > 1 && ceil_div(n_tok, S) < 4 * FK) break;
    const double rounds = std::ceil(tiles * S / kCUs);
    const double t = rounds * t_tile / S + 2.0 * S * dp * dp * 4 * t_byte;
    if (t < best_t * 0.98) { best_t = t; best = S; }
  }
  const int64_t chunk = ceil_div(ceil_div(n_tok, best), FK) * FK;
  return (int)ceil_div(n_tok, chunk);
}



}  // namespace

int hessian_splits(int64_t d, int64_t n_tok) { return fast_splits(d, n_tok); }

size_t hessian_ws_bytes(int64_t d, int64_t n_tok) {
  const int64_t dpg = ceil_div(d, FT) * FT;
  const size_t fast = (size_t)(fast_splits(d, n_tok) + 1) * dpg * dpg * sizeof(float);   // + mixed plan's
  const size_t gen = (size_t)generic_splits(d, n_tok) * dpg * dpg * sizeof(float);
  // partials, then the shift μ (dp 16-bit values), then a 256-byte zero
  // chunk (source of out-of-range copies)
  return align_up(std::max<size_t>(std::max(fast, gen), 256)) + align_up((size_t)dpg * 2) + 256;
}

size_t hessian_min_ws_bytes(int64_t d) {
  const int64_t dp = ceil_div(d, FT) * FT;
  return (size_t)dp * dp * 4 + align_up((size_t)dp * 2) + 256;
}

// Workspace layout: S partial Hessians (S as the path wants, at most what
// ws_bytes holds), then μ (dp 16-bit values), then the 256-byte zero chunk.
hipError_t hessian_launch(float* H, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                          int64_t ld_x, void* ws, size_t ws_bytes, hipStream_t s, bool overwrite) {
  if (n_tok <= 0) {
    if (overwrite) {   // H = 2·XᵀX over no tokens: zeros (a fill kernel, no memset)
      fill_zero_kernel<<<(unsigned)std::min<int64_t>(ceil_div(d * d, 1024), 4096), 256, 0, s>>>(H, d * d);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  const int64_t dp = ceil_div(d, FT) * FT;   // partial Hessians are dp x dp
  float* P = static_cast<float*>(ws);
  const size_t part = (size_t)dp * dp * 4;
  const int fit = (int)std::min<size_t>(64, (ws_bytes - align_up((size_t)dp * 2) - 256) / part);
  hipError_t e;
  const bool fast = x_dtype != GPTQ_F32 && d % 8 == 0 && ld_x % 8 == 0 && (uintptr_t)X % 16 == 0;
  // splits: the path's choice, capped by the workspace; the token chunk of
  // each split is a whole number of stages
  const int want = fast ? fast_splits(d, n_tok) : generic_splits(d, n_tok);
  const int step = fast ? FK : HK;
  const int64_t chunk = ceil_div(ceil_div(n_tok, std::min(want, fit)), step) * step;
  const int splits = (int)ceil_div(n_tok, chunk);
  SplitPlan plan{chunk, chunk, splits, 0, 0, 0, 0};
  if (fast && fit > splits) plan = mixed_plan(d, n_tok, splits, chunk, FT, FK, kCUs);
  const int nslots = plan.hi_tiles > 0 ? splits + 1 : splits;   // partial Hessians written
  uint16_t* mu = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + align_up(part * nslots));
  uint16_t* zero16 = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(mu) + align_up((size_t)dp * 2));
  const bool bf = x_dtype == GPTQ_BF16;
  double shift_tok = 0.0;   // tokens' worth of μμᵀ the shift MFMAs took out
  ReducePlan rp{splits, 0, 0, 0.0, 0.0};
  if (x_dtype != GPTQ_F32) {
    const int n0 = (int)std::min<int64_t>(n_tok, kShiftSample);
    const int vec = ((uintptr_t)X % 16 == 0) && (ld_x % 8 == 0);
    const unsigned gm = (unsigned)ceil_div(dp, 16);
    if (bf) shift_mean_kernel<true><<<gm, 256, 0, s>>>(static_cast<const uint16_t*>(X), ld_x, (int)d,
                                                        (int)dp, n0, vec, mu);
    else shift_mean_kernel<false><<<gm, 256, 0, s>>>(static_cast<const uint16_t*>(X), ld_x, (int)d,
                                                      (int)dp, n0, vec, mu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (fast) {
    const int nt = (int)ceil_div(d, FT);
    const int tiles = nt * (nt + 1) / 2;
    const unsigned grid = (unsigned)(plan.hi_tiles > 0
                                         ? (tiles - plan.hi_tiles) * splits + plan.hi_tiles * (splits + 1)
                                         : tiles * splits);
    shift_tok = shift_count(n_tok, chunk, splits, FK, kShiftTok);
    if (plan.hi_tiles > 0) {
      rp.ng_hi = nt / 4;
      rp.hi_mask = plan.hi_mask;
      rp.shift_hi = shift_count(n_tok, plan.chunk_hi, splits + 1, FK, kShiftTok);
    }
    zero_chunk_kernel<<<1, 64, 0, s>>>(reinterpret_cast<uint32_t*>(zero16));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (x_dtype == GPTQ_BF16)
      syrk256_kernel<true><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(X), ld_x, (int)d, n_tok,
                                                plan, nt, P, dp, zero16, mu);
    else
      syrk256_kernel<false><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(X), ld_x, (int)d,
                                                 n_tok, plan, nt, P, dp, zero16, mu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    const int nt = (int)ceil_div(d, HT);
    const int tiles = nt * (nt + 1) / 2;
    if (x_dtype == GPTQ_F32) {
      GemmArgs g{};
      g.M = (int)d; g.N = (int)d;
      g.K = (int)chunk; g.k_last = (int)(n_tok - (int64_t)(splits - 1) * chunk);
      g.batch = splits; g.alpha = 1.f; g.beta = 0.f;
      g.A = static_cast<const float*>(X); g.lda = ld_x; g.strideA = chunk * ld_x; g.trans_a = true;
      g.B = static_cast<const float*>(X); g.ldb = ld_x; g.strideB = chunk * ld_x; g.trans_b = false;
      g.C = P; g.ldc = dp; g.strideC = dp * dp; g.tri = 2;
      if ((e = gemm_f32(g, s)) != hipSuccess) return e;
    } else {
      const int vec = ((uintptr_t)X % 16 == 0) && (ld_x % 8 == 0);
      dim3 grid(tiles, splits);
      for (int sp = 0; sp < splits; ++sp) {   // shift MFMAs per split: one per 8 stages
        const int64_t rows = std::min<int64_t>(n_tok, (sp + 1) * chunk) - sp * chunk;
        shift_tok += (double)(ceil_div(rows, HK) / (kShiftTok / HK)) * kShiftTok;
      }
      if (x_dtype == GPTQ_BF16)
        syrk16_generic_kernel<true><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(X), ld_x, (int)d,
                                                         n_tok, chunk, nt, P, dp, vec, mu);
      else
        syrk16_generic_kernel<false><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(X), ld_x, (int)d,
                                                          n_tok, chunk, nt, P, dp, vec, mu);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  const int nt128 = (int)(dp / HT);
  const int vec_h = ((uintptr_t)H % 16 == 0) && (d % 4 == 0);
  const unsigned gr = (unsigned)(4 * nt128 * (nt128 + 1) / 2);   // four strips per tile
  const uint16_t* mu_r = x_dtype == GPTQ_F32 ? nullptr : mu;
  rp.shift_lo = shift_tok;
  if (bf || x_dtype == GPTQ_F32)
    reduce_mirror_kernel<true><<<gr, 256, 0, s>>>(H, (int)d, P, dp, rp, nt128, vec_h, mu_r,
                                                  overwrite ? 0 : 1);
  else
    reduce_mirror_kernel<false><<<gr, 256, 0, s>>>(H, (int)d, P, dp, rp, nt128, vec_h, mu_r,
                                                   overwrite ? 0 : 1);
  return hipGetLastError();
}

// ---------------------------------------------------------------- no-allocation variant
// A workspace in the library's own device memory: a file-scope array that
// every GPU the library runs on holds until the process ends.  In host code
// its name stands for a host-side shadow, not a device address, so the
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is passed to kernels.  Every
// call on one GPU uses the same array: calls that overlap on one GPU race.
// What must start at zero (the zero chunk) is written by a fill kernel on
// every call; the partials and μ are fully written before they are read.
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_for_device(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t hessian_launch_static(float* H, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                                 int64_t ld_x, hipStream_t s) {
  if (hessian_min_ws_bytes(d) > kScratchBytes) return hipErrorInvalidValue;
  if (n_tok <= 0) return hipSuccess;
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  void* ws = nullptr;
  if ((e = scratch_for_device(dev, &ws)) != hipSuccess) return e;
  return hessian_launch(H, d, X, x_dtype, n_tok, ld_x, ws, kScratchBytes, s);
}

}  // namespace gq
