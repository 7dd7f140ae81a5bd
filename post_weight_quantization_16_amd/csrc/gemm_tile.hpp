// fp32 MFMA GEMM tile for gfx950, shared by the stand-alone GEMM kernel and
// the fused Cholesky step of the preparation.
//
// Square T x T output tile (T = 128 or 64) per workgroup of 256 threads:
// 4 waves in a 2x2 grid, each wave (T/2)x(T/2) = (T/64)^2 tiles of
// v_mfma_f32_32x32x2f32, whose operands are one float per lane:
// A(m = lane%32, k = lane/32) and B(k = lane/32, n = lane%32).
// K advances in chunks of 32 through a double-buffered LDS stage: the next
// chunk is fetched into registers while the current one is multiplied, then
// stored into the other buffer; one barrier per chunk.  Each operand is kept
// in LDS in its memory orientation:
//   contiguous along m (or n): [k][T + 32] -- a half-wave reads 32
//     consecutive words, the other half-wave's row is 32 banks away;
//   contiguous along k: [m][32 + 2] -- the odd-pair stride 34 sends the 32
//     rows a half-wave reads to 32 distinct banks.
// T = 128 takes 80 KB of LDS (two workgroups per CU); T = 64 serves
// products whose 128-tiles would not fill the chip or whose K is long and
// uneven across tiles.
#pragma once

#include "common.hpp"

namespace gq {
namespace gemm_detail {

constexpr int TK = 32;
template <int T> struct Tile {
  static constexpr int SA = T + 32;   // stride of a [k][T] operand (floats)
  static constexpr int SK = TK + 2;   // stride of a [T][k] operand (floats)
  static constexpr int OPF = TK * SA > T * SK ? TK * SA : T * SK;   // floats per operand buffer
  static constexpr int NV = TK * T / (256 * 4);                       // float4 per thread per chunk
  static constexpr int ES = T + 8;    // epilogue stride: 4·ES ≡ 32 (mod 64), half-waves' rows disjoint
  static constexpr int FI = T / 64;   // MFMA tiles per wave along each edge
  static_assert(T * ES <= 4 * OPF, "the epilogue tile must fit in the operand buffers");
};
constexpr int GEMM_SMEM_FLOATS = 4 * Tile<128>::OPF;   // enough for either tile size
static_assert(4 * Tile<64>::OPF <= GEMM_SMEM_FLOATS, "");
// the 128 tile is used by callers that name these
constexpr int TM = 128, TN = 128;

struct KArgs {
  int M, N, K, k_last;
  int k_from_n, k_to_m;
  float alpha, beta;
  const float* A; int64_t lda, strideA;
  const float* B; int64_t ldb, strideB;
  float* C; int64_t ldc, strideC;
  int tri;
  int vec_a, vec_b, vec_c;
};

// One 32 x T operand chunk in registers: NV float4 per thread.
// ALONG: the T-wide dimension is contiguous in memory; otherwise k is.
template <int T, bool ALONG>
__device__ __forceinline__ void load_chunk(const float* __restrict__ p, int64_t ld, int rows_valid,
                                           int k0, int kvalid, int t, bool vec,
                                           f32x4 (&r)[Tile<T>::NV]) {
#pragma unroll
  for (int i = 0; i < Tile<T>::NV; ++i) {
    const int idx = t + 256 * i;
    int a, b;  // a: index along the T-wide dim, b: k
    if (ALONG) { b = idx / (T / 4); a = (idx % (T / 4)) * 4; }
    else       { a = idx >> 3; b = (idx & 7) * 4; }
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

template <int T, bool ALONG>
__device__ __forceinline__ void store_chunk(float* __restrict__ s, int t,
                                            const f32x4 (&r)[Tile<T>::NV]) {
#pragma unroll
  for (int i = 0; i < Tile<T>::NV; ++i) {
    const int idx = t + 256 * i;
    if (ALONG) {
      const int b = idx / (T / 4), a = (idx % (T / 4)) * 4;
      *reinterpret_cast<f32x4*>(s + b * Tile<T>::SA + a) = r[i];
    } else {
      const int a = idx >> 3, b = (idx & 7) * 4;
      typedef __attribute__((ext_vector_type(2))) float f32x2;
      f32x2 lo = {r[i][0], r[i][1]}, hi = {r[i][2], r[i][3]};
      *reinterpret_cast<f32x2*>(s + a * Tile<T>::SK + b) = lo;
      *reinterpret_cast<f32x2*>(s + a * Tile<T>::SK + b + 2) = hi;
    }
  }
}

template <int T, bool ALONG>
__device__ __forceinline__ float opread(const float* s, int a, int k) {
  return ALONG ? s[k * Tile<T>::SA + a] : s[a * Tile<T>::SK + k];
}

// Whether the tile (m0, n0) takes the vector epilogue (in range, float4 C).
template <int T>
__device__ __forceinline__ bool c_vec(const KArgs& g, int m0, int n0) {
  return g.M - m0 >= T && g.N - n0 >= T && g.vec_c;
}
// This thread's float4 share of a vector-epilogue tile of C (issued early by
// callers that can hide the read).
template <int T>
__device__ __forceinline__ void load_c(const KArgs& g, const float* C, int m0, int n0, int t,
                                       f32x4 (&cv)[T * T / 1024]) {
#pragma unroll
  for (int u = 0; u < T * T / 1024; ++u) {
    const int idx = t + 256 * u, row = idx / (T / 4), c4 = (idx % (T / 4)) * 4;
    cv[u] = *reinterpret_cast<const f32x4*>(C + (int64_t)(m0 + row) * g.ldc + n0 + c4);
  }
}

// C[m0.., n0..] = E + beta·C for one T x T tile staged in LDS (row stride
// ES), honouring the edges and the triangle mask (tri 1: lower, 2: upper).
// All of a thread's C reads are issued before any of its writes: C is read
// and written through one pointer, so a read placed after a write would
// wait for that write's full round trip.  In-range tiles move float4; their
// C values come in cv when the caller loaded them already (have_c).  Where
// the triangle crosses an in-range tile and C was read, the elements outside
// it are stored back unchanged; with beta = 0 a float4 straddling the
// diagonal is written element by element.
template <int T, int ES>
__device__ __forceinline__ void store_tile(const KArgs& g, const float* E, float* C, int m0,
                                           int n0, int t, f32x4 (&cv)[T * T / 1024],
                                           bool have_c) {
  const bool has_beta = g.beta != 0.f;
  const int mvalid = g.M - m0, nvalid = g.N - n0;
  if (c_vec<T>(g, m0, n0)) {
    constexpr int NE = T * T / 1024;
    if (has_beta && !have_c) load_c<T>(g, C, m0, n0, t, cv);
    // a tile the triangle mask keeps whole: straight-line float4 stores
    // (the per-element checks below cost more than the stores themselves)
    const bool whole = g.tri == 0 || (g.tri == 1 && n0 + T - 1 <= m0) ||
                       (g.tri == 2 && n0 >= m0 + T - 1);
    if (whole) {
      const float beta = g.beta;
      if (has_beta) {
#pragma unroll
        for (int u = 0; u < NE; ++u) {
          const int idx = t + 256 * u, row = idx / (T / 4), c4 = (idx % (T / 4)) * 4;
          f32x4 v = *reinterpret_cast<const f32x4*>(E + row * ES + c4);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = fmaf(beta, cv[u][q], v[q]);
          *reinterpret_cast<f32x4*>(C + (int64_t)(m0 + row) * g.ldc + n0 + c4) = v;
        }
      } else {
#pragma unroll
        for (int u = 0; u < NE; ++u) {
          const int idx = t + 256 * u, row = idx / (T / 4), c4 = (idx % (T / 4)) * 4;
          *reinterpret_cast<f32x4*>(C + (int64_t)(m0 + row) * g.ldc + n0 + c4) =
              *reinterpret_cast<const f32x4*>(E + row * ES + c4);
        }
      }
      return;
    }
    if (has_beta) {
      // a tile the triangle crosses: elements outside it are written back
      // unchanged from cv (they belong to this tile alone), so every store
      // is a whole float4 and needs no branch
      const float beta = g.beta;
#pragma unroll
      for (int u = 0; u < NE; ++u) {
        const int idx = t + 256 * u, row = idx / (T / 4), c4 = (idx % (T / 4)) * 4;
        f32x4 v = *reinterpret_cast<const f32x4*>(E + row * ES + c4);
        const int gr = m0 + row, gc = n0 + c4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool keep = g.tri == 1 ? gc + q <= gr : gc + q >= gr;
          v[q] = keep ? fmaf(beta, cv[u][q], v[q]) : cv[u][q];
        }
        *reinterpret_cast<f32x4*>(C + (int64_t)gr * g.ldc + gc) = v;
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int idx = t + 256 * u, row = idx / (T / 4), c4 = (idx % (T / 4)) * 4;
      f32x4 v = *reinterpret_cast<const f32x4*>(E + row * ES + c4);
      if (has_beta) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = fmaf(g.beta, cv[u][q], v[q]);
      }
      float* dst = C + (int64_t)(m0 + row) * g.ldc + n0 + c4;
      const int gr = m0 + row, gc = n0 + c4;
      const bool all = g.tri == 0 || (g.tri == 1 && gc + 3 <= gr) || (g.tri == 2 && gc >= gr);
      if (all) {
        *reinterpret_cast<f32x4*>(dst) = v;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (g.tri == 1 ? gc + q <= gr : gc + q >= gr) dst[q] = v[q];
      }
    }
  } else {
    // edge tile: element-wise, every read (at a clamped, valid address)
    // issued before the masked writes
    constexpr int NE = T * T / 256;
    float cs[NE];
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = t + 256 * u, row = e / T, col = e % T;
      const int rr = min(row, mvalid - 1), cc = min(col, nvalid - 1);
      cs[u] = has_beta ? C[(int64_t)(m0 + rr) * g.ldc + n0 + cc] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = t + 256 * u, row = e / T, col = e % T;
      const int gr = m0 + row, gc = n0 + col;
      bool ok = row < mvalid && col < nvalid;
      if (g.tri == 1) ok = ok && gc <= gr;
      if (g.tri == 2) ok = ok && gc >= gr;
      if (ok) C[(int64_t)gr * g.ldc + gc] = fmaf(g.beta, cs[u], E[row * ES + col]);
    }
  }
}

// One T x T output tile (bx, by) of batch z; nz = number of batches.
// Sm: GEMM_SMEM_FLOATS floats of LDS.  All 256 threads of the workgroup
// must call it (it synchronizes).
template <int T, bool TA, bool TB>
__device__ __forceinline__ void gemm_tile(const KArgs& g, int bx, int by, int z, int nz,
                                          float* __restrict__ Sm) {
  using TL = Tile<T>;
  constexpr int OPF = TL::OPF, FI = TL::FI, WT = T / 2;
  const int m0 = by * T, n0 = bx * T;
  if (g.tri == 1 && n0 > m0 + T - 1) return;
  if (g.tri == 2 && n0 + T - 1 < m0) return;
  const int Kz = (z == nz - 1) ? g.k_last : g.K;
  const int kbeg = g.k_from_n ? (n0 / TK) * TK : 0;
  const int K = g.k_to_m ? min(Kz, m0 + T) : Kz;
  const float* A = g.A + (int64_t)z * g.strideA;
  const float* B = g.B + (int64_t)z * g.strideB;
  float* C = g.C + (int64_t)z * g.strideC;

  // A: op(A)(m,k); TA: stored [K x M] (m contiguous) -> ALONG.  B: TB stored [N x K].
  constexpr bool AL_A = TA, AL_B = !TB;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const float* Ab = TA ? A + m0 : A + (int64_t)m0 * g.lda;
  const float* Bb = TB ? B + (int64_t)n0 * g.ldb : B + n0;
  const int mvalid = g.M - m0, nvalid = g.N - n0;

  f32x16 acc[FI][FI];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  f32x4 ra[TL::NV], rb[TL::NV];
  if (kbeg < K) {
    load_chunk<T, AL_A>(Ab, g.lda, mvalid, kbeg, K, t, g.vec_a, ra);
    load_chunk<T, AL_B>(Bb, g.ldb, nvalid, kbeg, K, t, g.vec_b, rb);
    store_chunk<T, AL_A>(Sm + 0 * OPF, t, ra);
    store_chunk<T, AL_B>(Sm + 1 * OPF, t, rb);
  }
  __syncthreads();

  int buf = 0;
  for (int k0 = kbeg; k0 < K; k0 += TK) {
    const bool more = k0 + TK < K;
    if (more) {
      load_chunk<T, AL_A>(Ab, g.lda, mvalid, k0 + TK, K, t, g.vec_a, ra);
      load_chunk<T, AL_B>(Bb, g.ldb, nvalid, k0 + TK, K, t, g.vec_b, rb);
    }
    const float* As = Sm + (2 * buf + 0) * OPF;
    const float* Bs = Sm + (2 * buf + 1) * OPF;
#pragma unroll
    for (int kk = 0; kk < TK / 2; ++kk) {
      const int ka = kk * 2 + (lane >> 5);
      float av[FI], bv[FI];
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        av[i] = opread<T, AL_A>(As, wm * WT + i * 32 + (lane & 31), ka);
        bv[i] = opread<T, AL_B>(Bs, wn * WT + i * 32 + (lane & 31), ka);
      }
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_chunk<T, AL_A>(Sm + (2 * (buf ^ 1) + 0) * OPF, t, ra);
      store_chunk<T, AL_B>(Sm + (2 * (buf ^ 1) + 1) * OPF, t, rb);
    }
    __syncthreads();
    buf ^= 1;
  }

  // Epilogue through LDS (the operand buffers are free after the loop's last
  // barrier): the tile goes to LDS as alpha·acc, then is merged into C.
  // MFMA layout: lane holds rows (r/4)*8 + (lane/32)*4 + r%4, column lane%32.
  float* E = Sm;
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * WT + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = wn * WT + j * 32 + (lane & 31);
        E[row * TL::ES + col] = g.alpha * acc[i][j][r];
      }
  __syncthreads();
  f32x4 cv[T * T / 1024];
  store_tile<T, TL::ES>(g, E, C, m0, n0, t, cv, false);
}

// Kernel arguments for a host-side GemmArgs (vector-load eligibility included).
KArgs make_kargs(const GemmArgs& a);

}  // namespace gemm_detail
}  // namespace gq
