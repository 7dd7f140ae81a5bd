// fp32 MFMA GEMM tile for gfx950 whose operands go from memory straight into
// an LDS ring (global_load_lds_dwordx4), used by the stand-alone GEMM kernel
// and by the fused Cholesky step when the shapes allow it (see dma_ok).
//
// Output tile T x T (T = 128 or 64) per workgroup of 256 threads: 4 waves in
// a 2x2 grid, each (T/2)x(T/2) as (T/64)^2 tiles of v_mfma_f32_32x32x2f32.
// K advances in stages of 16.  Stage s lives in ring buffer s % NS and is
// copied NS−1 stages ahead: no registers hold operands in flight and no LDS
// store instructions run.  A wave waits (s_waitcnt vmcnt) for its own copies
// of the stage it will read next, and one barrier per stage publishes every
// wave's copies and frees the buffer just read for the next copy.
//
// MFMA k-slots: the instruction contracts two k values, taken by lanes 0-31
// and 32-63.  Any assignment of actual k to (step, slot) gives the same
// product if A and B agree on it; here lanes 32-63 take the upper half of
// the stage (step kk: k = kk for lanes 0-31, k = 8 + kk for lanes 32-63),
// so a lane's 8 values of one row are contiguous.
//
// LDS layouts, per operand and stage (16-byte pieces, XOR-swizzled on the
// global side: a lane of the copy fetches the piece its LDS slot holds):
//   k-contiguous operand (row-major A, transposed B): [T rows][16 k],
//     64 bytes a row; piece p of row r sits in slot p ^ ((r >> 2) & 3), so a
//     lane reads its 8 values with two ds_read_b128 and any 16 consecutive
//     rows cover all 64 banks;
//   T-contiguous operand (transposed A, row-major B): [16 k][T], piece p of
//     k-row k in slot p ^ (8·((k >> 3) & 1)), so the two half-waves (k and
//     k + 8) read banks 32 apart with ds_read_b32.
// Edges: rows and columns past the matrix fetch a clamped in-range piece
// (their outputs are never written); K must be a multiple of 16, a
// T-contiguous operand's T extent a multiple of 4, and every operand 16-byte
// aligned with a leading dimension that is a multiple of 4 (dma_ok).
// The copies are inline asm: with the builtin the compiler cannot tell which
// ring buffer a copy writes and waits for all of them before each LDS read.
#pragma once

#include "gemm_tile.hpp"

namespace gq {
namespace gemm_detail {

constexpr int DK = 16;   // k per stage

template <int T, int NS> struct DTile {
  static constexpr int OPB = T * DK * 4;             // bytes per operand per stage
  static constexpr int SB = 2 * OPB;                 // bytes per stage
  static constexpr int NWI = T / 64;                 // copy instructions per wave per operand and stage
  static constexpr int NW = 2 * NWI;                 // per wave per stage
  static constexpr int ES = T + 8;                   // epilogue stride (floats)
  static constexpr int RING = NS * SB;
  static constexpr int EPI = T * ES * 4;
  static constexpr int SMEM = RING > EPI ? RING : EPI;   // bytes
  static_assert(NS >= 2 && NS <= 8 && (NS - 2) * NW <= 63, "vmcnt range");
};

// Shapes the DMA tile handles (otherwise the register-staged tile runs).
inline bool dma_ok(const KArgs& k, bool ta, bool tb) {
  if (k.K % DK != 0 || k.k_last % DK != 0) return false;
  if (!k.vec_a || !k.vec_b || !k.vec_c) return false;
  if (ta && k.M % 4 != 0) return false;    // A stored [K][M]
  if (!tb && k.N % 4 != 0) return false;   // B stored [K][N]
  return true;
}

// s_waitcnt immediate: vmcnt(n) (bits [3:0] and [15:14]) and lgkmcnt(0)
constexpr int vmcnt_imm(int n) { return ((n >> 4) << 14) | (n & 15) | 0x70; }

// s_waitcnt vmcnt(ahead·NW) with lgkmcnt(0): every copy but those of the
// last `ahead` stages issued has landed (loads complete in issue order)
template <int NW>
__device__ __forceinline__ void wait_stages(int ahead) {
  switch (ahead) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) ); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(NW) ); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NW) ); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * NW) ); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * NW) ); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * NW) ); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * NW) ); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) ); break;
  }
}

// Copy plan of one operand for this lane: source of each of the wave's
// copy instructions at stage 0, and the per-stage advance.
template <int T, bool KCONT>
struct OpCopy {
  const char* src[DTile<T, 2>::NWI];
  int64_t step;   // bytes per stage
  __device__ __forceinline__ void init(const float* base, int64_t ld, int valid, int kbeg, int w,
                                       int lane) {
    constexpr int NWI = DTile<T, 2>::NWI;
#pragma unroll
    for (int j = 0; j < NWI; ++j) {
      const int i = w * NWI + j;   // 1-KB segment of the operand's stage buffer
      if (KCONT) {
        const int rr = 16 * i + (lane >> 2);
        const int gp = (lane & 3) ^ ((rr >> 2) & 3);
        const int r = min(rr, valid - 1);
        src[j] = reinterpret_cast<const char*>(base + (int64_t)r * ld + kbeg + 4 * gp);
      } else {
        constexpr int RPI = 256 / T;   // k-rows per segment
        const int kr = RPI * i + lane / (T / 4);
        int gp = (lane % (T / 4)) ^ (((kr >> 3) & 1) << 3);
        gp = min(gp, valid / 4 - 1);
        src[j] = reinterpret_cast<const char*>(base + (int64_t)(kbeg + kr) * ld + 4 * gp);
      }
    }
    step = KCONT ? DK * 4 : (int64_t)DK * ld * 4;
  }
  __device__ __forceinline__ void issue(unsigned lds, int st, int w) const {
    constexpr int NWI = DTile<T, 2>::NWI;
#pragma unroll
    for (int j = 0; j < NWI; ++j) {
      const char* a = src[j] + (int64_t)st * step;
      // 16 bytes per lane from a to LDS M0 + 16·lane; no register result,
      // ordered before the reads by the stage waits
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(lds + (unsigned)(w * NWI + j) * 1024u), "v"(a) : "memory");
    }
  }
};

// Four of a lane's 8 k values (half hf: k = 8·(lane/32) + 4·hf + 0..3) of
// rows (or columns) base + i·32 + lane%32, i < FI, from one operand's stage
// buffer.
template <int T, bool KCONT, int FI>
__device__ __forceinline__ void read_half(const char* S, int base, int lane, int hf,
                                          float (&v)[FI][4]) {
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const int r = base + i * 32 + (lane & 31);
    if (KCONT) {
      const int sw = (r >> 2) & 3;
      const f32x4 x = *reinterpret_cast<const f32x4*>(S + r * 64 + (((2 * h + hf) ^ sw) << 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) v[i][q] = x[q];
    } else {
      const int off = ((((r >> 2) ^ (8 * h)) << 4)) + ((r & 3) << 2);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        v[i][kk] = *reinterpret_cast<const float*>(S + (8 * h + 4 * hf + kk) * (T * 4) + off);
    }
  }
}

// One T x T output tile (bx, by) of batch z; nz = number of batches.
// Sm: DTile<T, NS>::SMEM bytes of LDS, 1-KB aligned.  All 256 threads of
// the workgroup call it (it synchronizes).  The caller has checked dma_ok.
template <int T, int NS, bool TA, bool TB>
__device__ __forceinline__ void gemm_tile_dma(const KArgs& g, int bx, int by, int z, int nz,
                                              char* __restrict__ Sm) {
  using DT = DTile<T, NS>;
  constexpr int FI = T / 64, WT = T / 2, NW = DT::NW;
  constexpr bool KA = !TA, KB = TB;   // k-contiguous operands
  const int m0 = by * T, n0 = bx * T;
  if (m0 >= g.M || n0 >= g.N) return;   // a sub-tile wholly past the edge
  if (g.tri == 1 && n0 > m0 + T - 1) return;
  if (g.tri == 2 && n0 + T - 1 < m0) return;
  const int Kz = (z == nz - 1) ? g.k_last : g.K;
  const int kbeg = g.k_from_n ? (n0 / DK) * DK : 0;
  const int K = g.k_to_m ? min(Kz, m0 + T) : Kz;
  const int nst = K > kbeg ? (K - kbeg) / DK : 0;
  const float* A = g.A + (int64_t)z * g.strideA;
  const float* B = g.B + (int64_t)z * g.strideB;
  float* C = g.C + (int64_t)z * g.strideC;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int mvalid = g.M - m0, nvalid = g.N - n0;

  OpCopy<T, KA> ca;
  OpCopy<T, KB> cb;
  ca.init(KA ? A + (int64_t)m0 * g.lda : A + m0, g.lda, mvalid, kbeg, w, lane);
  cb.init(KB ? B + (int64_t)n0 * g.ldb : B + n0, g.ldb, nvalid, kbeg, w, lane);
  const unsigned sbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)Sm;
  auto copy = [&](int st) {
    const unsigned lb = sbase + (unsigned)((st % NS) * DT::SB);
    ca.issue(lb, st, w);
    cb.issue(lb + DT::OPB, st, w);
  };

  f32x16 acc[FI][FI];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // C's share of a vector-epilogue tile is read first: it arrives with the
  // first stage instead of after the K loop (loads complete in issue order,
  // so the stage waits below cover it)
  f32x4 cv[T * T / 1024];
  const bool early_c = g.beta != 0.f && c_vec<T>(g, m0, n0);
  if (early_c) load_c<T>(g, C, m0, n0, t, cv);
  for (int s0 = 0; s0 < NS - 1 && s0 < nst; ++s0) copy(s0);
  wait_stages<NW>(min(nst - 1, NS - 2));
  __syncthreads();
  // Each stage is two halves of 4 k: the second half of stage st is
  // multiplied after the barrier, while the first half of stage st+1 is
  // read, so the MFMAs do not start each stage waiting for LDS.
  float al[FI][4], bl[FI][4], ah[FI][4], bh[FI][4];
  auto mfma4 = [&](const float (&av)[FI][4], const float (&bv)[FI][4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][kk], bv[j][kk], acc[i][j], 0, 0, 0);
  };
  if (nst > 0) {
    read_half<T, KA, FI>(Sm, wm * WT, lane, 0, al);
    read_half<T, KB, FI>(Sm + DT::OPB, wn * WT, lane, 0, bl);
  }
  for (int st = 0; st < nst; ++st) {
    if (st + NS - 1 < nst) copy(st + NS - 1);   // into the buffer the last barrier freed
    const char* SA = Sm + (st % NS) * DT::SB;
    read_half<T, KA, FI>(SA, wm * WT, lane, 1, ah);
    read_half<T, KB, FI>(SA + DT::OPB, wn * WT, lane, 1, bh);
    mfma4(al, bl);
    // stage st+1 copied (later stages may stay in flight) and this wave's
    // reads of stage st done before the barrier frees its buffer
    wait_stages<NW>(min(nst - 1, st + NS - 1) - (st + 1));
    __syncthreads();
    if (st + 1 < nst) {
      const char* SN = Sm + ((st + 1) % NS) * DT::SB;
      read_half<T, KA, FI>(SN, wm * WT, lane, 0, al);
      read_half<T, KB, FI>(SN + DT::OPB, wn * WT, lane, 0, bl);
    }
    mfma4(ah, bh);
  }

  // Epilogue through LDS, as in the register-staged tile.
  float* E = reinterpret_cast<float*>(Sm);
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * WT + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = wn * WT + j * 32 + (lane & 31);
        E[row * DT::ES + col] = g.alpha * acc[i][j][r];
      }
  __syncthreads();
  store_tile<T, DT::ES>(g, E, C, m0, n0, t, cv, early_c);
}

}  // namespace gemm_detail
}  // namespace gq
