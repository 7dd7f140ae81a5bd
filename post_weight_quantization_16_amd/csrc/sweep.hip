// One 128-column block of the GPTQ column sweep ("GPTQ: Mathematical
// Foundations ...": The GPTQ Algorithmic Innovations 2-3 -- in-block updates
// and the Cholesky form of the compensation; walkthrough step 3; "INT4 and
// GPTQ Quantization": Uniform INT4 Quantization, Group Quantization).
//
// This file is compiled once per group-size variant (-DGQ_SWEEP_G=0/32/64/128)
// so the heavily unrolled variants build in parallel.
//
// Layout: one 16-lane DPP row per weight row; lane c holds the row's block
// columns 4c..4c+3 and 64+4c..64+4c+3 in registers (so the lanes of a row
// read one contiguous 256-byte span of a U row per half), a wave covers 4
// rows, a workgroup 4·W rows.  The block's 128x128 part of U and 1/U_jj are
// staged in LDS once per workgroup.  For each column j of the block:
//   w_j is broadcast inside the row from its owner lane (DPP row_newbcast),
//   at a group start the row reduces the group's current min/max (DPP),
//   v = w_j·(1/s) + z;  q = clamp(rint(v), 0, 2ᵇ−1);  ŵ = s(q − z)
//   err = (w_j − ŵ)·(1/U_jj);  every lane: w_k −= err·U_jk for its 8 columns
// (U is upper triangular, so columns left of j receive zeros and the update
// needs no per-lane bounds); the owner lane then keeps ŵ, err and q in the
// column's register slots, and the block is written back coalesced from the
// registers.  Every lane of a row computes the same v, q, ŵ and err.  The
// working copy is padded to whole blocks: padded columns hold 0 and their U
// rows/columns are 0 with a unit diagonal, so they quantize to 0 with err 0.
#include "common.hpp"

#ifndef GQ_SWEEP_G
#error "compile with -DGQ_SWEEP_G=<group size handled in registers, 0 = external>"
#endif

namespace gq {
namespace {

constexpr int QC = kBlock / 16;   // columns per lane
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// lane o of each 16-lane row to the whole row; o is a constant once the
// column loop is unrolled, so the switch folds away
__device__ __forceinline__ float row_bcast(float x, int o) {
  switch (o) {
    case 0: return dpp<0x150>(x);  case 1: return dpp<0x151>(x);
    case 2: return dpp<0x152>(x);  case 3: return dpp<0x153>(x);
    case 4: return dpp<0x154>(x);  case 5: return dpp<0x155>(x);
    case 6: return dpp<0x156>(x);  case 7: return dpp<0x157>(x);
    case 8: return dpp<0x158>(x);  case 9: return dpp<0x159>(x);
    case 10: return dpp<0x15A>(x); case 11: return dpp<0x15B>(x);
    case 12: return dpp<0x15C>(x); case 13: return dpp<0x15D>(x);
    case 14: return dpp<0x15E>(x); default: return dpp<0x15F>(x);
  }
}
// reductions over a 16-lane row: quad_perm [1,0,3,2], [2,3,0,1], then
// row_half_mirror and row_mirror; every lane ends with the row's result
__device__ __forceinline__ float row_min(float x) {
  x = fminf(x, dpp<0xB1>(x));
  x = fminf(x, dpp<0x4E>(x));
  x = fminf(x, dpp<0x141>(x));
  return fminf(x, dpp<0x140>(x));
}
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  return fmaxf(x, dpp<0x140>(x));
}

// One column's quantization: q = clamp(rint(w/s + z)) with 1/s as rs, and
// x = w − s(q − z) rounded once, so err = x·(1/U_jj).  Written out so the
// column loop and the write-back (which recomputes ŵ, err and q from the
// weight each column was quantized from) round identically.
struct QOut { float q, x; };
__device__ __forceinline__ QOut quant1(float wj, float s, float rs, float z, float fmaxq) {
  const float q = fminf(fmaxf(rintf(fmaf(wj, rs, z)), 0.f), fmaxq);
  return QOut{q, fmaf(-s, q - z, wj)};
}

// The rest of the super-block for the workgroup's rows (GPTQ's lazy batch
// update, restricted to the super-block): W[rows, n] −= Σ_k E[rows][k]·U[k][n]
// over the block's 128 k, for the nupd columns n after the block, on
// v_mfma_f32_16x16x4f32: a[x][k] = −E[x][k] from lane (x, kq), b[k][y] =
// U[k][y] from lane (y, kq), D[x][y] at lane (y, kq) for rows x = 4kq..4kq+3.
// Lane group kq takes k = 32kq + s at step s (the same for both operands),
// so a lane reads its E row as whole float4s.  The workgroup's 4·waves rows
// are M (rows of 16 beyond them, or beyond m, are computed and dropped);
// wave w takes the 16-column tiles w, w + waves, ...; each tile's 32 U values
// and 4 weights per lane are loaded a tile ahead, from clamped positions
// (columns past nupd are computed and dropped).
constexpr int kEs = kBlock + 4;   // LDS row stride of E (floats)
__device__ __forceinline__ void panel_update(const SweepArgs& a, float* Us, const float (&e)[8],
                                             int wave, int lane) {
  const int nw = blockDim.x >> 6, rows = 4 * nw;
  const int c = lane & 15, rloc = lane >> 4;
  __syncthreads();   // every wave is past the column loop: Us is free
  float* Es = Us;    // [16][kEs]: E of the workgroup's rows
  *reinterpret_cast<f32x4*>(Es + (4 * wave + rloc) * kEs + 4 * c) = f32x4{e[0], e[1], e[2], e[3]};
  *reinterpret_cast<f32x4*>(Es + (4 * wave + rloc) * kEs + 64 + 4 * c) = f32x4{e[4], e[5], e[6], e[7]};
  __syncthreads();
  const int l16 = lane & 15, kq = lane >> 4;
  float av[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(Es + l16 * kEs + 32 * kq + 4 * i);
#pragma unroll
    for (int u = 0; u < 4; ++u) av[4 * i + u] = -v[u];
  }
  const int64_t row0 = (int64_t)blockIdx.x * rows;
  const int ntiles = (a.nupd + 15) / 16;
  // the workgroup's rows of W from the first updated column, as a buffer:
  // lanes whose row or column is outside get an offset past its end, so
  // their loads read 0 and their stores are dropped, with no branch
  const int64_t c0 = a.b0 + kBlock;
  const int64_t nrows = a.m - row0 < rows ? a.m - row0 : rows;
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      a.Wk + row0 * a.ldw + c0, 0, (int)(nrows * a.ldw * 4), 0x00020000);
  constexpr uint32_t kOut = 0x80000000u;   // past any workgroup's rows (< 2^31 bytes)
  auto woff = [&](int v, int n) -> uint32_t {
    const int x = 4 * kq + v;
    const bool ok = (x < rows) & (n < a.nupd);   // no short-circuit branch
    return ok ? (uint32_t)((x * a.ldw + n) * 4) : kOut;
  };
  // the tile's weights first (the accumulator needs them first), then its
  // 32 U values (columns past nupd read the last column: computed, dropped)
  auto load = [&](int tile, float (&bv)[32], f32x4& cv) {
    const int tc = tile < ntiles ? tile : ntiles - 1;
    const int n0 = 16 * tc + l16, n = n0 < a.nupd ? n0 : a.nupd - 1;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      cv[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wrs, woff(v, n0), 0, 0));
    const float* ub = a.Upan + (int64_t)(32 * kq) * a.ldu + n;
#pragma unroll
    for (int s2 = 0; s2 < 32; ++s2) bv[s2] = ub[(int64_t)s2 * a.ldu];
    __builtin_amdgcn_sched_barrier(0);   // all issued before the chain that follows
  };
  auto compute = [&](int tile, const float (&bv)[32], f32x4 acc) {
#pragma unroll
    for (int s2 = 0; s2 < 32; ++s2) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s2], bv[s2], acc, 0, 0, 0);
    const int n = 16 * tile + l16;
    // bit-cast as a whole vector: a bit-cast of one element of a float4
    // (acc[v]) was compiled as a bit-cast of its first element for every v
    // (read in the ISA)
    const u32x4 o = __builtin_bit_cast(u32x4, acc);
#pragma unroll
    for (int v = 0; v < 4; ++v) __builtin_amdgcn_raw_buffer_store_b32(o[v], wrs, woff(v, n), 0, 0);
    // one tile at a time: the next tile's loads then have this whole chain
    // to land in
    __builtin_amdgcn_sched_barrier(0);
  };
  // this wave's tiles w + i·waves, two buffers, each loaded a tile ahead
  const int mine = wave < ntiles ? (ntiles - 1 - wave) / nw + 1 : 0;
  float b0v[32], b1v[32];
  f32x4 c0v, c1v;
  load(wave, b0v, c0v);
  int i = 0;
  for (; i + 2 <= mine; i += 2) {
    load(wave + (i + 1) * nw, b1v, c1v);
    compute(wave + i * nw, b0v, c0v);
    load(wave + (i + 2) * nw, b0v, c0v);
    compute(wave + (i + 1) * nw, b1v, c1v);
  }
  if (i < mine) compute(wave + i * nw, b0v, c0v);
}

// G > 0: groups of G columns inside the block (parameters from registers);
// G == 0: the block lies inside one group whose parameters are already in
// scales/zeros.  bw = number of real columns in the block.
template <int G>
__global__ __launch_bounds__(256) void sweep_kernel(SweepArgs a) {
  constexpr int GG = G > 0 ? G : 1;
  __shared__ __attribute__((aligned(16))) float Us[kBlock * kBlock];
  __shared__ __attribute__((aligned(16))) float rud[kBlock];
  const int nthr = blockDim.x, t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int c = lane & 15, rloc = lane >> 4;          // lane within the row, row in the wave
  const int64_t r = ((int64_t)blockIdx.x * (nthr >> 6) + wave) * 4 + (lane >> 4);
  const bool live = r < a.m;
  // Stage the block's U (64 KB) in LDS.  With 16-byte aligned rows it goes
  // from memory straight into LDS (global_load_lds_dwordx4, 1 KB = two U
  // rows per instruction, every copy in flight at once); otherwise all of a
  // thread's loads are issued before its stores.  The weights are loaded
  // meanwhile.
  const bool vec = (((uintptr_t)a.Ublk) % 16 == 0) && (a.ldu % 4 == 0);
  if (vec) {
    const unsigned sbase = (unsigned)(uintptr_t)(__attribute__((address_space(3))) float*)Us;
    for (int seg = wave; seg < kBlock * kBlock / 256; seg += nthr >> 6) {
      const int e = seg * 256 + lane * 4, i = e / kBlock, j = e % kBlock;
      const float* src = a.Ublk + (int64_t)i * a.ldu + j;
      // 16 bytes per lane to LDS M0 + 16·lane; no register result, waited
      // for by the vmcnt wait below
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(sbase + (unsigned)seg * 1024u), "v"(src) : "memory");
    }
  } else {
    for (int e0 = t * 4; e0 < kBlock * kBlock; e0 += nthr * 4 * 16) {
      f32x4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int e = e0 + u * nthr * 4, i = e / kBlock, j = e % kBlock;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[u][q] = e < kBlock * kBlock ? a.Ublk[(int64_t)i * a.ldu + j + q] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int e = e0 + u * nthr * 4;
        if (e < kBlock * kBlock) *reinterpret_cast<f32x4*>(&Us[e]) = v[u];
      }
    }
  }
  // slot sl < 4: column 4c+sl; slot sl >= 4: column 64+4c+sl-4; after
  // column j the owner lane's slot keeps the weight column j was quantized
  // from (U's diagonal is zeroed in LDS, and later columns' rows of U are
  // zero there), from which the write-back recomputes ŵ, err and q
  float w[QC];
  {
    const float* src = a.Wk + (live ? r : 0) * a.ldw + a.b0 + 4 * c;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 64);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q] = lo[q]; w[4 + q] = hi[q];
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): U copies and weights have landed
  __syncthreads();
  for (int j = t; j < kBlock; j += nthr) {
    rud[j] = 1.f / Us[j * kBlock + j];
    Us[j * kBlock + j] = 0.f;
  }
  __syncthreads();

  float s = 1.f, z = 0.f, rs = 1.f;
  if (G == 0) {
    const int64_t gi = a.b0 / a.g;
    if (live) {
      s = a.scales[r * a.ng + gi];
      z = (float)a.zeros[r * a.ng + gi];
    }
    rs = 1.f / s;
  }
  const float fmaxq = (float)a.maxq;
  constexpr int NG = G > 0 ? kBlock / GG : 1;   // groups starting in this block
  float gs[NG], gz[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) { gs[k] = 1.f; gz[k] = 0.f; }
  // U row j is read from LDS two columns ahead (its first half only while
  // j < 64: afterwards the lanes' columns below 64 are all done) and 1/U_jj
  // four at a time; the scheduling barrier at the end of each column keeps
  // the compiler from hoisting all 128 columns' reads (which would not fit
  // in registers)
  constexpr int PF = 2;
  f32x4 ub0[PF], ub1[PF];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    ub0[p] = *reinterpret_cast<const f32x4*>(Us + p * kBlock + 4 * c);
    ub1[p] = *reinterpret_cast<const f32x4*>(Us + p * kBlock + 64 + 4 * c);
  }
  f32x4 ru4 = *reinterpret_cast<const f32x4*>(rud), ru4n = *reinterpret_cast<const f32x4*>(rud + 4);
#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    const int o = (j & 63) >> 2, slot = (j >> 6) * 4 + (j & 3);
    const f32x4 u0 = ub0[j % PF], u1 = ub1[j % PF];
    if (j % 4 == 0 && j > 0) {
      ru4 = ru4n;
      if (j + 4 < kBlock) ru4n = *reinterpret_cast<const f32x4*>(rud + j + 4);
    }
    const float ru = ru4[j % 4];
    if (j + PF < kBlock) {
      if (j + PF < 64) ub0[j % PF] = *reinterpret_cast<const f32x4*>(Us + (j + PF) * kBlock + 4 * c);
      ub1[j % PF] = *reinterpret_cast<const f32x4*>(Us + (j + PF) * kBlock + 64 + 4 * c);
    }
    if (G > 0 && j % GG == 0) {
      // the group's columns [j, j+G) ∩ real columns, spread over the row
      float mn = INFINITY, mx = -INFINITY, am = 0.f;
#pragma unroll
      for (int sl = 0; sl < QC; ++sl) {
        const int col = (sl < 4) ? 4 * c + sl : 64 + 4 * c + (sl - 4);
        const bool in = col >= j && col < j + GG && col < a.bw;
        mn = fminf(mn, in ? w[sl] : INFINITY); mx = fmaxf(mx, in ? w[sl] : -INFINITY);
        am = fmaxf(am, in ? fabsf(w[sl]) : 0.f);
      }
      mn = row_min(mn); mx = row_max(mx); am = row_max(am);
      float s2, z2;
      group_qparams(mn, mx, am, a.maxq, a.sym, s2, z2);
      // groups starting beyond the real columns keep the previous parameters
      const bool real = j < a.bw;
      s = real ? s2 : s;
      z = real ? z2 : z;
      rs = 1.f / s;
      gs[j / GG] = s;
      gz[j / GG] = z;
    }
    const float wj = row_bcast(w[slot], o);
    const float err = quant1(wj, s, rs, z, fmaxq).x * ru;
    // columns below 64 are all done once j >= 64 (U is upper triangular)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      if (j < 64) w[q4] = fmaf(-err, u0[q4], w[q4]);
      w[4 + q4] = fmaf(-err, u1[q4], w[4 + q4]);
    }
    // keep the compiler from deferring column updates to the end of the
    // block (which holds every column's err in registers): the updated
    // weights must exist here
#pragma unroll
    for (int k = 0; k < QC; ++k) asm volatile("" : "+v"(w[k]));
    __builtin_amdgcn_sched_barrier(0);
  }
  // ŵ, err and the code of each of the lane's columns, from the weight it
  // was quantized from, with its group's parameters
  float e[QC], qc[QC];
  {
    const f32x4 rlo = *reinterpret_cast<const f32x4*>(rud + 4 * c);
    const f32x4 rhi = *reinterpret_cast<const f32x4*>(rud + 64 + 4 * c);
#pragma unroll
    for (int sl = 0; sl < QC; ++sl) {
      const int col = (sl < 4) ? 4 * c + sl : 64 + 4 * c + (sl - 4);
      float sv = s, zv = z, rsv = rs;
      if (G > 0) {
        const int gi = col / GG;
        sv = gs[0];
        zv = gz[0];
#pragma unroll
        for (int u = 1; u < NG; ++u) { sv = (gi == u) ? gs[u] : sv; zv = (gi == u) ? gz[u] : zv; }
        rsv = 1.f / sv;
      }
      const QOut r1 = quant1(w[sl], sv, rsv, zv, fmaxq);
      e[sl] = r1.x * (sl < 4 ? rlo[sl] : rhi[sl - 4]);
      qc[sl] = r1.q;
      w[sl] = sv * (r1.q - zv);
    }
  }
  if (G > 0 && live && c == 0) {
    for (int k = 0; k < NG && k * GG < a.bw; ++k) {
      const int64_t gi = (a.b0 + k * GG) / GG;
      float sv = gs[0], zv = gz[0];
#pragma unroll
      for (int u = 1; u < NG; ++u) { sv = (u == k) ? gs[u] : sv; zv = (u == k) ? gz[u] : zv; }
      a.scales[r * a.ng + gi] = sv;
      a.zeros[r * a.ng + gi] = (uint8_t)zv;
    }
  }
  // row loss ½·Σ err²: the lane's 8 columns, then the row
  float loss = 0.f;
#pragma unroll
  for (int k = 0; k < QC; ++k) loss = fmaf(e[k], e[k], loss);
  loss += dpp<0xB1>(loss);
  loss += dpp<0x4E>(loss);
  loss += dpp<0x141>(loss);
  loss += dpp<0x140>(loss);
  if (live && c == 0 && a.row_loss) a.row_loss[r] += 0.5f * loss;
  // write back: lane c stores its row's columns 4c..4c+3 and 64+4c..64+4c+3
  if (live) {
    float* dw = a.Wk + r * a.ldw + a.b0 + 4 * c;
    float* de = a.Err + r * a.lde + 4 * c;
    uint8_t* dq = a.codes + r * a.ldw + a.b0 + 4 * c;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 vw, ve;
      uint32_t pk = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        vw[q] = w[4 * h + q];
        ve[q] = e[4 * h + q];
        pk |= (uint32_t)qc[4 * h + q] << (8 * q);
      }
      *reinterpret_cast<f32x4*>(dw + 64 * h) = vw;
      *reinterpret_cast<f32x4*>(de + 64 * h) = ve;
      *reinterpret_cast<uint32_t*>(dq + 64 * h) = pk;
    }
  }
  if (a.nupd > 0) panel_update(a, Us, e, wave, lane);
}

}  // namespace

template <>
hipError_t launch_sweep<GQ_SWEEP_G>(const SweepArgs& a, hipStream_t s) {
  // waves per workgroup: enough workgroups to cover the CUs, at most 4 waves
  const int64_t waves = ceil_div(a.m, 4);
  const int W = (int)std::max<int64_t>(1, std::min<int64_t>(4, waves / 256));
  sweep_kernel<GQ_SWEEP_G><<<(unsigned)ceil_div(waves, W), 64 * W, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace gq
