// One 128-column block of the GPTQ column sweep ("GPTQ: Mathematical
// Foundations ...": The GPTQ Algorithmic Innovations 2-3 -- in-block updates
// and the Cholesky form of the compensation; walkthrough step 3; "INT4 and
// GPTQ Quantization": Uniform INT4 Quantization, Group Quantization).
//
// This file is compiled once per group-size variant (-DGQ_SWEEP_G=0/32/64/128)
// so the heavily unrolled variants build in parallel.
//
// Layout: four lanes (a DPP quad) per weight row, lane c of the quad holding
// the row's columns 32c..32c+31 of the block in registers; a wave covers 16
// rows, a workgroup 16·W rows.  The block's 128x128 part of U and 1/U_jj are
// staged in LDS once per workgroup.  For each column j of the block:
//   w_j is broadcast inside the quad from its owner lane (DPP quad_perm),
//   at a group start the quad reduces the group's current min/max,
//   v = w_j·(1/s) + z;  q = clamp(rint(v), 0, 2ᵇ−1);  ŵ = s(q − z)
//   err = (w_j − ŵ)·(1/U_jj);  every lane: w_k −= err·U_jk for its 32 columns
// (U is upper triangular, so columns at or left of j receive zeros and the
// update needs no per-lane bounds).  ŵ, err and q go to LDS and are written
// back coalesced after the block.  The working copy is padded to whole blocks:
// padded columns hold 0 and their U rows/columns are 0 with a unit diagonal,
// so they quantize to 0 with err 0.
#include "common.hpp"

#ifndef GQ_SWEEP_G
#error "compile with -DGQ_SWEEP_G=<group size handled in registers, 0 = external>"
#endif

namespace gq {
namespace {

constexpr int QC = kBlock / 4;        // columns per lane
constexpr int SROW = kBlock + 1;      // LDS staging row stride (odd: no bank conflicts)
constexpr int QROW = kBlock + 4;      // code staging row stride (bytes)
constexpr size_t kWaveStage = (size_t)2 * 16 * SROW * sizeof(float) + 16 * QROW;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// quad_perm selector with every lane reading quad lane o
template <int O>
__device__ __forceinline__ float quad_bcast(float x) {
  return dpp<O | (O << 2) | (O << 4) | (O << 6)>(x);
}
__device__ __forceinline__ float quad_min(float x) {
  x = fminf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  return fminf(x, dpp<0x4E>(x)); // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  return fmaxf(x, dpp<0x4E>(x));
}

// G > 0: groups of G columns inside the block (parameters from registers);
// G == 0: the block lies inside one group whose parameters are already in
// scales/zeros.  bw = number of real columns in the block.
template <int G>
__global__ __launch_bounds__(256) void sweep_kernel(SweepArgs a) {
  constexpr int GG = G > 0 ? G : 1;
  __shared__ __attribute__((aligned(16))) float Us[kBlock * kBlock];
  __shared__ float rud[kBlock];
  extern __shared__ __attribute__((aligned(16))) char dyn[];  // per wave: ŵ, err [16][SROW] fp32, codes [16][QROW] u8
  const int nthr = blockDim.x, t = threadIdx.x;
  {
    const bool vec = (((uintptr_t)a.Ublk) % 16 == 0) && (a.ldu % 4 == 0);
    for (int e = t * 4; e < kBlock * kBlock; e += nthr * 4) {
      const int i = e / kBlock, j = e % kBlock;
      f32x4 v;
      if (vec) {
        v = *reinterpret_cast<const f32x4*>(a.Ublk + (int64_t)i * a.ldu + j);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = a.Ublk[(int64_t)i * a.ldu + j + q];
      }
      *reinterpret_cast<f32x4*>(&Us[e]) = v;
    }
  }
  __syncthreads();
  for (int j = t; j < kBlock; j += nthr) rud[j] = 1.f / Us[j * kBlock + j];
  __syncthreads();

  const int wave = t >> 6, lane = t & 63;
  const int rloc = lane >> 2, c = lane & 3;          // row within the wave, quad lane
  const int64_t rbase = ((int64_t)blockIdx.x * (nthr >> 6) + wave) * 16;
  const int64_t r = rbase + rloc;
  const bool live = r < a.m;
  float* SW = reinterpret_cast<float*>(dyn + wave * kWaveStage);   // ŵ
  float* SE = SW + 16 * SROW;                                        // err
  uint8_t* SQ = reinterpret_cast<uint8_t*>(SE + 16 * SROW);          // codes

  float w[QC];
  {
    const float* src = a.Wk + (live ? r : 0) * a.ldw + a.b0 + c * QC;
#pragma unroll
    for (int k = 0; k < QC; k += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + k);
      w[k] = v[0]; w[k + 1] = v[1]; w[k + 2] = v[2]; w[k + 3] = v[3];
    }
  }

  float s = 1.f, z = 0.f, rs = 1.f;
  if (G == 0) {
    const int64_t gi = a.b0 / a.g;
    if (live) {
      s = a.scales[r * a.ng + gi];
      z = (float)a.zeros[r * a.ng + gi];
    }
    rs = 1.f / s;
  }
  float loss = 0.f;
  const float fmaxq = (float)a.maxq;
  constexpr int NG = G > 0 ? kBlock / GG : 1;   // groups starting in this block
  float gs[NG], gz[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) { gs[k] = 1.f; gz[k] = 0.f; }
#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    const int o = j / QC, jj = j % QC;
    if (G > 0 && j % GG == 0) {
      // the group's columns [j, j+G) ∩ real columns, spread over the quad
      float mn = INFINITY, mx = -INFINITY, am = 0.f;
#pragma unroll
      for (int k = 0; k < QC; ++k) {
        const int col = c * QC + k;
        const bool in = col >= j && col < j + GG && col < a.bw;
        mn = fminf(mn, in ? w[k] : INFINITY); mx = fmaxf(mx, in ? w[k] : -INFINITY);
        am = fmaxf(am, in ? fabsf(w[k]) : 0.f);
      }
      mn = quad_min(mn); mx = quad_max(mx); am = quad_max(am);
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
    float wj;
    switch (o) {
      case 0: wj = quad_bcast<0>(w[jj]); break;
      case 1: wj = quad_bcast<1>(w[jj]); break;
      case 2: wj = quad_bcast<2>(w[jj]); break;
      default: wj = quad_bcast<3>(w[jj]); break;
    }
    const float v = wj * rs + z;
    const float q = fminf(fmaxf(rintf(v), 0.f), fmaxq);
    const float wq = s * (q - z);
    const float err = (wj - wq) * rud[j];
    // every lane of the quad holds the same ŵ, err, q: same-address writes
    SW[rloc * SROW + j] = wq;
    SE[rloc * SROW + j] = err;
    SQ[rloc * QROW + j] = (uint8_t)q;
    loss = (c == o) ? fmaf(err, err, loss) : loss;
    const float* Urow = Us + j * kBlock + c * QC;
#pragma unroll
    for (int k = 0; k < QC; ++k) w[k] = fmaf(-err, Urow[k], w[k]);
  }
  // row loss: sum the quad's partial sums
  loss += dpp<0xB1>(loss);
  loss += dpp<0x4E>(loss);
  if (live && c == 0 && a.row_loss) a.row_loss[r] += 0.5f * loss;
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
  __syncthreads();
  // write back: lane (row, c) stores its row's columns c*32 .. +31
  if (live) {
    float* dw = a.Wk + r * a.ldw + a.b0 + c * QC;
    float* de = a.Err + r * kBlock + c * QC;
    uint8_t* dq = a.codes + r * a.ldw + a.b0 + c * QC;
#pragma unroll
    for (int k = 0; k < QC; k += 4) {
      f32x4 vw, ve;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        vw[q] = SW[rloc * SROW + c * QC + k + q];
        ve[q] = SE[rloc * SROW + c * QC + k + q];
      }
      *reinterpret_cast<f32x4*>(dw + k) = vw;
      *reinterpret_cast<f32x4*>(de + k) = ve;
      *reinterpret_cast<uint32_t*>(dq + k) =
          *reinterpret_cast<const uint32_t*>(SQ + rloc * QROW + c * QC + k);
    }
  }
}

}  // namespace

template <>
hipError_t launch_sweep<GQ_SWEEP_G>(const SweepArgs& a, hipStream_t s) {
  // waves per workgroup: enough workgroups to cover the CUs, at most 4 waves
  const int64_t waves = ceil_div(a.m, 16);
  const int W = (int)std::max<int64_t>(1, std::min<int64_t>(4, waves / 256));
  const size_t dyn = (size_t)W * kWaveStage;
  sweep_kernel<GQ_SWEEP_G><<<(unsigned)ceil_div(waves, W), 64 * W, dyn, s>>>(a);
  return hipGetLastError();
}

}  // namespace gq
