// One 128-column block of the GPTQ column sweep ("GPTQ: Mathematical
// Foundations ...": The GPTQ Algorithmic Innovations 2-3 -- in-block updates
// and the Cholesky form of the compensation; walkthrough step 3; "INT4 and
// GPTQ Quantization": Uniform INT4 Quantization, Group Quantization).
//
// This file is compiled once per group-size variant (-DGQ_SWEEP_G=0/32/64/128)
// so the heavily unrolled variants build in parallel.
//
// One thread per row keeps the block's 128 weights in registers and runs the
// sequential loop over the block's columns j:
//   at a group start: (s, z) from the current values of the group's columns
//   v = w_j/s + z;  q = clamp(rint(v), 0, 2ᵇ−1);  ŵ = s(q − z)
//   err = (w_j − ŵ) / U_jj;  w_k −= err·U_jk  for the block's later columns
// U's row j is the same for every row, so its entries are wave-uniform loads.
// The working copy is padded to whole blocks: padded columns hold 0, their U
// rows/columns are 0 with a unit diagonal, so they quantize to 0 with err 0.
#include "common.hpp"

#ifndef GQ_SWEEP_G
#error "compile with -DGQ_SWEEP_G=<group size handled in registers, 0 = external>"
#endif

namespace gq {
namespace {

// G > 0: groups of G columns inside the block (parameters from registers);
// G == 0: the block lies inside one group whose parameters are already in
// scales/zeros.  bw = number of real columns in the block.
template <int G>
__global__ __launch_bounds__(64) void sweep_kernel(SweepArgs a) {
  constexpr int GG = G > 0 ? G : 1;
  const int64_t r = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (r >= a.m) return;
  float* wrow = a.Wk + r * a.ldw + a.b0;
  float w[kBlock];
#pragma unroll
  for (int j = 0; j < kBlock; ++j) w[j] = wrow[j];

  float s = 1.f, z = 0.f, rs = 1.f;
  if (G == 0) {
    const int64_t gi = a.b0 / a.g;
    s = a.scales[r * a.ng + gi];
    z = (float)a.zeros[r * a.ng + gi];
    rs = 1.f / s;
  }
  float loss = 0.f;
  const float fmaxq = (float)a.maxq;
#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    if (G > 0 && j % GG == 0 && j < a.bw) {
      float mn = INFINITY, mx = -INFINITY, am = 0.f;
#pragma unroll
      for (int k = 0; k < GG; ++k) {
        const int kk = j + k;
        if (kk < kBlock && kk < a.bw) {
          mn = fminf(mn, w[kk]); mx = fmaxf(mx, w[kk]); am = fmaxf(am, fabsf(w[kk]));
        }
      }
      group_qparams(mn, mx, am, a.maxq, a.sym, s, z);
      rs = 1.f / s;
      const int64_t gi = (a.b0 + j) / GG;
      a.scales[r * a.ng + gi] = s;
      a.zeros[r * a.ng + gi] = (uint8_t)z;
    }
    const float* Urow = a.Ublk + (int64_t)j * a.ldu;
    const float v = w[j] * rs + z;
    const float q = fminf(fmaxf(rintf(v), 0.f), fmaxq);
    const float wq = s * (q - z);
    const float err = (w[j] - wq) / Urow[j];
    loss += err * err;
#pragma unroll
    for (int k = j + 1; k < kBlock; ++k) w[k] = fmaf(-err, Urow[k], w[k]);
    wrow[j] = wq;
    a.codes[r * a.ldw + a.b0 + j] = (uint8_t)q;
    a.Err[r * kBlock + j] = err;
  }
  if (a.row_loss) a.row_loss[r] += 0.5f * loss;
}

}  // namespace

template <>
hipError_t launch_sweep<GQ_SWEEP_G>(const SweepArgs& a, hipStream_t s) {
  sweep_kernel<GQ_SWEEP_G><<<(unsigned)ceil_div(a.m, 64), 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace gq
