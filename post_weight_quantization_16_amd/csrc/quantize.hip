// The GPTQ column sweep with lazy block updates ("GPTQ: Mathematical
// Foundations ...": The GPTQ Algorithmic Innovations 1-3, walkthrough step 3;
// "INT4 and GPTQ Quantization": Uniform INT4 Quantization, Group Quantization).
//
// Working state: Wk [m x d] fp32, columns already in quantization order and
// dead columns zeroed.  For each block of 128 columns:
//   sweep   16 lanes per row keep the block's 128 weights in registers and
//           run the sequential column loop: group (s, z) at group starts,
//           q = clamp(rint(w/s + z)), ŵ = s(q − z), err = (w − ŵ)/U_cc and
//           w_k −= err·U_ck for the block's later columns (sweep.hip).
//   update  the "lazy batch" product W[:, later] −= Err[:, block]·U[block, later]
//           on the fp32 MFMA GEMM, in two levels: blocks are grouped into
//           super-blocks of 4; after a block only the rest of its
//           super-block is updated, and after the super-block everything to
//           its right receives the whole super-block's update at once
//           (K = 512).  The sum of the four rank-128 products is the same
//           update; the columns right of the super-block are not read until
//           it is done.  Group parameters taken at a group start need the
//           group's columns current, so super-blocks are used only when every
//           group start is a super-block start or the group lies inside one.
// Finally codes are packed and Ŵ is written in the original column order.
//
// Reading where the pages disagree: U (the upper Cholesky factor of H_d⁻¹)
// drives both the in-block and the between-block update; the walkthrough's
// between-block product with H⁻¹ does not reproduce the OBS update.
#include <algorithm>

#include "common.hpp"

namespace gq {
namespace {

struct QWs { float* Wk; float* Err; uint8_t* codes; int* inv; float* Upad; };

// Working copy and codes are padded to whole blocks (dp = ceil(d/128)·128).
QWs carve(void* ws, int64_t m, int64_t d) {
  const int64_t dp = ceil_div(d, kBlock) * kBlock;
  char* p = static_cast<char*>(ws);
  QWs w;
  w.Wk = reinterpret_cast<float*>(p); p += align_up((size_t)m * dp * 4);
  w.Err = reinterpret_cast<float*>(p); p += align_up((size_t)m * kSuper * kBlock * 4);
  w.codes = reinterpret_cast<uint8_t*>(p); p += align_up((size_t)m * dp);
  w.inv = reinterpret_cast<int*>(p); p += align_up((size_t)d * 4);
  w.Upad = reinterpret_cast<float*>(p);
  return w;
}

__device__ __forceinline__ float load_w(const void* W, int dt, int64_t i) {
  if (dt == GPTQ_F32) return static_cast<const float*>(W)[i];
  const uint16_t b = static_cast<const uint16_t*>(W)[i];
  if (dt == GPTQ_BF16) return __uint_as_float((uint32_t)b << 16);
  return (float)__builtin_bit_cast(_Float16, b);
}

// Wk[r][a] = W[r][π(a)] (0 for dead channels and padding a >= d);
// inv[π(a)] = a; row_loss = 0.  Each thread writes 4 consecutive columns
// (one float4: dp is a multiple of 128).
__global__ __launch_bounds__(256) void init_kernel(const void* __restrict__ W, int dt, int64_t ld_w,
                                                   int64_t m, int64_t d, int64_t dp,
                                                   const int* __restrict__ perm,
                                                   const uint8_t* __restrict__ dead,
                                                   float* __restrict__ Wk, int* __restrict__ inv,
                                                   float* __restrict__ row_loss) {
  const int64_t a0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    if (row_loss && blockIdx.x == 0 && threadIdx.x == 0) row_loss[r] = 0.f;
    if (a0 >= dp) continue;
    f32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t a = a0 + q;
      float x = 0.f;
      if (a < d) {
        const int c = perm ? perm[a] : (int)a;
        x = load_w(W, dt, r * ld_w + c);
        if (dead && dead[c]) x = 0.f;
        if (r == 0) inv[c] = (int)a;
      }
      v[q] = x;
    }
    *reinterpret_cast<f32x4*>(Wk + r * dp + a0) = v;
  }
}

// Per-row (s, z) of the group [c0, c1) from the current Wk (groups spanning
// whole blocks).  One wave per row.
__global__ __launch_bounds__(256) void group_params_kernel(const float* __restrict__ Wk, int64_t m,
                                                           int64_t ldw, int64_t c0, int64_t c1,
                                                           int maxq, int sym,
                                                           float* __restrict__ scales,
                                                           uint8_t* __restrict__ zeros, int ng,
                                                           int gi) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= m) return;
  float mn = INFINITY, mx = -INFINITY, am = 0.f;
  for (int64_t c = c0 + lane; c < c1; c += 64) {
    const float v = Wk[r * ldw + c];
    mn = fminf(mn, v); mx = fmaxf(mx, v); am = fmaxf(am, fabsf(v));
  }
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
    am = fmaxf(am, __shfl_xor(am, o));
  }
  if (lane == 0) {
    float s, z;
    group_qparams(mn, mx, am, maxq, sym, s, z);
    scales[r * ng + gi] = s;
    zeros[r * ng + gi] = (uint8_t)z;
  }
}

// U's last (short) diagonal block, padded to 128x128: zeros outside the real
// part, 1 on the padded diagonal.
__global__ __launch_bounds__(256) void pad_u_kernel(const float* __restrict__ U, int64_t d,
                                                    int64_t b0, int bw, float* __restrict__ Upad) {
  for (int e = threadIdx.x; e < kBlock * kBlock; e += 256) {
    const int i = e / kBlock, j = e % kBlock;
    float v = (i == j) ? 1.f : 0.f;
    if (i < bw && j < bw) v = U[(b0 + i) * d + b0 + j];
    Upad[e] = v;
  }
}

// Write Ŵ / g_idx and pack the codes, in the original column order.  The
// first loop gives each thread 4 consecutive output columns of Ŵ (gathered
// through inv, which is contiguous without act-order); the second gives
// each thread one packed word.
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ Wk,
                                                       const uint8_t* __restrict__ codes,
                                                       const int* __restrict__ inv, int64_t m,
                                                       int64_t d, int64_t dp, int bits, int64_t g,
                                                       uint32_t* __restrict__ qweight,
                                                       float* __restrict__ W_hat,
                                                       int32_t* __restrict__ g_idx, int vec_w) {
  const int cpw = bits <= 4 ? 8 : 4, cwid = 32 / cpw;
  const int64_t nw = (d + cpw - 1) / cpw;
  const int64_t lin = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    const int64_t c0 = lin * 4;
    if ((W_hat || (g_idx && r == 0)) && c0 < d) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t c = c0 + q;
        v[q] = 0.f;
        if (c < d) {
          const int a = inv[c];
          v[q] = Wk[r * dp + a];
          if (g_idx && r == 0) g_idx[c] = (int32_t)(a / g);
        }
      }
      if (W_hat) {
        if (vec_w && c0 + 3 < d) {
          const f32x4 o = {v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4*>(W_hat + r * d + c0) = o;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (c0 + q < d) W_hat[r * d + c0 + q] = v[q];
        }
      }
    }
    for (int64_t k = lin; k < nw; k += (int64_t)gridDim.x * 256) {
      uint32_t word = 0;
      for (int i = 0; i < cpw; ++i) {
        const int64_t c = k * cpw + i;
        if (c >= d) break;
        word |= (uint32_t)codes[r * dp + inv[c]] << (cwid * i);
      }
      qweight[r * nw + k] = word;
    }
  }
}

template <int G>
hipError_t run_blocks(QWs& w, int64_t m, int64_t d, const float* U, const gptq_params& p,
                      int64_t g, int ng, float* scales, uint8_t* zeros, float* row_loss,
                      hipStream_t s) {
  const int64_t dp = ceil_div(d, kBlock) * kBlock;
  const int maxq = (1 << p.bits) - 1;
  // super-blocks only where no group straddles a super-block boundary
  // with its start inside it (groups of G > 0 columns stay inside a block)
  const int64_t sbw = kSuper * kBlock;
  const bool two_level = G > 0 || g >= d || g % sbw == 0 || sbw % g == 0;
  const int64_t sb = two_level ? sbw : kBlock;
  const int64_t lde = kSuper * kBlock;
  hipError_t e;
  for (int64_t sb0 = 0; sb0 < d; sb0 += sb) {
    const int64_t se = std::min<int64_t>(sb0 + sb, d);
    for (int64_t b0 = sb0; b0 < se; b0 += kBlock) {
      const int bw = (int)std::min<int64_t>(kBlock, d - b0);
      if (G == 0 && b0 % g == 0) {
        group_params_kernel<<<(unsigned)ceil_div(m, 4), 256, 0, s>>>(
            w.Wk, m, dp, b0, std::min<int64_t>(b0 + g, d), maxq, p.sym, scales, zeros, ng,
            (int)(b0 / g));
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      SweepArgs a{};
      a.Wk = w.Wk; a.ldw = dp; a.m = m; a.b0 = b0; a.bw = bw;
      if (bw == kBlock) {
        a.Ublk = U + b0 * d + b0; a.ldu = d;
      } else {
        pad_u_kernel<<<1, 256, 0, s>>>(U, d, b0, bw, w.Upad);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        a.Ublk = w.Upad; a.ldu = kBlock;
      }
      a.maxq = maxq; a.sym = p.sym; a.scales = scales; a.zeros = zeros; a.ng = ng; a.g = g;
      a.Err = w.Err + (b0 - sb0); a.lde = lde;
      a.codes = w.codes; a.row_loss = row_loss;
      if ((e = launch_sweep<G>(a, s)) != hipSuccess) return e;
      const int64_t b1 = b0 + bw;
      if (b1 < se) {  // the rest of the super-block: W[:, b1:se] −= Err_b · U[b, b1:se]
        GemmArgs u{};
        u.M = (int)m; u.N = (int)(se - b1); u.K = bw; u.k_last = bw; u.batch = 1;
        u.alpha = -1.f; u.beta = 1.f;
        u.A = w.Err + (b0 - sb0); u.lda = lde; u.trans_a = false;
        u.B = U + b0 * d + b1; u.ldb = d; u.trans_b = false;
        u.C = w.Wk + b1; u.ldc = dp; u.tri = 0;
        if ((e = gemm_f32(u, s)) != hipSuccess) return e;
      }
    }
    if (se < d) {  // everything right of it: W[:, se:] −= Err_sb · U[sb, se:]
      GemmArgs u{};
      u.M = (int)m; u.N = (int)(d - se); u.K = (int)(se - sb0); u.k_last = u.K; u.batch = 1;
      u.alpha = -1.f; u.beta = 1.f;
      u.A = w.Err; u.lda = lde; u.trans_a = false;
      u.B = U + sb0 * d + se; u.ldb = d; u.trans_b = false;
      u.C = w.Wk + se; u.ldc = dp; u.tri = 0;
      if ((e = gemm_f32(u, s)) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

size_t quantize_ws_bytes(int64_t m, int64_t d) {
  const int64_t dp = ceil_div(d, kBlock) * kBlock;
  return align_up((size_t)m * dp * 4) + align_up((size_t)m * kSuper * kBlock * 4) +
         align_up((size_t)m * dp) +
         align_up((size_t)d * 4) + align_up((size_t)kBlock * kBlock * 4);
}

hipError_t quantize_launch(const void* W, int w_dtype, int64_t m, int64_t d, int64_t ld_w,
                           const float* U, const int32_t* perm, const uint8_t* dead,
                           const gptq_params& p, uint32_t* qweight, float* scales,
                           uint8_t* zeros, float* W_hat, int32_t* g_idx, float* row_loss,
                           void* ws, hipStream_t s) {
  QWs w = carve(ws, m, d);
  const int64_t g = (p.group_size <= 0 || p.group_size >= d) ? d : p.group_size;
  const int ng = (int)ceil_div(d, g);
  const unsigned gy = (unsigned)std::min<int64_t>(m, 65535);
  const int64_t dp = ceil_div(d, kBlock) * kBlock;
  init_kernel<<<dim3((unsigned)ceil_div(dp, 1024), gy), 256, 0, s>>>(W, w_dtype, ld_w, m, d, dp,
                                                                    perm, dead, w.Wk, w.inv,
                                                                    row_loss);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (g) {
    case 32: e = run_blocks<32>(w, m, d, U, p, g, ng, scales, zeros, row_loss, s); break;
    case 64: e = run_blocks<64>(w, m, d, U, p, g, ng, scales, zeros, row_loss, s); break;
    case 128: e = run_blocks<128>(w, m, d, U, p, g, ng, scales, zeros, row_loss, s); break;
    default: e = run_blocks<0>(w, m, d, U, p, g, ng, scales, zeros, row_loss, s); break;
  }
  if (e != hipSuccess) return e;
  const int vec_w = W_hat && ((uintptr_t)W_hat % 16 == 0) && (d % 4 == 0);
  finalize_kernel<<<dim3((unsigned)ceil_div(d, 1024), gy), 256, 0, s>>>(
      w.Wk, w.codes, w.inv, m, d, dp, p.bits, g, qweight, W_hat, g_idx, vec_w);
  return hipGetLastError();
}

}  // namespace gq
