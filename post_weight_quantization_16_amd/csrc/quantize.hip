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

struct QWs {
  float* Wk; float* Err; uint8_t* codes; int* inv; int* src; float* Upad;
  float* S; uint8_t* Z; float* RL;   // stacked rows' scales/zeros/losses (several layers)
};
// group-count bound used for sizing (the smallest group the sweep runs is 32)
inline int64_t max_groups(int64_t d) { return ceil_div(d, 32); }

// Working copy and codes are padded to whole blocks (dp = ceil(d/128)·128).
QWs carve(void* ws, int64_t m, int64_t d) {
  const int64_t dp = ceil_div(d, kBlock) * kBlock;
  char* p = static_cast<char*>(ws);
  QWs w;
  w.Wk = reinterpret_cast<float*>(p); p += align_up((size_t)m * dp * 4);
  w.Err = reinterpret_cast<float*>(p); p += align_up((size_t)m * kSuper * kBlock * 4);
  w.codes = reinterpret_cast<uint8_t*>(p); p += align_up((size_t)m * dp);
  w.inv = reinterpret_cast<int*>(p); p += align_up((size_t)d * 4);
  w.src = reinterpret_cast<int*>(p); p += align_up((size_t)dp * 4);
  w.Upad = reinterpret_cast<float*>(p); p += align_up((size_t)kBlock * kBlock * 4);
  w.S = reinterpret_cast<float*>(p); p += align_up((size_t)m * max_groups(d) * 4);
  w.Z = reinterpret_cast<uint8_t*>(p); p += align_up((size_t)m * max_groups(d));
  w.RL = reinterpret_cast<float*>(p);
  return w;
}

__device__ __forceinline__ float load_w(const void* W, int dt, int64_t i) {
  if (dt == GPTQ_F32) return static_cast<const float*>(W)[i];
  const uint16_t b = static_cast<const uint16_t*>(W)[i];
  if (dt == GPTQ_BF16) return __uint_as_float((uint32_t)b << 16);
  return (float)__builtin_bit_cast(_Float16, b);
}

// Wk[r][a] = W[r][π(a)] (0 for dead channels and padding a >= d);
// inv[π(a)] = a; row_loss = 0.  Each thread writes 8 consecutive working
// columns (two float4: dp is a multiple of 128), every load issued before
// the stores; without a permutation (perm null) the row is read
// contiguously (vec_in: 16-byte loads are aligned).
__global__ __launch_bounds__(256) void init_kernel(const void* __restrict__ W, int dt, int64_t ld_w,
                                                   int64_t m, int64_t d, int64_t dp,
                                                   const int* __restrict__ perm,
                                                   const uint8_t* __restrict__ dead,
                                                   float* __restrict__ Wk, int* __restrict__ inv,
                                                   float* __restrict__ row_loss, int vec_in) {
  const int64_t a0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  int c[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) c[q] = (int)(a0 + q);
  if (perm && a0 < d) {
    if (a0 + 7 < d && ((uintptr_t)perm & 15) == 0) {
      const int4 p0 = *reinterpret_cast<const int4*>(perm + a0);
      const int4 p1 = *reinterpret_cast<const int4*>(perm + a0 + 4);
      c[0] = p0.x; c[1] = p0.y; c[2] = p0.z; c[3] = p0.w;
      c[4] = p1.x; c[5] = p1.y; c[6] = p1.z; c[7] = p1.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) c[q] = a0 + q < d ? perm[a0 + q] : 0;
    }
  }
  // the 8 mask bytes are loaded together (clamped, unconditional), then
  // tested: a load behind each test waited for the one before it
  bool dz[8];
  if (dead) {
    uint8_t dv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) dv[q] = dead[a0 + q < d ? c[q] : 0];
#pragma unroll
    for (int q = 0; q < 8; ++q) dz[q] = a0 + q >= d || dv[q] != 0;
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) dz[q] = a0 + q >= d;
  }
  // rows blockIdx.y·RB .. +RB−1 per step of the grid: every row's loads
  // are issued before the first store
  constexpr int RB = 4;
  for (int64_t r0 = (int64_t)blockIdx.y * RB; r0 < m; r0 += (int64_t)gridDim.y * RB) {
    if (a0 >= dp) {
      if (row_loss && threadIdx.x == 0 && blockIdx.x == 0)
        for (int64_t r = r0; r < r0 + RB && r < m; ++r) row_loss[r] = 0.f;
      continue;
    }
    float xs[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t r = r0 + rb < m ? r0 + rb : r0;
      float* x = xs[rb];
      const bool contig = !perm && vec_in && a0 + 7 < d;
      if (contig && dt == GPTQ_F32) {
        const float* src = static_cast<const float*>(W) + r * ld_w + a0;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) { x[q] = lo[q]; x[4 + q] = hi[q]; }
      } else if (contig) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + r * ld_w + a0);
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint16_t h = (uint16_t)(wd[q >> 1] >> (16 * (q & 1)));
          x[q] = dt == GPTQ_BF16 ? __uint_as_float((uint32_t)h << 16)
                                 : (float)__builtin_bit_cast(_Float16, h);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = a0 + q < d ? load_w(W, dt, r * ld_w + c[q]) : 0.f;
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t r = r0 + rb;
      if (r >= m) break;
      if (row_loss && blockIdx.x == 0 && threadIdx.x == 0) row_loss[r] = 0.f;
      f32x4 lo, hi;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo[q] = dz[q] ? 0.f : xs[rb][q];
        hi[q] = dz[4 + q] ? 0.f : xs[rb][4 + q];
      }
      *reinterpret_cast<f32x4*>(Wk + r * dp + a0) = lo;
      *reinterpret_cast<f32x4*>(Wk + r * dp + a0 + 4) = hi;
      if (r == 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (a0 + q < d) inv[c[q]] = (int)(a0 + q);
      }
    }
  }
}

// Permuted working copy for rows that fit in LDS (dp ≤ kRowLds): src[a] =
// π(a), or −1 for a dead column or a ≥ d (src_index_kernel, once), then one
// row of W per workgroup step, staged in LDS with coalesced loads
// (converted to fp32) and gathered as Wk[r][a] = W[r][src[a]] (0 where src
// is −1), written coalesced.  The source indices are re-read for every row
// (the same 4·dp bytes each time, from cache): kept in registers they would
// cost the occupancy that hides each row's load latency.
constexpr int kRowLds = 16384;            // staged row length limit (64 KB of fp32)
__global__ __launch_bounds__(256) void src_index_kernel(const int* __restrict__ perm,
                                                        const uint8_t* __restrict__ dead, int d,
                                                        int dp, int* __restrict__ src,
                                                        int* __restrict__ inv) {
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a >= dp) return;
  int c = -1;
  if (a < d) {
    const int pa = perm[a];
    inv[pa] = a;
    c = (dead && dead[pa]) ? -1 : pa;
  }
  src[a] = c;
}

__global__ __launch_bounds__(256) void init_rows_kernel(const void* __restrict__ W, int dt,
                                                        int64_t ld_w, int64_t m, int d, int dp,
                                                        const int* __restrict__ src_idx,
                                                        float* __restrict__ Wk,
                                                        float* __restrict__ row_loss, int vec_in) {
  extern __shared__ __attribute__((aligned(16))) float row[];
  const int t = threadIdx.x;
  for (int64_t r = blockIdx.x; r < m; r += gridDim.x) {
    __syncthreads();
    // every load of the row before the first LDS store
    if (dt == GPTQ_F32 && vec_in) {
      const float* src = static_cast<const float*>(W) + r * ld_w;
      for (int e0 = 0; e0 < d; e0 += 8192) {
        f32x4 buf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + 1024 * u + 4 * t;
          if (e + 3 < d) buf[u] = *reinterpret_cast<const f32x4*>(src + e);
          else
#pragma unroll
            for (int q = 0; q < 4; ++q) buf[u][q] = e + q < d ? src[e + q] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + 1024 * u + 4 * t;
          if (e < d) *reinterpret_cast<f32x4*>(row + e) = buf[u];
        }
      }
    } else if (dt != GPTQ_F32 && vec_in) {
      const uint16_t* src = static_cast<const uint16_t*>(W) + r * ld_w;
      uint4 buf[kRowLds / 2048];
#pragma unroll
      for (int u = 0; u < kRowLds / 2048; ++u) {
        const int e = 2048 * u + 8 * t;
        if (e + 7 < d) {
          buf[u] = *reinterpret_cast<const uint4*>(src + e);
        } else {
          uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (e + q < d) wd[q >> 1] |= (uint32_t)src[e + q] << (16 * (q & 1));
          buf[u] = uint4{wd[0], wd[1], wd[2], wd[3]};
        }
      }
#pragma unroll
      for (int u = 0; u < kRowLds / 2048; ++u) {
        const int e = 2048 * u + 8 * t;
        if (e >= d) break;
        const uint32_t wd[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
        f32x4 lo, hi;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint16_t h = (uint16_t)(wd[q >> 1] >> (16 * (q & 1)));
          const float x = dt == GPTQ_BF16 ? __uint_as_float((uint32_t)h << 16)
                                          : (float)__builtin_bit_cast(_Float16, h);
          if (q < 4) lo[q] = x; else hi[q - 4] = x;
        }
        *reinterpret_cast<f32x4*>(row + e) = lo;       // row has room up to dp >= e + 8
        *reinterpret_cast<f32x4*>(row + e + 4) = hi;
      }
    } else {
      for (int e0 = 0; e0 < d; e0 += 4096) {
        float buf[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + 256 * u + t;
          buf[u] = e < d ? load_w(W, dt, r * ld_w + e) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + 256 * u + t;
          if (e < d) row[e] = buf[u];
        }
      }
    }
    if (row_loss && t == 0) row_loss[r] = 0.f;
    __syncthreads();
    for (int a0 = 8 * t; a0 < dp; a0 += 2048) {   // src_idx is 256-byte aligned, dp % 128 == 0
      const int4 s0 = *reinterpret_cast<const int4*>(src_idx + a0);
      const int4 s1 = *reinterpret_cast<const int4*>(src_idx + a0 + 4);
      const int c[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      f32x4 lo, hi;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo[q] = c[q] < 0 ? 0.f : row[c[q]];
        hi[q] = c[4 + q] < 0 ? 0.f : row[c[4 + q]];
      }
      *reinterpret_cast<f32x4*>(Wk + r * dp + a0) = lo;
      *reinterpret_cast<f32x4*>(Wk + r * dp + a0 + 4) = hi;
    }
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

// Outputs in the original column order: Ŵ[r][c] = Wk[r][inv[c]], codes
// packed little-end first (8 per 32-bit word up to 4 bits, else 4), g_idx
// (row 0).  Each thread handles 8 consecutive output columns, every load
// issued before the stores; without a permutation (ident) the working row
// is read contiguously.
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ Wk,
                                                       const uint8_t* __restrict__ codes,
                                                       const int* __restrict__ inv, int64_t m,
                                                       int64_t d, int64_t dp, int bits, int64_t g,
                                                       uint32_t* __restrict__ qweight,
                                                       float* __restrict__ W_hat,
                                                       int32_t* __restrict__ g_idx, int vec_w,
                                                       int ident) {
  const int cpw = bits <= 4 ? 8 : 4, cwid = 32 / cpw;
  const int64_t nw = (d + cpw - 1) / cpw;
  const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (c0 >= d) return;
  const bool full = c0 + 7 < d;
  int a[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) a[q] = (int)(c0 + q);
  if (!ident) {
    if (full) {   // inv sits 256-byte aligned in the workspace
      const int4 p0 = *reinterpret_cast<const int4*>(inv + c0);
      const int4 p1 = *reinterpret_cast<const int4*>(inv + c0 + 4);
      a[0] = p0.x; a[1] = p0.y; a[2] = p0.z; a[3] = p0.w;
      a[4] = p1.x; a[5] = p1.y; a[6] = p1.z; a[7] = p1.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) a[q] = c0 + q < d ? inv[c0 + q] : 0;
    }
  }
  if (g_idx && blockIdx.y == 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (c0 + q < d) g_idx[c0 + q] = (int32_t)(a[q] / g);
  }
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    float v[8];
    uint32_t cd[8];
    const float* wr = Wk + r * dp;
    const uint8_t* qr = codes + r * dp;
    if (ident && full) {   // dp is a multiple of 128: these loads are aligned
      const f32x4 lo = *reinterpret_cast<const f32x4*>(wr + c0);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(wr + c0 + 4);
      const uint2 qq = *reinterpret_cast<const uint2*>(qr + c0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = lo[q]; v[4 + q] = hi[q];
        cd[q] = (qq.x >> (8 * q)) & 255u;
        cd[4 + q] = (qq.y >> (8 * q)) & 255u;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool in = c0 + q < d;
        v[q] = in ? wr[a[q]] : 0.f;
        cd[q] = in ? qr[a[q]] : 0u;
      }
    }
    if (W_hat) {
      float* dst = W_hat + r * d + c0;
      if (vec_w && full) {
        const f32x4 lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
        *reinterpret_cast<f32x4*>(dst) = lo;
        *reinterpret_cast<f32x4*>(dst + 4) = hi;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (c0 + q < d) dst[q] = v[q];
      }
    }
    // 8 columns = one word (cpw 8) or two (cpw 4); columns past d pack as 0
    if (cpw == 8) {
      uint32_t word = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) word |= cd[q] << (cwid * q);
      qweight[r * nw + c0 / 8] = word;
    } else {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w0 |= cd[q] << (cwid * q);
        w1 |= cd[4 + q] << (cwid * q);
      }
      qweight[r * nw + c0 / 4] = w0;
      if (c0 + 4 < d) qweight[r * nw + c0 / 4 + 1] = w1;
    }
  }
}

// Outputs in the original column order for rows that fit in LDS (dp ≤
// kFinLds): one row per workgroup step; the working row and its codes are
// staged in LDS with coalesced loads, then each thread gathers its 8-column
// chunks (inv re-read from cache for every row, as in init_rows_kernel),
// writes Ŵ coalesced and packs the codes.  The workgroup that takes row 0
// writes g_idx.
constexpr int kFinLds = 13056;   // floats + code bytes of one row within 64 KB
__global__ __launch_bounds__(256) void finalize_rows_kernel(const float* __restrict__ Wk,
                                                            const uint8_t* __restrict__ codes,
                                                            const int* __restrict__ inv, int64_t m,
                                                            int d, int dp, int bits, int64_t g,
                                                            uint32_t* __restrict__ qweight,
                                                            float* __restrict__ W_hat,
                                                            int32_t* __restrict__ g_idx, int vec_w) {
  extern __shared__ __attribute__((aligned(16))) float row[];
  uint8_t* qrow = reinterpret_cast<uint8_t*>(row + dp);   // dp is a multiple of 128
  const int t = threadIdx.x;
  const int cpw = bits <= 4 ? 8 : 4, cwid = 32 / cpw;
  const int64_t nw = (d + cpw - 1) / cpw;
  if (g_idx && blockIdx.x == 0)
    for (int cc = t; cc < d; cc += 256) g_idx[cc] = (int32_t)(inv[cc] / g);
  for (int64_t r = blockIdx.x; r < m; r += gridDim.x) {
    __syncthreads();
    const float* wr = Wk + r * dp;
    const uint8_t* qr = codes + r * dp;
    // every load of the row and its codes before the first LDS store
    for (int e0 = 0; e0 < dp; e0 += 8192) {
      f32x4 wb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + 1024 * u + 4 * t;
        if (e < dp) wb[u] = *reinterpret_cast<const f32x4*>(wr + e);
      }
      const int eq0 = e0 + 16 * t, eq1 = e0 + 4096 + 16 * t;
      uint4 qb0 = {0u, 0u, 0u, 0u}, qb1 = {0u, 0u, 0u, 0u};
      if (eq0 < dp) qb0 = *reinterpret_cast<const uint4*>(qr + eq0);
      if (eq1 < dp) qb1 = *reinterpret_cast<const uint4*>(qr + eq1);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + 1024 * u + 4 * t;
        if (e < dp) *reinterpret_cast<f32x4*>(row + e) = wb[u];
      }
      if (eq0 < dp) *reinterpret_cast<uint4*>(qrow + eq0) = qb0;
      if (eq1 < dp) *reinterpret_cast<uint4*>(qrow + eq1) = qb1;
    }
    __syncthreads();
    for (int c0 = 8 * t; c0 < d; c0 += 2048) {
      const bool full = c0 + 7 < d;
      int a[8];
      if (full) {   // inv sits 256-byte aligned in the workspace
        const int4 p0 = *reinterpret_cast<const int4*>(inv + c0);
        const int4 p1 = *reinterpret_cast<const int4*>(inv + c0 + 4);
        a[0] = p0.x; a[1] = p0.y; a[2] = p0.z; a[3] = p0.w;
        a[4] = p1.x; a[5] = p1.y; a[6] = p1.z; a[7] = p1.w;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) a[q] = c0 + q < d ? inv[c0 + q] : 0;
      }
      float v[8];
      uint32_t cd[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v[q] = c0 + q < d ? row[a[q]] : 0.f;
        cd[q] = c0 + q < d ? qrow[a[q]] : 0u;
      }
      if (W_hat) {
        float* dst = W_hat + r * d + c0;
        if (vec_w && full) {
          const f32x4 lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
          *reinterpret_cast<f32x4*>(dst) = lo;
          *reinterpret_cast<f32x4*>(dst + 4) = hi;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (c0 + q < d) dst[q] = v[q];
        }
      }
      if (cpw == 8) {
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) word |= cd[q] << (cwid * q);
        qweight[r * nw + c0 / 8] = word;
      } else {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w0 |= cd[q] << (cwid * q);
          w1 |= cd[4 + q] << (cwid * q);
        }
        qweight[r * nw + c0 / 4] = w0;
        if (c0 + 4 < d) qweight[r * nw + c0 / 4 + 1] = w1;
      }
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
      // the rest of the super-block, W[:, b1:se] −= Err_b · U[b, b1:se], in
      // the sweep kernel itself (a ragged block is the last one, so the
      // update always follows a full block)
      const int64_t b1 = b0 + bw;
      const bool fused = b1 < se && bw == kBlock;
      a.Upan = U + b0 * d + b1;
      a.nupd = fused ? (int)(se - b1) : 0;
      {
        TimerScope ts(kTimerSweep, s);
        if ((e = launch_sweep<G>(a, s)) != hipSuccess) return e;
      }
      if (b1 < se && !fused) {  // the rest of the super-block: W[:, b1:se] −= Err_b · U[b, b1:se]
        GemmArgs u{};
        u.M = (int)m; u.N = (int)(se - b1); u.K = bw; u.k_last = bw; u.batch = 1;
        u.alpha = -1.f; u.beta = 1.f;
        u.A = w.Err + (b0 - sb0); u.lda = lde; u.trans_a = false;
        u.B = U + b0 * d + b1; u.ldb = d; u.trans_b = false;
        u.C = w.Wk + b1; u.ldc = dp; u.tri = 0;
        TimerScope ts(kTimerUpdate, s);
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
      TimerScope ts(kTimerUpdate, s);
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
         align_up((size_t)d * 4) + align_up((size_t)dp * 4) + align_up((size_t)kBlock * kBlock * 4) +
         align_up((size_t)m * max_groups(d) * 4) + align_up((size_t)m * max_groups(d)) +
         align_up((size_t)m * 4);
}

// Several layers against one factor: their rows are stacked into one working
// matrix (rows are independent problems sharing H and U), swept together,
// and written back per layer.  Every row's arithmetic is the one a separate
// call would do (the block products' k order does not depend on the row
// count), so the results are bitwise those of separate calls.  With one
// layer the scales, zeros and losses go straight to its outputs.
hipError_t quantize_layers_launch(const LayerIO* L, int n, int64_t d, const float* U,
                                  const int32_t* perm, const uint8_t* dead, const gptq_params& p,
                                  int32_t* g_idx, void* ws, hipStream_t s) {
  int64_t M = 0;
  for (int i = 0; i < n; ++i) M += L[i].m;
  QWs w = carve(ws, M, d);
  const int64_t g = (p.group_size <= 0 || p.group_size >= d) ? d : p.group_size;
  const int ng = (int)ceil_div(d, g);
  const int64_t dp = ceil_div(d, kBlock) * kBlock;
  const bool single = n == 1;
  float* S = single ? L[0].scales : w.S;
  uint8_t* Z = single ? L[0].zeros : w.Z;
  float* RL = single ? L[0].row_loss : w.RL;
  hipError_t e;
  const bool rows_path = perm && dp <= kRowLds;
  if (rows_path) {
    src_index_kernel<<<(unsigned)ceil_div(dp, 256), 256, 0, s>>>(perm, dead, (int)d, (int)dp, w.src,
                                                                 w.inv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  int64_t off = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t m = L[i].m;
    const int esz = L[i].dt == GPTQ_F32 ? 4 : 2;
    const int vec_in = ((uintptr_t)L[i].W % 16 == 0) && ((L[i].ld_w * esz) % 16 == 0);
    const unsigned gy4 = (unsigned)std::min<int64_t>(ceil_div(m, 4), 65535);
    float* rl = RL ? RL + off : nullptr;
    if (rows_path)
      init_rows_kernel<<<(unsigned)std::min<int64_t>(m, 1024), 256, (size_t)dp * 4, s>>>(
          L[i].W, L[i].dt, L[i].ld_w, m, (int)d, (int)dp, w.src, w.Wk + off * dp, rl, vec_in);
    else
      init_kernel<<<dim3((unsigned)ceil_div(dp, 2048), gy4), 256, 0, s>>>(
          L[i].W, L[i].dt, L[i].ld_w, m, d, dp, perm, dead, w.Wk + off * dp, w.inv, rl, vec_in);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    off += m;
  }
  switch (g) {
    case 32: e = run_blocks<32>(w, M, d, U, p, g, ng, S, Z, RL, s); break;
    case 64: e = run_blocks<64>(w, M, d, U, p, g, ng, S, Z, RL, s); break;
    case 128: e = run_blocks<128>(w, M, d, U, p, g, ng, S, Z, RL, s); break;
    default: e = run_blocks<0>(w, M, d, U, p, g, ng, S, Z, RL, s); break;
  }
  if (e != hipSuccess) return e;
  off = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t m = L[i].m;
    const unsigned gy = (unsigned)std::min<int64_t>(m, 65535);
    float* W_hat = L[i].W_hat;
    int32_t* gi = i == 0 ? g_idx : nullptr;
    const int vec_w = W_hat && ((uintptr_t)W_hat % 16 == 0) && (d % 4 == 0);
    if (perm && dp <= kFinLds)
      finalize_rows_kernel<<<(unsigned)std::min<int64_t>(m, 1024), 256, (size_t)dp * 5, s>>>(
          w.Wk + off * dp, w.codes + off * dp, w.inv, m, (int)d, (int)dp, p.bits, g, L[i].qweight,
          W_hat, gi, vec_w);
    else
      finalize_kernel<<<dim3((unsigned)ceil_div(d, 2048), gy), 256, 0, s>>>(
          w.Wk + off * dp, w.codes + off * dp, w.inv, m, d, dp, p.bits, g, L[i].qweight, W_hat, gi,
          vec_w, perm ? 0 : 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!single) {
      e = hipMemcpyAsync(L[i].scales, w.S + off * ng, (size_t)m * ng * 4, hipMemcpyDeviceToDevice, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(L[i].zeros, w.Z + off * ng, (size_t)m * ng, hipMemcpyDeviceToDevice, s);
      if (e == hipSuccess && L[i].row_loss)
        e = hipMemcpyAsync(L[i].row_loss, w.RL + off, (size_t)m * 4, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return e;
    }
    off += m;
  }
  return hipSuccess;
}

hipError_t quantize_launch(const void* W, int w_dtype, int64_t m, int64_t d, int64_t ld_w,
                           const float* U, const int32_t* perm, const uint8_t* dead,
                           const gptq_params& p, uint32_t* qweight, float* scales,
                           uint8_t* zeros, float* W_hat, int32_t* g_idx, float* row_loss,
                           void* ws, hipStream_t s) {
  const LayerIO one{W, w_dtype, m, ld_w, qweight, scales, zeros, W_hat, row_loss};
  return quantize_layers_launch(&one, 1, d, U, perm, dead, p, g_idx, ws, s);
}

}  // namespace gq
