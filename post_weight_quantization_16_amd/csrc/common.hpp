// Internal declarations shared by the library's HIP translation units.
// Nothing here is part of the public C ABI (include/gptq.h).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "gptq.h"

namespace gq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kBlock = 128;   // lazy-update block width B used by this library
constexpr int kPanel = 64;    // Cholesky panel width
constexpr int kSuper = 4;     // blocks per super-block of the two-level lazy update

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Per-group quantizer parameters ("INT4 and GPTQ Quantization": Uniform INT4
// Quantization, Group Quantization; "Quantization (INT8, INT4, GPTQ)":
// Deriving the scale and zero-point).  Asymmetric: s = (max − min)/(2ᵇ−1),
// z = clamp(rint(−min/s), 0, 2ᵇ−1); a constant group gets s = |min| (1 when
// it is 0).  Symmetric: s = max|w|/(2ᵇ⁻¹−1) (1 for an all-zero group),
// z = 2ᵇ⁻¹ (unsigned storage).
__device__ __forceinline__ void group_qparams(float mn, float mx, float amax, int maxq, int sym,
                                              float& s, float& z) {
  if (sym) {
    s = amax / (float)((maxq + 1) / 2 - 1);
    if (!(s > 0.f)) s = 1.f;
    z = (float)((maxq + 1) / 2);
  } else {
    s = (mx - mn) / (float)maxq;
    if (s == 0.f) s = (mn != 0.f) ? fabsf(mn) : 1.f;
    z = fminf(fmaxf(rintf(-mn / s), 0.f), (float)maxq);
  }
}
inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- fp32 GEMM
// C = beta*C + alpha * op(A) * op(B), fp32 MFMA (v_mfma_f32_32x32x2f32),
// batched over blockIdx.z with element strides.  op(A)(m,k) = A[m*lda+k], or
// A[k*lda+m] when trans_a; op(B)(k,n) = B[k*ldb+n], or B[n*ldb+k] when trans_b.
// tri: 0 full, 1 only n <= m is written (lower), 2 only n >= m (upper); tiles
// entirely outside the triangle are skipped.  k_last: K of the last batch
// (split-K over one long dimension), or K when all batches are equal.
// k_from_n: op(B) is lower triangular (B(k,n) = 0 for k < n), so a tile at
// column n0 starts its K loop at n0.  k_to_m: op(A) is lower triangular
// (A(m,k) = 0 for k > m), so a tile at row m0 stops at m0 + 128.
struct GemmArgs {
  int M, N, K, k_last, batch;
  int k_from_n, k_to_m;
  float alpha, beta;
  const float* A; int64_t lda, strideA; bool trans_a;
  const float* B; int64_t ldb, strideB; bool trans_b;
  float* C; int64_t ldc, strideC;
  int tri;
};
hipError_t gemm_f32(const GemmArgs& g, hipStream_t s);

// ---------------------------------------------------------------- Hessian
int hessian_splits(int64_t d, int64_t n_tok);
size_t hessian_ws_bytes(int64_t d, int64_t n_tok);
// smallest workspace the Hessian runs with (one partial Hessian)
size_t hessian_min_ws_bytes(int64_t d);
// overwrite: H = 2·XᵀX instead of H += 2·XᵀX (H is not read)
hipError_t hessian_launch(float* H, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                          int64_t ld_x, void* ws, size_t ws_bytes, hipStream_t s,
                          bool overwrite = false);
// the same with the library's static device scratch as the workspace (no
// allocation); ERR: hipErrorInvalidValue when d needs more than it holds
constexpr size_t kScratchBytes = (size_t)65 << 20;
hipError_t hessian_launch_static(float* H, int64_t d, const void* X, int x_dtype, int64_t n_tok,
                                 int64_t ld_x, hipStream_t s);

// ---------------------------------------------------------------- prepare
size_t prepare_ws_bytes(int64_t d);
// Runs dead fix, damping, act-order, blocked Cholesky and triangular inverse.
// Leaves the failing pivot (or -1) in the device int at *status_dev.
hipError_t prepare_launch(float* H, int64_t d, float percdamp, int act_order, float* U,
                          int32_t* perm, uint8_t* dead_mask, void* ws, int32_t** status_dev,
                          hipStream_t s);

// ---------------------------------------------------------------- quantize
// One block of the sweep (sweep.hip, one object per group-size variant G).
struct SweepArgs {
  float* Wk; int64_t ldw;        // working weights [m x ldw], block at column b0
  int64_t m, b0; int bw;          // rows, block start, real columns in the block
  const float* Ublk; int64_t ldu; // U's diagonal block for this block (row j at Ublk + j*ldu)
  int maxq, sym;
  float* scales; uint8_t* zeros; int ng; int64_t g;
  float* Err; int64_t lde;        // the block's errors: [m x 128] at Err, row stride lde
  uint8_t* codes;                 // [m x ldw]
  float* row_loss;                // may be null
  // the rest of the super-block, updated by the same kernel after the sweep:
  // W[:, b0+128 : b0+128+nupd] −= Err·U[block, b0+128 : ...] with U's panel
  // row j at Upan + j*ldu (nupd = 0: none; only for full blocks)
  const float* Upan; int nupd;
};
template <int G> hipError_t launch_sweep(const SweepArgs& a, hipStream_t s);
template <> hipError_t launch_sweep<0>(const SweepArgs& a, hipStream_t s);
template <> hipError_t launch_sweep<32>(const SweepArgs& a, hipStream_t s);
template <> hipError_t launch_sweep<64>(const SweepArgs& a, hipStream_t s);
template <> hipError_t launch_sweep<128>(const SweepArgs& a, hipStream_t s);

size_t quantize_ws_bytes(int64_t m, int64_t d);
// one layer of a multi-layer call (all layers share d_in, U, perm and dead)
struct LayerIO {
  const void* W; int dt; int64_t m, ld_w;
  uint32_t* qweight; float* scales; uint8_t* zeros; float* W_hat; float* row_loss;
};
hipError_t quantize_layers_launch(const LayerIO* L, int n, int64_t d, const float* U,
                                  const int32_t* perm, const uint8_t* dead, const gptq_params& p,
                                  int32_t* g_idx, void* ws, hipStream_t s);
hipError_t quantize_launch(const void* W, int w_dtype, int64_t m, int64_t d, int64_t ld_w,
                           const float* U, const int32_t* perm, const uint8_t* dead,
                           const gptq_params& p, uint32_t* qweight, float* scales,
                           uint8_t* zeros, float* W_hat, int32_t* g_idx, float* row_loss,
                           void* ws, hipStream_t s);

// ---------------------------------------------------------------- stage timing
// (diagnostics, timing.hip): a scope records a HIP event pair around the
// launches it encloses while timing is enabled.
enum { kTimerUpdate = 0, kTimerSweep = 1, kTimerChol = 2, kTimerInverse = 3, kTimerHessian = 4,
       kTimerLead = 5, kTimerCount = 6 };
class TimerScope {
 public:
  TimerScope(int which, hipStream_t s);
  ~TimerScope();
  TimerScope(const TimerScope&) = delete;
  TimerScope& operator=(const TimerScope&) = delete;
 private:
  int which_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr;
};
int timing_enable(int on);
hipError_t timing_read(float* ms, int n);

// ---------------------------------------------------------------- OBQ comparator
int obq_max_din();
size_t obq_ws_bytes(int64_t d);
hipError_t obq_launch(const void* W, int w_dtype, int64_t m, int64_t d, int64_t ld_w,
                      const float* H, const gptq_params& p, uint32_t* qweight, float* scales,
                      uint8_t* zeros, float* W_hat, int32_t* order, float* row_loss, void* ws,
                      int32_t** status_dev, hipStream_t s);

// ---------------------------------------------------------------- W4A16 inference
hipError_t w4a16_launch(const void* A, int a_dtype, int64_t M, int64_t K, int64_t lda,
                        const uint32_t* qweight, int bits, const uint16_t* s16, const uint16_t* z16,
                        const int32_t* g_idx, int64_t g, int64_t ng, int64_t N, float* C,
                        int64_t ldc, void* ws, size_t ws_bytes, hipStream_t s);
size_t w4a16_ws_bytes(int64_t M, int64_t N, int64_t K);

// ---------------------------------------------------------------- export
hipError_t export_launch(int bits, int64_t m, int64_t d, int64_t ng, const uint32_t* qweight,
                         const float* scales, const uint8_t* zeros, uint32_t* qdense,
                         uint16_t* s16, uint16_t* z16, hipStream_t s);

}  // namespace gq
