// Optimal Brain Quantization with the greedy order, the comparator for
// GPTQ's fixed order on tiny layers ("GPTQ: Mathematical Foundations ...":
// Optimal Brain Surgeon (OBS) and Optimal Brain Quantization (OBQ),
// Lagrangian Derivation, Minimal Error Penalty, Recursive Inverse Hessian
// Updating, The Computational Bottleneck of OBQ; The GPTQ Algorithmic
// Innovations §1 for the fixed-order alternative).
//
// Per row, with F the free columns and H_F⁻¹ their inverse Hessian:
//   ΔE_c = (w_c − quant(w_c))² / (2·[H_F⁻¹]_cc) for every c in F;
//   q = argmin ΔE (the lower index on ties);
//   w_F −= (w_q − quant(w_q)) / [H_F⁻¹]_qq · (H_F⁻¹)_{F,q},  w_q := quant(w_q);
//   H_{F∖q}⁻¹ = H_F⁻¹ − (H_F⁻¹)_{:,q}(H_F⁻¹)_{q,:} / [H_F⁻¹]_qq on F∖q.
// quant() is one grid per row from the row's own dead-fixed weights (the
// grid GPTQ uses with one group per row).  Every row has its own order and
// its own copy of H_F⁻¹ (d² doubles), so the work is O(d³) per row: the
// bottleneck the pages describe, run here on d_in <= 128 in fp64 (the
// comparator's job is to be exact, not fast).
//
// obq_inverse_kernel: dead fix, damping, H_d⁻¹ by an in-LDS Gauss-Jordan
//   sweep (no pivoting: H_d is positive definite; a non-positive pivot is
//   reported).  One workgroup.
// obq_row_kernel: one workgroup per row; H_F⁻¹ lives in LDS; thread t owns
//   column t's saliency, and the downdate is spread over all threads.
#include <cfloat>
#include <climits>

#include "common.hpp"

namespace gq {
namespace {

constexpr int kObqMax = 128;   // largest d_in (H_F⁻¹ of 128² doubles = 128 KB of LDS)
constexpr int kObqLd = kObqMax + 1;

__global__ __launch_bounds__(256) void obq_inverse_kernel(const float* __restrict__ H, int d,
                                                          float percdamp, double* __restrict__ Hinv,
                                                          uint8_t* __restrict__ dead,
                                                          int* __restrict__ status) {
  __shared__ double A[kObqMax * kObqLd];
  __shared__ double red[256];
  __shared__ double prow[kObqMax];
  __shared__ double pcol[kObqMax];
  const int t = threadIdx.x;
  // dead fix, then λ = percdamp·mean(diag) (the mean includes the fixed 1s)
  double acc = 0.0;
  for (int i = t; i < d; i += 256) {
    double h = (double)H[(int64_t)i * d + i];
    const bool dd = h == 0.0;
    dead[i] = dd ? 1 : 0;
    acc += dd ? 1.0 : h;
  }
  red[t] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  const double lam = (double)percdamp * (red[0] / d);
  for (int e = t; e < d * d; e += 256) {
    const int i = e / d, j = e % d;
    double h = (double)H[(int64_t)i * d + j];
    if (i == j) h = (h == 0.0 ? 1.0 : h) + lam;
    A[i * kObqLd + j] = h;
  }
  if (t == 0) status[0] = INT_MAX;
  __syncthreads();
  // Gauss-Jordan: after step k, columns < k+1 of A hold the inverse's part
  for (int k = 0; k < d; ++k) {
    const double piv = A[k * kObqLd + k];
    const bool bad = !(piv > 0.0) || !(piv < DBL_MAX);
    const double ip = bad ? 1.0 : 1.0 / piv;
    if (bad && t == 0) atomicMin(status, k);
    for (int j = t; j < d; j += 256) {
      prow[j] = (j == k) ? ip : A[k * kObqLd + j] * ip;
      pcol[j] = A[j * kObqLd + k];
    }
    __syncthreads();
    for (int e = t; e < d * d; e += 256) {
      const int i = e / d, j = e % d;
      if (i == k) continue;
      const double f = pcol[i];
      A[i * kObqLd + j] = (j == k) ? -f * ip : A[i * kObqLd + j] - f * prow[j];
    }
    __syncthreads();
    for (int j = t; j < d; j += 256) A[k * kObqLd + j] = prow[j];
    __syncthreads();
  }
  // symmetrize (as the oracle does with its LAPACK inverse)
  for (int e = t; e < d * d; e += 256) {
    const int i = e / d, j = e % d;
    Hinv[e] = 0.5 * (A[i * kObqLd + j] + A[j * kObqLd + i]);
  }
}

__device__ __forceinline__ double load_w64(const void* W, int dt, int64_t i) {
  if (dt == GPTQ_F32) return (double)static_cast<const float*>(W)[i];
  const uint16_t b = static_cast<const uint16_t*>(W)[i];
  if (dt == GPTQ_BF16) return (double)__uint_as_float((uint32_t)b << 16);
  return (double)(float)__builtin_bit_cast(_Float16, b);
}

struct ObqArgs {
  const void* W; int dt; int64_t m; int d; int64_t ld_w;
  const double* Hinv; const uint8_t* dead;
  int maxq, sym;
  uint32_t* qweight; float* scales; uint8_t* zeros; float* W_hat; int32_t* order;
  float* row_loss;
};

__global__ __launch_bounds__(256) void obq_row_kernel(ObqArgs a) {
  __shared__ double Hi[kObqMax * kObqLd];
  __shared__ double w[kObqMax];
  __shared__ double col[kObqMax];
  __shared__ double rv[8];
  __shared__ int ri[8];
  __shared__ int code[kObqMax];
  __shared__ int ord[kObqMax];
  __shared__ unsigned char freef[kObqMax];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int d = a.d;
  const int64_t r = blockIdx.x;
  for (int e = t; e < d * d; e += 256) Hi[(e / d) * kObqLd + e % d] = a.Hinv[e];
  if (t < d) {
    w[t] = a.dead[t] ? 0.0 : load_w64(a.W, a.dt, r * a.ld_w + t);
    freef[t] = 1;
  }
  __syncthreads();
  // the row's grid, from its dead-fixed weights
  double mn = DBL_MAX, mx = -DBL_MAX, am = 0.0;
  if (t < d) { mn = w[t]; mx = w[t]; am = fabs(w[t]); }
  for (int o = 32; o > 0; o >>= 1) {
    mn = fmin(mn, __shfl_xor(mn, o));
    mx = fmax(mx, __shfl_xor(mx, o));
    am = fmax(am, __shfl_xor(am, o));
  }
  if (lane == 0) { rv[wv] = mn; rv[4 + wv] = mx; col[wv] = am; }
  __syncthreads();
  mn = fmin(fmin(rv[0], rv[1]), fmin(rv[2], rv[3]));
  mx = fmax(fmax(rv[4], rv[5]), fmax(rv[6], rv[7]));
  am = fmax(fmax(col[0], col[1]), fmax(col[2], col[3]));
  const double fq = (double)a.maxq;
  double s, z;
  if (a.sym) {
    s = am / (double)((a.maxq + 1) / 2 - 1);
    if (!(s > 0.0)) s = 1.0;
    z = (double)((a.maxq + 1) / 2);
  } else {
    s = (mx - mn) / fq;
    if (s == 0.0) s = mn != 0.0 ? fabs(mn) : 1.0;
    z = fmin(fmax(rint(-mn / s), 0.0), fq);
  }
  double loss = 0.0;   // Σ ΔE of the row (thread 0)
  __syncthreads();
  for (int step = 0; step < d; ++step) {
    // saliency of every free column; argmin with the lower index on ties
    double best = DBL_MAX;
    int bi = INT_MAX;
    if (t < d && freef[t]) {
      const double wt = w[t];
      const double q = fmin(fmax(rint(wt / s + z), 0.0), fq);
      const double df = wt - s * (q - z);
      best = df * df / (2.0 * Hi[t * kObqLd + t]);
      bi = t;
    }
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oi = __shfl_xor(bi, o);
      if (ob < best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    if (lane == 0) { rv[wv] = best; ri[wv] = bi; }
    __syncthreads();
    best = rv[0]; bi = ri[0];
    for (int u = 1; u < 4; ++u)
      if (rv[u] < best || (rv[u] == best && ri[u] < bi)) { best = rv[u]; bi = ri[u]; }
    const int q = bi;
    const double wq = w[q];
    const double qc = fmin(fmax(rint(wq / s + z), 0.0), fq);
    const double quant = s * (qc - z);
    const double hqq = Hi[q * kObqLd + q];
    const double coef = (wq - quant) / hqq;
    if (t < d) col[t] = Hi[t * kObqLd + q];
    if (t == 0) {
      loss += (wq - quant) * (wq - quant) / (2.0 * hqq);
      code[q] = (int)qc;
      ord[step] = q;
    }
    __syncthreads();   // everyone has q's column and the step's values
    if (t < d && freef[t]) w[t] = (t == q) ? quant : w[t] - coef * col[t];
    if (t == q) freef[t] = 0;
    __syncthreads();
    // downdate on F∖q; q's row and column are never read again
    for (int e = t; e < d * d; e += 256) {
      const int i = e / d, j = e % d;
      if (freef[i] && freef[j]) Hi[i * kObqLd + j] -= col[i] * col[j] / hqq;
    }
    __syncthreads();
  }
  // outputs: codes in the quantize container (8 per word up to 4 bits, else 4)
  const int cpw = a.maxq <= 15 ? 8 : 4, cw = 32 / cpw;
  const int nw = (d + cpw - 1) / cpw;
  if (t < nw) {
    uint32_t word = 0;
    for (int u = 0; u < cpw; ++u) {
      const int c = t * cpw + u;
      if (c < d) word |= (uint32_t)code[c] << (cw * u);
    }
    a.qweight[r * nw + t] = word;
  }
  if (t < d) {
    // Ŵ from the stored fp32 scale, as the quantize path writes it
    if (a.W_hat) a.W_hat[r * d + t] = (float)s * ((float)code[t] - (float)z);
    if (a.order) a.order[r * d + t] = ord[t];
  }
  if (t == 0) {
    a.scales[r] = (float)s;
    a.zeros[r] = (uint8_t)z;
    if (a.row_loss) a.row_loss[r] = (float)loss;
  }
}

}  // namespace

int obq_max_din() { return kObqMax; }

size_t obq_ws_bytes(int64_t d) { return 256 + align_up((size_t)d * d * 8) + align_up((size_t)d); }

hipError_t obq_launch(const void* W, int w_dtype, int64_t m, int64_t d, int64_t ld_w,
                      const float* H, const gptq_params& p, uint32_t* qweight, float* scales,
                      uint8_t* zeros, float* W_hat, int32_t* order, float* row_loss, void* ws,
                      int32_t** status_dev, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  int* status = reinterpret_cast<int*>(base);
  double* Hinv = reinterpret_cast<double*>(base + 256);
  uint8_t* dead = reinterpret_cast<uint8_t*>(base + 256 + align_up((size_t)d * d * 8));
  *status_dev = status;
  obq_inverse_kernel<<<1, 256, 0, s>>>(H, (int)d, p.percdamp, Hinv, dead, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ObqArgs a{W, w_dtype, m, (int)d, ld_w, Hinv, dead, (1 << p.bits) - 1, p.sym,
            qweight, scales, zeros, W_hat, order, row_loss};
  obq_row_kernel<<<(unsigned)m, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace gq
