// Storage export of a quantized layer ("GPTQ: Mathematical Foundations ...":
// Quantization Formats and Group Size -- b bits per weight plus a 16-bit
// scale and a 16-bit zero per group; Inference Execution -- codes packed
// into 32-bit words).
//
// Input: the outputs of gptq_quantize_layer (codes in their word container:
// eight per 32-bit word for b <= 4, four for b = 8; fp32 scales; 8-bit
// zeros).  Output: the dense layout, one little-endian bit stream per row in
// which the code of column c occupies bits [c·b, c·b + b) (for b = 3, 32
// codes fill three words), and the scales and zeros as IEEE half precision
// (round to nearest even; zeros are small integers and convert exactly).
// HBM-bound: every output word is written once, its source words read once
// per output word that needs them (from cache).
#include "common.hpp"

namespace gq {
namespace {

// code c of a row in the container layout
__device__ __forceinline__ uint32_t container_code(const uint32_t* __restrict__ row, int64_t c,
                                                   int bits) {
  if (bits == 8) return (row[c >> 2] >> (8 * (c & 3))) & 0xFFu;
  return (row[c >> 3] >> (4 * (c & 7))) & 0xFu;
}

// One dense output word per thread: word w of row r holds the bits
// [32w, 32w + 32) of the row's stream, i.e. parts of codes
// floor(32w / b) .. floor((32w + 31) / b).
__global__ __launch_bounds__(256) void dense_kernel(const uint32_t* __restrict__ qw, int64_t m,
                                                    int64_t d, int bits, int64_t nw_in,
                                                    int64_t nw_out, uint32_t* __restrict__ out) {
  const int64_t w = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (w >= nw_out) return;
  const int64_t p0 = 32 * w;
  const int64_t c0 = p0 / bits, c1 = min(d - 1, (p0 + 31) / bits);
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    const uint32_t* row = qw + r * nw_in;
    uint64_t acc = 0;   // bits from stream position c0·b on
    for (int64_t c = c0; c <= c1; ++c)
      acc |= (uint64_t)container_code(row, c, bits) << (int)(c * bits - c0 * bits);
    out[r * nw_out + w] = (uint32_t)(acc >> (int)(p0 - c0 * bits));
  }
}

__global__ __launch_bounds__(256) void half_meta_kernel(const float* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros,
                                                        int64_t n, uint16_t* __restrict__ s16,
                                                        uint16_t* __restrict__ z16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    if (s16) s16[i] = __builtin_bit_cast(uint16_t, (_Float16)scales[i]);
    if (z16) z16[i] = __builtin_bit_cast(uint16_t, (_Float16)(float)zeros[i]);
  }
}

}  // namespace

hipError_t export_launch(int bits, int64_t m, int64_t d, int64_t ng, const uint32_t* qweight,
                         const float* scales, const uint8_t* zeros, uint32_t* qdense,
                         uint16_t* s16, uint16_t* z16, hipStream_t s) {
  if (qdense) {
    const int64_t nw_in = bits == 8 ? ceil_div(d, 4) : ceil_div(d, 8);
    const int64_t nw_out = ceil_div(d * bits, 32);
    const dim3 grid((unsigned)ceil_div(nw_out, 256), (unsigned)std::min<int64_t>(m, 65535));
    dense_kernel<<<grid, 256, 0, s>>>(qweight, m, d, bits, nw_in, nw_out, qdense);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (s16 || z16) {
    const int64_t n = m * ng;
    half_meta_kernel<<<(unsigned)std::min<int64_t>(ceil_div(n, 256), 65535), 256, 0, s>>>(
        scales, zeros, n, s16, z16);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gq
