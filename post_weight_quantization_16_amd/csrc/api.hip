// C ABI entry points (include/gptq.h): argument validation, workspace sizing,
// launch sequencing and error reporting.  Every check runs before the first
// HIP call, so invalid arguments never touch the device.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "common.hpp"

namespace {

thread_local std::string g_err = "no error";

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(const char* where, hipError_t e) {
  return fail(GPTQ_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

constexpr int64_t kMaxDin = 65536;
constexpr int64_t kMaxDout = int64_t(1) << 24;

bool valid_dtype(int dt) { return dt == GPTQ_F32 || dt == GPTQ_BF16 || dt == GPTQ_F16; }

// Checks the quantizer parameters for a layer with d_in columns.
int check_params(const gptq_params* p, int64_t d_in) {
  if (!p) return fail(GPTQ_ERR_INVALID_ARG, "params is NULL");
  if (p->bits != 2 && p->bits != 3 && p->bits != 4 && p->bits != 8)
    return fail(GPTQ_ERR_INVALID_ARG, "bits must be 2, 3, 4 or 8 (got %d)", p->bits);
  if (p->group_size == 0 || p->group_size < -1)
    return fail(GPTQ_ERR_INVALID_ARG, "group_size must be > 0 or -1 (got %d)", p->group_size);
  if (p->block_size <= 0)
    return fail(GPTQ_ERR_INVALID_ARG, "block_size must be > 0 (got %d)", p->block_size);
  if (!(p->percdamp >= 0.f) || !std::isfinite(p->percdamp))
    return fail(GPTQ_ERR_INVALID_ARG, "percdamp must be finite and >= 0");
  if (p->act_order != 0 && p->act_order != 1)
    return fail(GPTQ_ERR_INVALID_ARG, "act_order must be 0 or 1");
  if (p->sym != 0 && p->sym != 1) return fail(GPTQ_ERR_INVALID_ARG, "sym must be 0 or 1");
  if (p->block_size != gq::kBlock)
    return fail(GPTQ_ERR_UNSUPPORTED, "block_size %d: this library runs B = %d", p->block_size,
                gq::kBlock);
  if (d_in > 0) {
    const int64_t g = (p->group_size < 0 || p->group_size >= d_in) ? d_in : p->group_size;
    const bool ok = g == d_in || g % gq::kBlock == 0 || g == 32 || g == 64;
    if (!ok)
      return fail(GPTQ_ERR_UNSUPPORTED,
                  "group_size %lld with block %d: groups must start on block starts or lie "
                  "inside blocks (g in {32,64} or a multiple of %d, or one group per row)",
                  (long long)g, gq::kBlock, gq::kBlock);
  }
  return GPTQ_OK;
}

int check_ws(void* ws, size_t have, size_t need, const char* what) {
  if (need && !ws) return fail(GPTQ_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", what, need);
  if (have < need)
    return fail(GPTQ_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", what, have, need);
  if ((uintptr_t)ws % 256)
    return fail(GPTQ_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", what);
  return GPTQ_OK;
}

}  // namespace

extern "C" {

const char* gptq_last_error(void) { return g_err.c_str(); }

const char* gptq_version(void) { return "gptq_mi355x 0.1.0 (gfx950)"; }

size_t gptq_workspace_bytes(int which, int64_t d_out, int64_t d_in, int64_t n_tok,
                            const gptq_params* p) {
  if (d_in <= 0 || d_in > kMaxDin) return 0;
  switch (which) {
    case GPTQ_WS_HESSIAN:
      if (n_tok < 0) return 0;
      return n_tok == 0 ? 256 : gq::hessian_ws_bytes(d_in, n_tok);
    case GPTQ_WS_PREPARE:
      return gq::prepare_ws_bytes(d_in);
    case GPTQ_WS_QUANTIZE:
      if (d_out <= 0 || d_out > kMaxDout) return 0;
      (void)p;
      return gq::quantize_ws_bytes(d_out, d_in);
    default:
      return 0;
  }
}

int gptq_hessian_accumulate(float* H, int64_t d_in, const void* X, int x_dtype, int64_t n_tok,
                            int64_t ld_x, void* ws, size_t ws_bytes, gptq_stream stream) {
  if (!H) return fail(GPTQ_ERR_INVALID_ARG, "H is NULL");
  if (d_in <= 0 || d_in > kMaxDin)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in must be in [1, %lld] (got %lld)", (long long)kMaxDin,
                (long long)d_in);
  if (n_tok < 0) return fail(GPTQ_ERR_INVALID_ARG, "n_tok must be >= 0");
  if (!valid_dtype(x_dtype)) return fail(GPTQ_ERR_INVALID_ARG, "unknown x_dtype %d", x_dtype);
  if (n_tok == 0) return GPTQ_OK;
  if (!X) return fail(GPTQ_ERR_INVALID_ARG, "X is NULL");
  if (ld_x < d_in) return fail(GPTQ_ERR_INVALID_ARG, "ld_x (%lld) < d_in (%lld)", (long long)ld_x,
                               (long long)d_in);
  int rc = check_ws(ws, ws_bytes, gq::hessian_ws_bytes(d_in, n_tok), "hessian_accumulate");
  if (rc) return rc;
  hipError_t e = gq::hessian_launch(H, d_in, X, x_dtype, n_tok, ld_x, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("hessian_accumulate", e);
  return GPTQ_OK;
}

int gptq_prepare_hinv(float* H, int64_t d_in, const gptq_params* p, float* U, int32_t* perm,
                      uint8_t* dead_mask, void* ws, size_t ws_bytes, int64_t* info,
                      gptq_stream stream) {
  if (info) *info = -1;
  if (!H || !U) return fail(GPTQ_ERR_INVALID_ARG, "H and U must not be NULL");
  if (d_in <= 0 || d_in > kMaxDin)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in must be in [1, %lld]", (long long)kMaxDin);
  int rc = check_params(p, d_in);
  if (rc) return rc;
  if (p->act_order && !perm) return fail(GPTQ_ERR_INVALID_ARG, "act_order needs a perm output");
  rc = check_ws(ws, ws_bytes, gq::prepare_ws_bytes(d_in), "prepare_hinv");
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  int32_t* status_dev = nullptr;
  hipError_t e = gq::prepare_launch(H, d_in, p->percdamp, p->act_order, U, perm, dead_mask, ws,
                                    &status_dev, s);
  if (e != hipSuccess) return hip_fail("prepare_hinv", e);
  int32_t st = 0;
  e = hipMemcpyAsync(&st, status_dev, sizeof st, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail("prepare_hinv (status read-back)", e);
  if (st != INT_MAX) {
    const int64_t piv = d_in - 1 - (int64_t)st;
    if (info) *info = piv;
    return fail(GPTQ_ERR_NOT_SPD,
                "damped Hessian is not positive definite (pivot %lld of the quantization order); "
                "raise percdamp",
                (long long)piv);
  }
  return GPTQ_OK;
}

int gptq_quantize_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ld_w,
                        const float* U, const int32_t* perm, const uint8_t* dead_mask,
                        const gptq_params* p, uint32_t* qweight, float* scales, uint8_t* zeros,
                        float* W_hat, int32_t* g_idx, float* row_loss, void* ws, size_t ws_bytes,
                        gptq_stream stream) {
  if (!W || !U || !qweight || !scales || !zeros)
    return fail(GPTQ_ERR_INVALID_ARG, "W, U, qweight, scales and zeros must not be NULL");
  if (!valid_dtype(w_dtype)) return fail(GPTQ_ERR_INVALID_ARG, "unknown w_dtype %d", w_dtype);
  if (d_in <= 0 || d_in > kMaxDin)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in must be in [1, %lld]", (long long)kMaxDin);
  if (d_out <= 0 || d_out > kMaxDout)
    return fail(GPTQ_ERR_INVALID_ARG, "d_out must be in [1, %lld]", (long long)kMaxDout);
  if (ld_w < d_in) return fail(GPTQ_ERR_INVALID_ARG, "ld_w < d_in");
  int rc = check_params(p, d_in);
  if (rc) return rc;
  rc = check_ws(ws, ws_bytes, gq::quantize_ws_bytes(d_out, d_in), "quantize_layer");
  if (rc) return rc;
  hipError_t e = gq::quantize_launch(W, w_dtype, d_out, d_in, ld_w, U, perm, dead_mask, *p,
                                     qweight, scales, zeros, W_hat, g_idx, row_loss, ws,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("quantize_layer", e);
  return GPTQ_OK;
}

}  // extern "C"
