// C ABI entry points (include/gptq.h): argument validation, workspace sizing,
// launch sequencing and error reporting.  Every check runs before the first
// HIP call, so invalid arguments never touch the device.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"
#include "status_map.hpp"

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

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

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

// One job of gptq_quantize_independent: the Hessian uses the whole workspace
// (as much as gptq_hessian_accumulate would), the preparation its first part
// and the quantization the part after it, so the preparation's status words
// are still there when the job is done.
size_t layer_prep_bytes(int64_t d) { return (gq::prepare_ws_bytes(d) + 255) / 256 * 256; }
size_t layer_ws_bytes(int64_t m, int64_t d, int64_t n_tok) {
  const size_t h = n_tok > 0 ? gq::hessian_ws_bytes(d, n_tok) : 0;
  const size_t pq = layer_prep_bytes(d) + gq::quantize_ws_bytes(m, d);
  return h > pq ? h : pq;
}

// Streams the independent jobs run on, per device, created on first use and
// kept until the process ends (default priority, not synchronizing with the
// null stream), with an event to fork from the caller's stream and one per
// stream to join back.  A call holds the device's lock while it enqueues.
constexpr int kJobStreams = 8;
struct JobStreams {
  hipStream_t s[kJobStreams] = {};
  hipEvent_t fork = nullptr, join[kJobStreams] = {};
  std::mutex mu;
  hipError_t err = hipSuccess;
};

JobStreams* job_streams(int dev) {
  static std::mutex map_mu;
  static std::map<int, JobStreams*> pools;
  std::lock_guard<std::mutex> g(map_mu);
  auto it = pools.find(dev);
  if (it != pools.end()) return it->second;
  JobStreams* js = new JobStreams();
  hipError_t e = hipEventCreateWithFlags(&js->fork, hipEventDisableTiming);
  for (int i = 0; i < kJobStreams && e == hipSuccess; ++i) {
    e = hipStreamCreateWithFlags(&js->s[i], hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&js->join[i], hipEventDisableTiming);
  }
  js->err = e;
  pools[dev] = js;
  return js;
}

}  // namespace

namespace {
// Checks and enqueues the preparation; status_dev receives the device
// address of its two status words.
int prepare_enqueue(float* H, int64_t d_in, const gptq_params* p, float* U, int32_t* perm,
                    uint8_t* dead_mask, void* ws, size_t ws_bytes, int32_t** status_dev,
                    hipStream_t s) {
  if (!H || !U) return fail(GPTQ_ERR_INVALID_ARG, "H and U must not be NULL");
  if (d_in <= 0 || d_in > kMaxDin)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in must be in [1, %lld]", (long long)kMaxDin);
  int rc = check_params(p, d_in);
  if (rc) return rc;
  if (p->act_order && !perm) return fail(GPTQ_ERR_INVALID_ARG, "act_order needs a perm output");
  rc = check_ws(ws, ws_bytes, gq::prepare_ws_bytes(d_in), "prepare_hinv");
  if (rc) return rc;
  hipError_t e = gq::prepare_launch(H, d_in, p->percdamp, p->act_order, U, perm, dead_mask, ws,
                                    status_dev, s);
  if (e != hipSuccess) return hip_fail("prepare_hinv", e);
  return GPTQ_OK;
}

int status_result(const int32_t* st, int64_t d_in, int64_t* info) {
  int64_t piv = -1;
  const int rc = gq::prepare_status(st[0], st[1], d_in, &piv);
  if (info) *info = piv;
  if (rc == GPTQ_ERR_NOT_SPD)
    return fail(GPTQ_ERR_NOT_SPD,
                "damped Hessian is not positive definite (pivot %lld of the quantization order); "
                "raise percdamp",
                (long long)piv);
  if (rc != GPTQ_OK)
    return fail(rc, "prepare_hinv: a factorization wave ran out of its bounded wait for "
                    "another wave (status words %d, %d); the outputs are undefined",
                (int)st[0], (int)st[1]);
  return GPTQ_OK;
}
}  // namespace

namespace {
int hessian_call(float* H, int64_t d_in, const void* X, int x_dtype, int64_t n_tok, int64_t ld_x,
                 void* ws, size_t ws_bytes, gptq_stream stream, bool overwrite) {
  if (!H) return fail(GPTQ_ERR_INVALID_ARG, "H is NULL");
  if (d_in <= 0 || d_in > kMaxDin)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in must be in [1, %lld] (got %lld)", (long long)kMaxDin,
                (long long)d_in);
  if (n_tok < 0) return fail(GPTQ_ERR_INVALID_ARG, "n_tok must be >= 0");
  if (!valid_dtype(x_dtype)) return fail(GPTQ_ERR_INVALID_ARG, "unknown x_dtype %d", x_dtype);
  if (n_tok == 0 && !overwrite) return GPTQ_OK;
  if (n_tok == 0) {   // H = 0
    const hipError_t e = gq::hessian_launch(H, d_in, nullptr, x_dtype, 0, d_in, nullptr, 0,
                                            (hipStream_t)stream, true);
    return e == hipSuccess ? GPTQ_OK : hip_fail("hessian", e);
  }
  if (!X) return fail(GPTQ_ERR_INVALID_ARG, "X is NULL");
  if (ld_x < d_in) return fail(GPTQ_ERR_INVALID_ARG, "ld_x (%lld) < d_in (%lld)", (long long)ld_x,
                               (long long)d_in);
  int rc = check_ws(ws, ws_bytes, gq::hessian_ws_bytes(d_in, n_tok), "hessian_accumulate");
  if (rc) return rc;
  hipError_t e;
  {
    gq::TimerScope ts(gq::kTimerHessian, (hipStream_t)stream);
    e = gq::hessian_launch(H, d_in, X, x_dtype, n_tok, ld_x, ws, ws_bytes, (hipStream_t)stream,
                           overwrite);
  }
  if (e != hipSuccess) return hip_fail("hessian_accumulate", e);
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
    case GPTQ_WS_OBQ:
      if (d_in > gq::obq_max_din()) return 0;
      return gq::obq_ws_bytes(d_in);
    case GPTQ_WS_LAYER:
      if (d_out <= 0 || d_out > kMaxDout || n_tok < 0) return 0;
      return layer_ws_bytes(d_out, d_in, n_tok);
    case GPTQ_WS_W4A16:   // d_out = N, d_in = K, n_tok = M
      if (d_out <= 0 || d_out > kMaxDout || n_tok <= 0 || n_tok > kMaxDout) return 0;
      return gq::w4a16_ws_bytes(n_tok, d_out, d_in);
    default:
      return 0;
  }
}

int gptq_hessian_accumulate(float* H, int64_t d_in, const void* X, int x_dtype, int64_t n_tok,
                            int64_t ld_x, void* ws, size_t ws_bytes, gptq_stream stream) {
  return hessian_call(H, d_in, X, x_dtype, n_tok, ld_x, ws, ws_bytes, stream, false);
}

int gptq_hessian(float* H, int64_t d_in, const void* X, int x_dtype, int64_t n_tok, int64_t ld_x,
                 void* ws, size_t ws_bytes, gptq_stream stream) {
  return hessian_call(H, d_in, X, x_dtype, n_tok, ld_x, ws, ws_bytes, stream, true);
}

int gptq_hessian_accumulate_noalloc(float* H, int64_t d_in, const void* X, int x_dtype,
                                    int64_t n_tok, int64_t ld_x, gptq_stream stream) {
  if (!H) return fail(GPTQ_ERR_INVALID_ARG, "H is NULL");
  if (d_in <= 0 || d_in > kMaxDin)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in must be in [1, %lld] (got %lld)", (long long)kMaxDin,
                (long long)d_in);
  if (n_tok < 0) return fail(GPTQ_ERR_INVALID_ARG, "n_tok must be >= 0");
  if (!valid_dtype(x_dtype)) return fail(GPTQ_ERR_INVALID_ARG, "unknown x_dtype %d", x_dtype);
  if (gq::hessian_min_ws_bytes(d_in) > gq::kScratchBytes)
    return fail(GPTQ_ERR_UNSUPPORTED,
                "hessian_accumulate_noalloc: d_in %lld needs %zu bytes of scratch, the static "
                "scratch holds %zu (d_in <= 4096); use gptq_hessian_accumulate with a workspace",
                (long long)d_in, gq::hessian_min_ws_bytes(d_in), gq::kScratchBytes);
  if (n_tok == 0) return GPTQ_OK;
  if (!X) return fail(GPTQ_ERR_INVALID_ARG, "X is NULL");
  if (ld_x < d_in) return fail(GPTQ_ERR_INVALID_ARG, "ld_x (%lld) < d_in (%lld)", (long long)ld_x,
                               (long long)d_in);
  hipError_t e = gq::hessian_launch_static(H, d_in, X, x_dtype, n_tok, ld_x, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("hessian_accumulate_noalloc", e);
  return GPTQ_OK;
}

int gptq_prepare_hinv(float* H, int64_t d_in, const gptq_params* p, float* U, int32_t* perm,
                      uint8_t* dead_mask, void* ws, size_t ws_bytes, int64_t* info,
                      gptq_stream stream) {
  if (info) *info = -1;
  hipStream_t s = (hipStream_t)stream;
  int32_t* status_dev = nullptr;
  int rc = prepare_enqueue(H, d_in, p, U, perm, dead_mask, ws, ws_bytes, &status_dev, s);
  if (rc) return rc;
  int32_t st[2] = {0, 0};   // failing pivot (or INT_MAX), stall flag
  hipError_t e = hipMemcpyAsync(st, status_dev, sizeof st, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail("prepare_hinv (status read-back)", e);
  return status_result(st, d_in, info);
}

int gptq_prepare_hinv_async(float* H, int64_t d_in, const gptq_params* p, float* U,
                            int32_t* perm, uint8_t* dead_mask, void* ws, size_t ws_bytes,
                            int32_t* status, gptq_stream stream) {
  if (!status) return fail(GPTQ_ERR_INVALID_ARG, "status must not be NULL");
  hipStream_t s = (hipStream_t)stream;
  int32_t* status_dev = nullptr;
  int rc = prepare_enqueue(H, d_in, p, U, perm, dead_mask, ws, ws_bytes, &status_dev, s);
  if (rc) return rc;
  hipError_t e = hipMemcpyAsync(status, status_dev, 2 * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail("prepare_hinv_async (status copy)", e);
  return GPTQ_OK;
}

int gptq_prepare_status(const int32_t* status, int64_t d_in, int64_t* info) {
  if (info) *info = -1;
  if (!status) return fail(GPTQ_ERR_INVALID_ARG, "status must not be NULL");
  if (d_in <= 0 || d_in > kMaxDin)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in must be in [1, %lld]", (long long)kMaxDin);
  return status_result(status, d_in, info);
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
  if (p->act_order && !perm)
    return fail(GPTQ_ERR_INVALID_ARG,
                "act_order needs the perm from gptq_prepare_hinv (U is in that order)");
  rc = check_ws(ws, ws_bytes, gq::quantize_ws_bytes(d_out, d_in), "quantize_layer");
  if (rc) return rc;
  hipError_t e = gq::quantize_launch(W, w_dtype, d_out, d_in, ld_w, U, perm, dead_mask, *p,
                                     qweight, scales, zeros, W_hat, g_idx, row_loss, ws,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("quantize_layer", e);
  return GPTQ_OK;
}

int gptq_quantize_layers(int n_layers, const gptq_layer* layers, int64_t d_in, const float* U,
                         const int32_t* perm, const uint8_t* dead_mask, const gptq_params* p,
                         int32_t* g_idx, void* ws, size_t ws_bytes, gptq_stream stream) {
  if (n_layers < 1 || n_layers > 1024)
    return fail(GPTQ_ERR_INVALID_ARG, "n_layers must be in [1, 1024] (got %d)", n_layers);
  if (!layers || !U) return fail(GPTQ_ERR_INVALID_ARG, "layers and U must not be NULL");
  if (d_in <= 0 || d_in > kMaxDin)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in must be in [1, %lld]", (long long)kMaxDin);
  int64_t total = 0;
  std::vector<gq::LayerIO> io((size_t)n_layers);
  for (int i = 0; i < n_layers; ++i) {
    const gptq_layer& L = layers[i];
    if (!L.W || !L.qweight || !L.scales || !L.zeros)
      return fail(GPTQ_ERR_INVALID_ARG, "layer %d: W, qweight, scales and zeros must not be NULL", i);
    if (!valid_dtype(L.w_dtype)) return fail(GPTQ_ERR_INVALID_ARG, "layer %d: unknown w_dtype", i);
    if (L.d_out <= 0 || L.d_out > kMaxDout)
      return fail(GPTQ_ERR_INVALID_ARG, "layer %d: d_out must be in [1, %lld]", i, (long long)kMaxDout);
    if (L.ld_w < d_in) return fail(GPTQ_ERR_INVALID_ARG, "layer %d: ld_w < d_in", i);
    total += L.d_out;
    io[(size_t)i] = gq::LayerIO{L.W, L.w_dtype, L.d_out, L.ld_w, L.qweight, L.scales, L.zeros,
                                L.W_hat, L.row_loss};
  }
  if (total > kMaxDout)
    return fail(GPTQ_ERR_INVALID_ARG, "the layers' rows add up to more than %lld", (long long)kMaxDout);
  int rc = check_params(p, d_in);
  if (rc) return rc;
  if (p->act_order && !perm)
    return fail(GPTQ_ERR_INVALID_ARG,
                "act_order needs the perm from gptq_prepare_hinv (U is in that order)");
  rc = check_ws(ws, ws_bytes, gq::quantize_ws_bytes(total, d_in), "quantize_layers");
  if (rc) return rc;
  hipError_t e = gq::quantize_layers_launch(io.data(), n_layers, d_in, U, perm, dead_mask, *p, g_idx,
                                            ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("quantize_layers", e);
  return GPTQ_OK;
}

int gptq_quantize_independent(int n_jobs, gptq_layer_job* jobs, const gptq_params* p,
                              gptq_stream stream) {
  if (n_jobs < 1 || n_jobs > 1024)
    return fail(GPTQ_ERR_INVALID_ARG, "n_jobs must be in [1, 1024] (got %d)", n_jobs);
  if (!jobs) return fail(GPTQ_ERR_INVALID_ARG, "jobs is NULL");
  for (int i = 0; i < n_jobs; ++i) {
    const gptq_layer_job& J = jobs[i];
    if (!J.W || !J.H || !J.U || !J.qweight || !J.scales || !J.zeros)
      return fail(GPTQ_ERR_INVALID_ARG, "job %d: W, H, U, qweight, scales and zeros must not be NULL", i);
    if (!valid_dtype(J.w_dtype) || !valid_dtype(J.x_dtype))
      return fail(GPTQ_ERR_INVALID_ARG, "job %d: unknown x_dtype or w_dtype", i);
    if (J.d_in <= 0 || J.d_in > kMaxDin)
      return fail(GPTQ_ERR_INVALID_ARG, "job %d: d_in must be in [1, %lld]", i, (long long)kMaxDin);
    if (J.d_out <= 0 || J.d_out > kMaxDout)
      return fail(GPTQ_ERR_INVALID_ARG, "job %d: d_out must be in [1, %lld]", i, (long long)kMaxDout);
    if (J.ld_w < J.d_in) return fail(GPTQ_ERR_INVALID_ARG, "job %d: ld_w < d_in", i);
    if (J.n_tok < 0) return fail(GPTQ_ERR_INVALID_ARG, "job %d: n_tok must be >= 0", i);
    if (J.n_tok > 0 && !J.X) return fail(GPTQ_ERR_INVALID_ARG, "job %d: X is NULL", i);
    if (J.n_tok > 0 && J.ld_x < J.d_in) return fail(GPTQ_ERR_INVALID_ARG, "job %d: ld_x < d_in", i);
    int rc = check_params(p, J.d_in);
    if (rc) return rc;
    if (p->act_order && !J.perm)
      return fail(GPTQ_ERR_INVALID_ARG, "job %d: act_order needs a perm output", i);
    rc = check_ws(J.ws, J.ws_bytes, layer_ws_bytes(J.d_out, J.d_in, J.n_tok), "quantize_independent");
    if (rc) return fail(rc, "job %d: %s", i, g_err.c_str());
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("quantize_independent", e);
  JobStreams* js = job_streams(dev);
  if (js->err != hipSuccess) return hip_fail("quantize_independent (streams)", js->err);
  hipStream_t s = (hipStream_t)stream;
  const int ns = n_jobs < kJobStreams ? n_jobs : kJobStreams;
  std::vector<int32_t*> status_dev((size_t)n_jobs, nullptr);
  {
    std::lock_guard<std::mutex> lock(js->mu);
    if ((e = hipEventRecord(js->fork, s)) != hipSuccess) return hip_fail("quantize_independent", e);
    for (int k = 0; k < ns; ++k)
      if ((e = hipStreamWaitEvent(js->s[k], js->fork, 0)) != hipSuccess)
        return hip_fail("quantize_independent", e);
    for (int i = 0; i < n_jobs; ++i) {
      const gptq_layer_job& J = jobs[i];
      hipStream_t sj = js->s[i % ns];
      char* ws = static_cast<char*>(J.ws);
      if (J.n_tok > 0) {
        e = gq::hessian_launch(J.H, J.d_in, J.X, J.x_dtype, J.n_tok, J.ld_x, ws,
                               gq::hessian_ws_bytes(J.d_in, J.n_tok), sj);
        if (e != hipSuccess) return hip_fail("quantize_independent (Hessian)", e);
      }
      e = gq::prepare_launch(J.H, J.d_in, p->percdamp, p->act_order, J.U, J.perm, J.dead_mask, ws,
                             &status_dev[(size_t)i], sj);
      if (e != hipSuccess) return hip_fail("quantize_independent (prepare)", e);
      e = gq::quantize_launch(J.W, J.w_dtype, J.d_out, J.d_in, J.ld_w, J.U,
                              p->act_order ? J.perm : nullptr, J.dead_mask, *p, J.qweight, J.scales,
                              J.zeros, J.W_hat, J.g_idx, J.row_loss, ws + layer_prep_bytes(J.d_in), sj);
      if (e != hipSuccess) return hip_fail("quantize_independent (quantize)", e);
    }
    for (int k = 0; k < ns; ++k) {
      if ((e = hipEventRecord(js->join[k], js->s[k])) != hipSuccess ||
          (e = hipStreamWaitEvent(s, js->join[k], 0)) != hipSuccess)
        return hip_fail("quantize_independent", e);
    }
  }
  std::vector<int32_t> st((size_t)n_jobs * 2, 0);
  for (int i = 0; i < n_jobs && e == hipSuccess; ++i)
    e = hipMemcpyAsync(&st[(size_t)i * 2], status_dev[(size_t)i], 2 * sizeof(int32_t),
                       hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail("quantize_independent (status read-back)", e);
  int first = GPTQ_OK, first_job = -1;
  for (int i = 0; i < n_jobs; ++i) {
    int64_t piv = -1;
    const int rc = gq::prepare_status(st[(size_t)i * 2], st[(size_t)i * 2 + 1], jobs[i].d_in, &piv);
    jobs[i].status = rc;
    jobs[i].info = rc == GPTQ_ERR_NOT_SPD ? piv : -1;
    if (rc != GPTQ_OK && first == GPTQ_OK) { first = rc; first_job = i; }
  }
  if (first == GPTQ_ERR_NOT_SPD)
    return fail(first, "job %d: damped Hessian is not positive definite (pivot %lld); raise percdamp",
                first_job, (long long)jobs[first_job].info);
  if (first != GPTQ_OK)
    return fail(first, "job %d: a factorization wave ran out of its bounded wait; outputs undefined",
                first_job);
  return GPTQ_OK;
}

int gptq_obq_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ld_w,
                   const float* H, const gptq_params* p, uint32_t* qweight, float* scales,
                   uint8_t* zeros, float* W_hat, int32_t* order, float* row_loss, void* ws,
                   size_t ws_bytes, gptq_stream stream) {
  if (!W || !H || !qweight || !scales || !zeros)
    return fail(GPTQ_ERR_INVALID_ARG, "W, H, qweight, scales and zeros must not be NULL");
  if (!valid_dtype(w_dtype)) return fail(GPTQ_ERR_INVALID_ARG, "unknown w_dtype %d", w_dtype);
  if (d_in <= 0 || d_out <= 0 || d_out > kMaxDout)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in and d_out must be positive");
  if (ld_w < d_in) return fail(GPTQ_ERR_INVALID_ARG, "ld_w < d_in");
  if (!p) return fail(GPTQ_ERR_INVALID_ARG, "params is NULL");
  if (p->bits != 2 && p->bits != 3 && p->bits != 4 && p->bits != 8)
    return fail(GPTQ_ERR_INVALID_ARG, "bits must be 2, 3, 4 or 8 (got %d)", p->bits);
  if (!(p->percdamp >= 0.f) || !std::isfinite(p->percdamp))
    return fail(GPTQ_ERR_INVALID_ARG, "percdamp must be finite and >= 0");
  if (p->sym != 0 && p->sym != 1) return fail(GPTQ_ERR_INVALID_ARG, "sym must be 0 or 1");
  if (p->group_size != -1 && p->group_size < d_in)
    return fail(GPTQ_ERR_UNSUPPORTED, "OBQ runs with one grid per row (group_size -1)");
  if (p->act_order) return fail(GPTQ_ERR_UNSUPPORTED, "OBQ chooses its own order (act_order 0)");
  if (d_in > gq::obq_max_din())
    return fail(GPTQ_ERR_UNSUPPORTED, "OBQ is the tiny-layer comparator: d_in <= %d (got %lld)",
                gq::obq_max_din(), (long long)d_in);
  int rc = check_ws(ws, ws_bytes, gq::obq_ws_bytes(d_in), "obq_layer");
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  int32_t* status_dev = nullptr;
  hipError_t e = gq::obq_launch(W, w_dtype, d_out, d_in, ld_w, H, *p, qweight, scales, zeros,
                                W_hat, order, row_loss, ws, &status_dev, s);
  if (e != hipSuccess) return hip_fail("obq_layer", e);
  int32_t st = 0;
  e = hipMemcpyAsync(&st, status_dev, sizeof st, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail("obq_layer (status read-back)", e);
  if (st != INT_MAX)
    return fail(GPTQ_ERR_NOT_SPD, "damped Hessian is not positive definite (pivot %d); raise percdamp",
                (int)st);
  return GPTQ_OK;
}

int gptq_w4a16_gemm(const void* A, int a_dtype, int64_t M, int64_t K, int64_t lda,
                    const uint32_t* qweight, int bits, const uint16_t* scales_f16,
                    const uint16_t* zeros_f16, const int32_t* g_idx, int group_size,
                    int64_t n_groups, int64_t N, float* C, int64_t ldc, void* ws,
                    size_t ws_bytes, gptq_stream stream) {
  if (!A || !qweight || !scales_f16 || !zeros_f16 || !C)
    return fail(GPTQ_ERR_INVALID_ARG, "A, qweight, scales, zeros and C must not be NULL");
  if (a_dtype != GPTQ_F16 && a_dtype != GPTQ_BF16)
    return fail(GPTQ_ERR_INVALID_ARG, "a_dtype must be GPTQ_F16 or GPTQ_BF16");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_ERR_INVALID_ARG, "bits must be 2, 3, 4 or 8 (got %d)", bits);
  if (M <= 0 || K <= 0 || N <= 0 || K > kMaxDin || N > kMaxDout || M > kMaxDout)
    return fail(GPTQ_ERR_INVALID_ARG, "M, K and N must be positive (K <= %lld)", (long long)kMaxDin);
  if (lda < K || ldc < N) return fail(GPTQ_ERR_INVALID_ARG, "lda < K or ldc < N");
  if (N * ceil_div64(K * bits, 32) * 4 >= ((int64_t)1 << 32) || ((M - 1) * lda + K) * 2 >= ((int64_t)1 << 32))
    return fail(GPTQ_ERR_UNSUPPORTED, "the weight words and A must each stay under 4 GiB");
  const int64_t g = (group_size <= 0 || group_size >= K) ? K : group_size;
  if (!g_idx && g % 32 != 0 && g != K)
    return fail(GPTQ_ERR_UNSUPPORTED, "group_size must be a multiple of 32 (or -1)");
  if (n_groups < ceil_div64(K, g) || n_groups > K)
    return fail(GPTQ_ERR_INVALID_ARG, "n_groups must cover the groups of K columns");
  if (ws) {
    const int rc = check_ws(ws, ws_bytes, gq::w4a16_ws_bytes(M, N, K), "w4a16_gemm");
    if (rc != GPTQ_OK) return rc;
  }
  hipError_t e = gq::w4a16_launch(A, a_dtype, M, K, lda, qweight, bits, scales_f16, zeros_f16,
                                  g_idx, g, n_groups, N, C, ldc, ws, ws_bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("w4a16_gemm", e);
  return GPTQ_OK;
}

int gptq_timing(int enable) { return gq::timing_enable(enable); }

int gptq_timing_read(float* ms, int n) {
  if (!ms || n <= 0) return fail(GPTQ_ERR_INVALID_ARG, "ms must hold n > 0 floats");
  hipError_t e = gq::timing_read(ms, n);
  if (e != hipSuccess) return hip_fail("timing_read", e);
  return GPTQ_OK;
}

int gptq_export(int bits, int64_t d_out, int64_t d_in, int64_t n_groups, const uint32_t* qweight,
                const float* scales, const uint8_t* zeros, uint32_t* qweight_dense,
                uint16_t* scales_f16, uint16_t* zeros_f16, gptq_stream stream) {
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_ERR_INVALID_ARG, "bits must be 2, 3, 4 or 8 (got %d)", bits);
  if (d_in <= 0 || d_in > kMaxDin)
    return fail(GPTQ_ERR_INVALID_ARG, "d_in must be in [1, %lld]", (long long)kMaxDin);
  if (d_out <= 0 || d_out > kMaxDout)
    return fail(GPTQ_ERR_INVALID_ARG, "d_out must be in [1, %lld]", (long long)kMaxDout);
  if (n_groups <= 0 || n_groups > d_in)
    return fail(GPTQ_ERR_INVALID_ARG, "n_groups must be in [1, d_in]");
  if (qweight_dense && !qweight)
    return fail(GPTQ_ERR_INVALID_ARG, "qweight_dense needs qweight");
  if (scales_f16 && !scales) return fail(GPTQ_ERR_INVALID_ARG, "scales_f16 needs scales");
  if (zeros_f16 && !zeros) return fail(GPTQ_ERR_INVALID_ARG, "zeros_f16 needs zeros");
  hipError_t e = gq::export_launch(bits, d_out, d_in, n_groups, qweight, scales, zeros,
                                   qweight_dense, scales_f16, zeros_f16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("export", e);
  return GPTQ_OK;
}

}  // extern "C"
