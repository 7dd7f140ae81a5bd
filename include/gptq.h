/*
 * gptq.h -- C ABI of the MI355X GPTQ layer-quantization library
 *           (libgptq_mi355x.so, HIP for gfx950).
 *
 * The library quantizes one linear layer W [d_out x d_in] with the GPTQ
 * method, in three calls that follow the method's own stages:
 *
 *   1. gptq_hessian_accumulate  H += 2·Xᵀ·X over calibration tokens
 *   2. gptq_prepare_hinv        dead-channel fix, damping, act-order,
 *                               upper Cholesky factor U of H_d⁻¹
 *   3. gptq_quantize_layer      blocked column sweep with OBS compensation
 *                               and lazy block updates; packed codes,
 *                               per-group scales/zeros, dequantized Ŵ
 *
 * Sources (pages cited by title and section):
 *  - "GPTQ: Mathematical Foundations, Optimal Brain Surgeon Inversion, and
 *    Second-Order Error Minimization in LLM Quantization" (below:
 *    "Foundations"): The Layer-Wise Reconstruction Problem; Second-Order
 *    Taylor Expansion and the Hessian; The GPTQ Algorithmic Innovations
 *    (Arbitrary Order Quantization, Lazy Batch Updates, Cholesky
 *    Decomposition and Pre-computation); Hessian Damping and Numerical
 *    Regularization; Activation Ordering; Quantization Formats and Group
 *    Size; GPTQ Algorithm Execution Walkthrough; Inference Execution.
 *  - "INT4 and GPTQ Quantization": Uniform INT4 Quantization; Group
 *    Quantization; GPTQ Algorithm in PyTorch-Style Pseudocode.
 *  - "GPTQ" (technology card): Hyperparameters (bits 3/4, group size 128,
 *    act-order, damping 0.01).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host".  Matrices are
 *    row-major.  The caller owns every buffer; the library allocates no
 *    device memory and keeps no state between calls except a thread-local
 *    error message.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *    and runs asynchronously, except where a call says it synchronizes.
 *  - Arguments are validated before any HIP call.  On a non-zero return
 *    nothing has been enqueued (except GPTQ_ERR_NOT_SPD and GPTQ_ERR_HIP,
 *    see the calls), and gptq_last_error() describes the problem.
 *  - Calls are re-entrant; concurrent calls must use distinct workspaces.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = -1,  /* null/ill-sized argument, bad parameter value   */
  GPTQ_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. g/B mismatch)  */
  GPTQ_ERR_NOT_SPD = -3,      /* damped Hessian not positive definite           */
  GPTQ_ERR_WORKSPACE = -4,    /* workspace null or smaller than required        */
  GPTQ_ERR_HIP = -5           /* a HIP runtime call failed                      */
} gptq_status;

typedef enum { GPTQ_F32 = 0, GPTQ_BF16 = 1, GPTQ_F16 = 2 } gptq_dtype;

/* Quantizer settings ("GPTQ" card, Hyperparameters; "Foundations",
 * walkthrough signature).
 *  bits        code width: 2, 3, 4 or 8.
 *  group_size  g > 0 consecutive input columns (in quantization order)
 *              share one (scale, zero) per row; -1 = one group per row.
 *  block_size  lazy-update block B.  This library runs B = 128; groups must
 *              start on block starts or lie inside blocks (g % 128 == 0,
 *              128 % g == 0, or one group per row), else GPTQ_ERR_UNSUPPORTED.
 *  percdamp    α in λ = α·mean(diag H) ("Foundations", Hessian Damping); >= 0.
 *  act_order   1: quantize columns in descending order of diag H
 *              ("Foundations", Activation Ordering).
 *  sym         1: symmetric grid s = max|w|/(2ᵇ⁻¹−1), codes stored unsigned
 *              with zero 2ᵇ⁻¹ ("INT4 and GPTQ Quantization", Uniform INT4
 *              Quantization); 0: asymmetric min/max grid.                  */
typedef struct {
  int32_t bits;
  int32_t group_size;
  int32_t block_size;
  float percdamp;
  int32_t act_order;
  int32_t sym;
} gptq_params;

typedef void* gptq_stream;

enum { GPTQ_WS_HESSIAN = 0, GPTQ_WS_PREPARE = 1, GPTQ_WS_QUANTIZE = 2 };

/* Workspace size in bytes that call `which` (GPTQ_WS_*) needs for the given
 * shape.  n_tok is used by the Hessian call only; p may be NULL for it.
 * Returns 0 for invalid arguments.  Workspaces need 256-byte alignment
 * (every hipMalloc'd pointer has it). */
size_t gptq_workspace_bytes(int which, int64_t d_out, int64_t d_in, int64_t n_tok,
                            const gptq_params* p);

/* H += 2·Xᵀ·X  ("Foundations", Second-Order Taylor Expansion and the
 * Hessian: H = 2XXᵀ with X stored there as d_in x N; here X is token-major).
 *  H      [d_in x d_in] fp32, in/out.  The caller zero-fills it before the
 *         first batch; further calls add more tokens.  Both triangles are
 *         written and the result is exactly symmetric.
 *  X      [n_tok x d_in] token-major, row stride ld_x >= d_in elements, of
 *         type x_dtype (GPTQ_BF16, GPTQ_F16: MFMA products exact in fp32;
 *         GPTQ_F32: fp32 MFMA).  Accumulation is fp32.
 *  n_tok  >= 0 (0 is a no-op).
 *  ws     workspace of gptq_workspace_bytes(GPTQ_WS_HESSIAN, 0, d_in, n_tok, NULL).
 * Asynchronous.  Deterministic: the same inputs give bit-identical H. */
int gptq_hessian_accumulate(float* H, int64_t d_in, const void* X, int x_dtype,
                            int64_t n_tok, int64_t ld_x, void* ws, size_t ws_bytes,
                            gptq_stream stream);

/* Prepare the inverse-Hessian factor ("Foundations": walkthrough steps 1-2,
 * Hessian Damping, Activation Ordering, Cholesky Decomposition):
 *   dead_i = (H_ii == 0) -> H_ii := 1;  λ = percdamp·mean(diag H);
 *   (act_order) π = stable descending argsort of diag H (ties: lower index);
 *   H_d = (H + λI)[π][:, π];  U upper, positive diagonal, H_d⁻¹ = UᵀU.
 *  H          in: accumulated H [d_in x d_in] fp32.  out: H_d (dead-fixed,
 *             damped, permuted).
 *  U          out [d_in x d_in] fp32, upper triangular (zeros below).
 *  perm       out [d_in] int32, quantization order (identity without
 *             act-order); may be NULL when act_order == 0.
 *  dead_mask  out [d_in] uint8, 1 for dead channels (original order); may be
 *             NULL.
 *  info       host, out: -1 on success, else the failing pivot (in the
 *             permuted order) when GPTQ_ERR_NOT_SPD; may be NULL.
 *  ws         workspace of gptq_workspace_bytes(GPTQ_WS_PREPARE, 0, d_in, 0, p).
 * SYNCHRONIZES `stream` before returning (it reads back the factorization
 * status).  On GPTQ_ERR_NOT_SPD, U is undefined; a larger percdamp is the
 * usual remedy ("GPTQ" card, Implementation pitfalls). */
int gptq_prepare_hinv(float* H, int64_t d_in, const gptq_params* p, float* U,
                      int32_t* perm, uint8_t* dead_mask, void* ws, size_t ws_bytes,
                      int64_t* info, gptq_stream stream);

/* Quantize the layer ("Foundations": The GPTQ Algorithmic Innovations 1-3,
 * walkthrough step 3, Quantization Formats and Group Size; "INT4 and GPTQ
 * Quantization": Group Quantization).  Columns are taken in the order perm;
 * for each column c: group (s, z) from the current values when c starts a
 * group; q = clamp(rint(w/s + z), 0, 2ᵇ−1); ŵ = s(q − z);
 * err = (w − ŵ)/U_cc; later columns of the block get w_k −= err·U_ck at once,
 * columns beyond the block get the whole block's update in one product.
 *  W          [d_out x d_in] of w_dtype (fp32/bf16/fp16), row stride ld_w.
 *  U          factor from gptq_prepare_hinv (quantization order).
 *  perm       [d_in] from gptq_prepare_hinv, or NULL for natural order.
 *  dead_mask  [d_in] or NULL; dead columns are quantized as zeros.
 *  qweight    out [d_out x ceil(d_in/8)] uint32 for bits <= 4 (column 8k+i in
 *             bits 4i..4i+3 of word k, ORIGINAL column order), or
 *             [d_out x ceil(d_in/4)] for bits == 8 (byte i of word k).
 *  scales     out [d_out x n_groups] fp32, groups in quantization order
 *             (n_groups = ceil(d_in/g), 1 for per-row).
 *  zeros      out [d_out x n_groups] uint8.
 *  W_hat      out [d_out x d_in] fp32 dequantized weights, original column
 *             order; may be NULL.
 *  g_idx      out [d_in] int32 group of each original column; may be NULL.
 *  row_loss   out [d_out] fp32, ½·Σ_c err_c² per row; may be NULL.
 *  ws         workspace of gptq_workspace_bytes(GPTQ_WS_QUANTIZE, d_out, d_in, 0, p).
 * Asynchronous. */
int gptq_quantize_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ld_w,
                        const float* U, const int32_t* perm, const uint8_t* dead_mask,
                        const gptq_params* p, uint32_t* qweight, float* scales,
                        uint8_t* zeros, float* W_hat, int32_t* g_idx, float* row_loss,
                        void* ws, size_t ws_bytes, gptq_stream stream);

/* Message for the last non-zero status on the calling thread (never NULL). */
const char* gptq_last_error(void);

/* Library version string. */
const char* gptq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GPTQ_MI355X_H */
