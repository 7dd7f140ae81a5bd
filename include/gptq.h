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
  GPTQ_ERR_HIP = -5,          /* a HIP runtime call failed                      */
  GPTQ_ERR_INTERNAL = -6      /* a kernel's bounded internal wait ran out: the
                                 outputs are undefined (a library fault)        */
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

enum { GPTQ_WS_HESSIAN = 0, GPTQ_WS_PREPARE = 1, GPTQ_WS_QUANTIZE = 2, GPTQ_WS_OBQ = 3,
       GPTQ_WS_W4A16 = 4, GPTQ_WS_LAYER = 5 };

/* Workspace size in bytes that call `which` (GPTQ_WS_*) needs for the given
 * shape.  n_tok is used by the Hessian call and GPTQ_WS_LAYER only; p may be
 * NULL for the Hessian.  GPTQ_WS_LAYER is one job of
 * gptq_quantize_independent (its Hessian, preparation and quantization).
 * For GPTQ_WS_W4A16 the shape is d_out = N, d_in = K, n_tok = M (p unused).
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

/* gptq_hessian_accumulate for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arithmetic, with the library's own static device
 * scratch of 65 MiB per GPU (held from the first call on that GPU until the
 * process ends) in place of a workspace.  That holds one partial Hessian of
 * d_in <= 4096; larger d_in returns GPTQ_ERR_UNSUPPORTED.  With less room
 * for split partials than the workspace version, the token range may be cut
 * into fewer splits, so H can differ from gptq_hessian_accumulate's in its
 * rounding (both stay within the same error bound).  Every call on one GPU
 * shares the scratch: calls that overlap on one GPU (other streams, other
 * threads) race and must not be issued.  Allocates nothing; asynchronous. */
int gptq_hessian_accumulate_noalloc(float* H, int64_t d_in, const void* X, int x_dtype,
                                    int64_t n_tok, int64_t ld_x, gptq_stream stream);

/* H = 2·Xᵀ·X: gptq_hessian_accumulate for a Hessian started from zero, in one
 * call ("Foundations", Second-Order Taylor Expansion and the Hessian).  H is
 * only written (the accumulating call reads it too); the arithmetic of every
 * element is that of gptq_hessian_accumulate on a zeroed H, bit for bit.
 * n_tok == 0 sets H to zeros (X may then be NULL).  Arguments, workspace and
 * errors as for gptq_hessian_accumulate.  Asynchronous. */
int gptq_hessian(float* H, int64_t d_in, const void* X, int x_dtype, int64_t n_tok, int64_t ld_x,
                 void* ws, size_t ws_bytes, gptq_stream stream);

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
 * usual remedy ("GPTQ" card, Implementation pitfalls).  GPTQ_ERR_INTERNAL
 * means a wave of the factorization gave up waiting for another wave (every
 * such wait is bounded, so the call never hangs); U and H are then
 * undefined. */
int gptq_prepare_hinv(float* H, int64_t d_in, const gptq_params* p, float* U,
                      int32_t* perm, uint8_t* dead_mask, void* ws, size_t ws_bytes,
                      int64_t* info, gptq_stream stream);

/* gptq_prepare_hinv without its wait ("Foundations", Cholesky Decomposition
 * and Pre-computation; the computation is the same, bit for bit): the call
 * returns once the work is enqueued, so a pipeline can queue the
 * quantization (and the next layer's work) right behind it and look at the
 * outcome later, instead of leaving the GPU idle while the host reads it.
 *  status   host, out: 2 int32 status words, written asynchronously on
 *           `stream` after the factorization.  Use pinned memory
 *           (hipHostMalloc) so the copy does not block the host; read the
 *           words only once the stream, or an event recorded on it after
 *           this call, has completed, and decode them with
 *           gptq_prepare_status.  They must stay valid until then.
 *  Other arguments as for gptq_prepare_hinv (no info).
 * Returns argument errors and GPTQ_ERR_HIP only; the factorization's own
 * outcome (GPTQ_ERR_NOT_SPD, GPTQ_ERR_INTERNAL) is in `status`, and until it
 * has been checked U must be treated as possibly undefined.  The workspace
 * may be reused as soon as the words have been copied (stream order). */
int gptq_prepare_hinv_async(float* H, int64_t d_in, const gptq_params* p, float* U,
                            int32_t* perm, uint8_t* dead_mask, void* ws, size_t ws_bytes,
                            int32_t* status, gptq_stream stream);

/* What gptq_prepare_hinv would have returned, from the status words that
 * gptq_prepare_hinv_async copied out (host only, no HIP call).
 *  status  host, in: the 2 words.   info  host, out (may be NULL): as for
 *  gptq_prepare_hinv. */
int gptq_prepare_status(const int32_t* status, int64_t d_in, int64_t* info);

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

/* One layer of gptq_quantize_layers: its weights and its outputs, with the
 * meaning, layout and NULL rules of the gptq_quantize_layer arguments of the
 * same names. */
typedef struct {
  const void* W;       /* [d_out x d_in] of w_dtype, row stride ld_w          */
  int32_t w_dtype;     /* GPTQ_F32 / GPTQ_BF16 / GPTQ_F16                     */
  int32_t reserved;    /* 0                                                   */
  int64_t d_out;
  int64_t ld_w;
  uint32_t* qweight;   /* out, packed codes                                   */
  float* scales;       /* out [d_out x n_groups]                              */
  uint8_t* zeros;      /* out [d_out x n_groups]                              */
  float* W_hat;        /* out [d_out x d_in] or NULL                          */
  float* row_loss;     /* out [d_out] or NULL                                 */
} gptq_layer;

/* Several layers quantized against one prepared factor ("Foundations",
 * Second-Order Taylor Expansion and the Hessian: H depends only on the
 * layer's inputs, so layers fed the same X -- e.g. the query, key and value
 * projections -- share H, U and the column order; The Layer-Wise
 * Reconstruction Problem: rows are independent problems).  The layers' rows
 * are stacked and swept together, which fills the GPU better than one small
 * layer at a time; every output equals, bit for bit, what gptq_quantize_layer
 * gives for that layer alone.
 *  layers     host array of n_layers (1..1024) descriptors; all share d_in.
 *  U, perm, dead_mask, p   as for gptq_quantize_layer.
 *  g_idx      out [d_in] (the same for every layer); may be NULL.
 *  ws         workspace of gptq_workspace_bytes(GPTQ_WS_QUANTIZE, Σ d_out, d_in, 0, p).
 * Asynchronous; argument errors only. */
int gptq_quantize_layers(int n_layers, const gptq_layer* layers, int64_t d_in, const float* U,
                         const int32_t* perm, const uint8_t* dead_mask, const gptq_params* p,
                         int32_t* g_idx, void* ws, size_t ws_bytes, gptq_stream stream);

/* One layer of gptq_quantize_independent: its own calibration inputs, weights,
 * outputs and workspace.  Meaning, layout and NULL rules of the fields are
 * those of the gptq_hessian_accumulate, gptq_prepare_hinv and
 * gptq_quantize_layer arguments of the same names. */
typedef struct {
  const void* X;       /* [n_tok x d_in] of x_dtype, row stride ld_x               */
  int32_t x_dtype;     /* GPTQ_F32 / GPTQ_BF16 / GPTQ_F16                          */
  int32_t w_dtype;     /* GPTQ_F32 / GPTQ_BF16 / GPTQ_F16                          */
  int64_t n_tok;       /* >= 0 (0: H is used as it comes)                          */
  int64_t ld_x;
  const void* W;       /* [d_out x d_in] of w_dtype, row stride ld_w               */
  int64_t d_out;
  int64_t d_in;
  int64_t ld_w;
  float* H;            /* in/out [d_in x d_in]: 2·XᵀX is added, then H_d replaces it */
  float* U;            /* out [d_in x d_in]                                        */
  int32_t* perm;       /* out [d_in]; required with act_order, else may be NULL    */
  uint8_t* dead_mask;  /* out [d_in] or NULL                                       */
  uint32_t* qweight;   /* out, packed codes                                        */
  float* scales;       /* out [d_out x n_groups]                                   */
  uint8_t* zeros;      /* out [d_out x n_groups]                                   */
  float* W_hat;        /* out [d_out x d_in] or NULL                               */
  int32_t* g_idx;      /* out [d_in] or NULL                                       */
  float* row_loss;     /* out [d_out] or NULL                                      */
  void* ws;            /* gptq_workspace_bytes(GPTQ_WS_LAYER, d_out, d_in, n_tok, p) */
  size_t ws_bytes;
  int32_t status;      /* out: this layer's factorization status (gptq_status)     */
  int32_t reserved;    /* 0                                                        */
  int64_t info;        /* out: failing pivot with GPTQ_ERR_NOT_SPD, else -1        */
} gptq_layer_job;

/* Independent layers -- each with its own inputs X, hence its own H and
 * factor -- quantized concurrently ("Foundations", The Layer-Wise
 * Reconstruction Problem: every layer is its own problem; "GPTQ" technology
 * card, Parallelism: layers can be processed independently).  For every job:
 * H += 2·XᵀX, the preparation of gptq_prepare_hinv, then gptq_quantize_layer
 * with that factor.  Jobs run on streams of the library's own (default
 * priority), forked from `stream` and joined back into it, so small layers
 * fill the GPU together; each job's outputs are, bit for bit, those of the
 * three calls made one after the other for that job alone.
 *  jobs   host array of n_jobs (1..1024) descriptors; shapes may differ; the
 *         workspaces must not overlap.
 *  p      quantizer parameters shared by all jobs.
 * Synchronizes `stream` once at the end (it reads every job's status).
 * Returns GPTQ_OK when every job succeeded; otherwise the status of the
 * first failed job (its `status` and `info` fields, like every job's, say
 * which); a failed job's outputs are undefined, the others' are valid.
 * Argument errors are found before anything is enqueued (no job runs then,
 * and no status field is written); after GPTQ_ERR_HIP, work enqueued before
 * the failure may still run.  Every job's pointers must be on the current
 * device. */
int gptq_quantize_independent(int n_jobs, gptq_layer_job* jobs, const gptq_params* p,
                              gptq_stream stream);

/* Optimal Brain Quantization, the greedy-order comparator for GPTQ's fixed
 * order on tiny layers ("Foundations": Optimal Brain Surgeon (OBS) and
 * Optimal Brain Quantization (OBQ), Lagrangian Derivation, Minimal Error
 * Penalty, Recursive Inverse Hessian Updating, The Computational Bottleneck
 * of OBQ; The GPTQ Algorithmic Innovations §1).  Every row runs its own
 * greedy sequence: quantize the free column with the smallest saliency
 * ΔE_c = (w_c − quant(w_c))²/(2·[H_F⁻¹]_cc) (the lower index on ties),
 * compensate the free columns with the OBS update, downdate H_F⁻¹.  quant()
 * is one grid per row from the row's dead-fixed weights (asymmetric min/max,
 * or symmetric).  fp64 throughout; O(d_in³) per row.
 *  W          [d_out x d_in] of w_dtype, row stride ld_w; d_in <= 128
 *             (larger returns GPTQ_ERR_UNSUPPORTED).
 *  H          [d_in x d_in] fp32 accumulated Hessian (not modified); the
 *             call applies the dead fix and p->percdamp damping itself.
 *  p          bits, percdamp, sym; group_size must be -1 (one grid per row)
 *             and act_order 0.
 *  qweight, scales [d_out x 1], zeros [d_out x 1], W_hat, row_loss: as for
 *             gptq_quantize_layer (row_loss = Σ ΔE along the row's steps).
 *  order      out [d_out x d_in] int32: the column quantized at each step;
 *             may be NULL.
 *  ws         workspace of gptq_workspace_bytes(GPTQ_WS_OBQ, d_out, d_in, 0, p).
 * SYNCHRONIZES `stream` (it reads back whether H_d was positive definite:
 * GPTQ_ERR_NOT_SPD otherwise, with the outputs undefined). */
int gptq_obq_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ld_w,
                   const float* H, const gptq_params* p, uint32_t* qweight, float* scales,
                   uint8_t* zeros, float* W_hat, int32_t* order, float* row_loss, void* ws,
                   size_t ws_bytes, gptq_stream stream);

/* Storage export of a quantized layer ("Foundations", Quantization Formats
 * and Group Size: b bits per weight plus a 16-bit scale and a 16-bit zero per
 * group, b + 32/g bits in all; Inference Execution: codes packed into 32-bit
 * words).  Reads the outputs of gptq_quantize_layer and writes
 *  qweight_dense  [d_out x ceil(d_in·bits/32)] uint32: each row one
 *                 little-endian bit stream, the code of original column c in
 *                 bits [c·bits, c·bits + bits) (bit p in bit p%32 of word
 *                 p/32; the row padded with zero bits).  For bits 4 and 8
 *                 this is the layout qweight already has; for bits 3, 32
 *                 codes fill three words; for bits 2, sixteen fill one.
 *  scales_f16     [d_out x n_groups] IEEE half of the fp32 scales, rounded to
 *                 nearest even (scales above 65504 become infinity).
 *  zeros_f16      [d_out x n_groups] IEEE half of the zero-points (exact).
 * Any output may be NULL; its input may then be NULL too.  n_groups is the
 * group count of the quantize call (1 for one group per row).  The inputs
 * stay as they are.  Asynchronous; argument errors only. */
int gptq_export(int bits, int64_t d_out, int64_t d_in, int64_t n_groups, const uint32_t* qweight,
                const float* scales, const uint8_t* zeros, uint32_t* qweight_dense,
                uint16_t* scales_f16, uint16_t* zeros_f16, gptq_stream stream);

/* Inference with an exported layer: C = A·Ŵᵀ ("Foundations", Inference
 * Execution and Modern Kernel Architectures: the FP16xINT4 pipeline --
 * dequantize the packed codes in registers as (q − zero)·scale, multiply with
 * the 16-bit activations, accumulate in fp32).  Each Ŵ value is the exact
 * product (q − z)·s of the 16-bit zero and scale, rounded once to the
 * activations' format; products are exact and accumulate in fp32.
 *  A          [M x K] 16-bit activations of a_dtype (GPTQ_F16 or GPTQ_BF16),
 *             row stride lda >= K.
 *  qweight    [N x ceil(K·bits/32)] uint32, the dense layout of gptq_export;
 *             bits 2, 3, 4 or 8.
 *  scales_f16, zeros_f16   [N x n_groups] IEEE half (gptq_export).
 *  g_idx      [K] group of each column (act-order layers) or NULL: column k
 *             is then in group k / group_size (group_size -1: one group).
 *  C          out [M x N] fp32, row stride ldc >= N.
 *  ws         NULL, or a workspace of gptq_workspace_bytes(GPTQ_WS_W4A16, N,
 *             K, M, NULL): products with few output tiles then split K and
 *             sum the fp32 partials in a fixed order (same result on every
 *             run); with NULL they run unsplit.  A non-NULL ws smaller than
 *             that size returns GPTQ_ERR_WORKSPACE.
 * M <= 4 runs a GEMV bound by the weights' HBM traffic; larger M an MFMA
 * product.  The weight words and A (from its first element to row M-1's
 * K-th value) must each stay under 4 GiB (GPTQ_ERR_UNSUPPORTED otherwise).
 * Asynchronous; argument errors only. */
int gptq_w4a16_gemm(const void* A, int a_dtype, int64_t M, int64_t K, int64_t lda,
                    const uint32_t* qweight, int bits, const uint16_t* scales_f16,
                    const uint16_t* zeros_f16, const int32_t* g_idx, int group_size,
                    int64_t n_groups, int64_t N, float* C, int64_t ldc, void* ws,
                    size_t ws_bytes, gptq_stream stream);

/* Per-stage timing, for measurement only.  gptq_timing(1) clears what was
 * recorded and starts bracketing, on the caller's stream, the launches of
 * each timed stage with a pair of HIP events; gptq_timing(0) stops.
 * gptq_timing_read() waits for the recorded events, writes the summed
 * milliseconds per stage to ms[0..n-1] (host) and clears the record:
 *   0 lazy block updates (the products W[:, later] −= Err·U[block, later]),
 *   1 in-block sweeps, 2 blocked Cholesky (panels and trailing updates),
 *   3 triangular inverse, 4 Hessian accumulation, 5 the factorization's
 *   leading panel (fp64). 
 * Timing is process-wide; enable it only while one thread issues calls. */
int gptq_timing(int enable);
int gptq_timing_read(float* ms, int n);

/* Message for the last non-zero status on the calling thread (never NULL). */
const char* gptq_last_error(void);

/* Library version string. */
const char* gptq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GPTQ_MI355X_H */
