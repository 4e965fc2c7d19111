/*
 * te_mi355x.h - C ABI of the fused norm / MLP library for AMD MI355X (gfx950).
 *
 * The operations follow the I/O contracts of three pages of the
 * TransformerEngine JAX documentation:
 *   [ACT]   "NVIDIA TransformerEngine JAX Activation"
 *   [MLP]   "NVIDIA TransformerEngine JAX LayerNorm MLP"
 *   [DENSE] "NVIDIA TransformerEngine JAX LayerNorm Dense"
 *
 * Conventions for every entry point:
 *  - Tensors are dense, row-major and contiguous in device memory. Leading
 *    axes are flattened into `rows`; the last axis is the feature axis.
 *    Weight matrices are [in_features, out_features] (the pages' x @ kernel).
 *  - All buffers, including the workspace and fp8 metadata, are owned by the
 *    caller. The library never allocates or frees device memory and keeps no
 *    pointer after a call returns. Device pointers must be 16-byte aligned.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *    null stream) and never synchronises the host. A call issues kernel
 *    launches only (no allocation, copy, memset or event), so it can be
 *    captured into a HIP graph and replayed; with timing on
 *    (te_timing_enable) the launches also carry events and must not be
 *    captured.
 *  - Arguments are fully validated before the first launch: a non-zero status
 *    means nothing was written. The message for the last failure on the
 *    calling thread is available from te_last_error(). Launch failures map to
 *    TE_ERR_HIP; faults inside kernels surface at the caller's synchronise.
 *  - Feature sizes (hidden, ffn, cols, out_features) must be positive
 *    multiples of 16 and at most 2^22, and each weight matrix must be
 *    smaller than 2 GiB (TE_ERR_UNSUPPORTED otherwise); rows may be 0: then
 *    no tensor element is written,
 *    except that te_dact_dbias sets dbias to zero and the single-tensor
 *    calls with E4M3 output (te_layernorm_fwd, te_act_lu) set their meta to
 *    amax 0, scale 1, scale_inv 1.
 *  - Supported dtype/quantisation combinations: TE_F32 with TE_QUANT_NONE;
 *    TE_BF16 with TE_QUANT_NONE or TE_QUANT_FP8_E4M3_CURRENT. Anything else
 *    returns TE_ERR_UNSUPPORTED.
 *  - fp8 is OCP E4M3 (largest finite value 448), encoded with
 *    round-to-nearest-even after saturating to +-448, with per-tensor current
 *    scaling: amax = max |t| over the whole tensor, scale = 448 / amax
 *    (1 if amax is 0), scale_inv = 1 / scale, code = E4M3(t * scale), all in
 *    fp32. Quantised values are decoded as E4M3(code) * scale_inv.
 *  - Output buffers must not overlap inputs.
 */
#ifndef TE_MI355X_H
#define TE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum te_status {
  TE_SUCCESS = 0,
  TE_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, bad size, bad enum */
  TE_ERR_UNSUPPORTED = 2,      /* valid but unsupported combination        */
  TE_ERR_WORKSPACE_TOO_SMALL = 3,
  TE_ERR_HIP = 4               /* a HIP launch or runtime call failed       */
} te_status;

typedef enum te_dtype { TE_F32 = 0, TE_BF16 = 1, TE_E4M3 = 2 } te_dtype;

/* [MLP] Inputs: norm_type "layernorm" or "rmsnorm". */
typedef enum te_norm_type { TE_LAYERNORM = 0, TE_RMSNORM = 1 } te_norm_type;

/* [ACT] Inputs: activation_type, a single name or a gated pair. A gated pair
 * (f, linear) reads a [rows, 2*cols] input whose first `cols` columns a go
 * through f and whose second `cols` columns b are the linear gate:
 * out = f(a) * b. GELU is the tanh approximation
 * 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))); GELU_ERF is x * Phi(x). */
typedef enum te_act_type {
  TE_ACT_RELU = 0,
  TE_ACT_GELU = 1,
  TE_ACT_GELU_ERF = 2,
  TE_ACT_SILU = 3,
  TE_ACT_LINEAR = 4,
  TE_ACT_REGLU = 5,  /* ("relu", "linear") */
  TE_ACT_GEGLU = 6,  /* ("gelu", "linear") */
  TE_ACT_SWIGLU = 7,  /* ("silu", "linear") */
  TE_ACT_GEGLU_ERF = 8  /* ("gelu_erf", "linear") */
} te_act_type;

/* [MLP]/[DENSE] Inputs: quantizer_set. NONE is the no-op quantizer set. */
typedef enum te_quant { TE_QUANT_NONE = 0, TE_QUANT_FP8_E4M3_CURRENT = 1 } te_quant;

/* Per-tensor fp8 metadata: three device pointers to one float each, written
 * by the call that quantises the tensor (amax, then scale and scale_inv). */
typedef struct te_fp8_meta {
  float* amax;
  float* scale;
  float* scale_inv;
} te_fp8_meta;

/* Forward context saved for the backward ([DENSE] Description: the backward
 * reuses the saved forward context). Every field is optional (NULL skips it).
 *   h1     [rows, G*ffn] GEMM1 output plus bias1, before the activation
 *          (bf16 for a TE_BF16 call, fp32 for TE_F32); this is the `x`
 *          input of te_dact_dbias.
 *   mu     [rows] fp32 per-row mean (LayerNorm only).
 *   rsigma [rows] fp32 per-row 1/sqrt(var + eps) (or 1/rms for RMSNorm).
 *   *_meta fp8 metadata of the normalised input, kernel1, the activation
 *          output and kernel2 (fp8 calls only; a meta with any NULL field is
 *          kept in the workspace instead).
 *   xq     [rows, hidden] E4M3 codes of the normalised input (fp8 only).
 *   w1q_t  [G*ffn, hidden] E4M3 codes of kernel1, transposed (fp8 only).
 *   w2q_t  [hidden, ffn] E4M3 codes of kernel2, transposed (fp8 only).
 *   actq   [rows, ffn] E4M3 codes of the activation output (fp8 only).
 *   The code buffers replace the matching workspace buffers when given. */
typedef struct te_mlp_saved {
  void* h1;
  float* mu;
  float* rsigma;
  te_fp8_meta x_meta;
  te_fp8_meta w1_meta;
  te_fp8_meta act_meta;
  te_fp8_meta w2_meta;
  uint8_t* xq;
  uint8_t* w1q_t;
  uint8_t* w2q_t;
  uint8_t* actq;
} te_mlp_saved;

/* te_layernorm_fwd - the normalisation step ([MLP] Description step (1);
 * [DENSE] Description and Inputs: gamma, beta, norm_type,
 * zero_centered_gamma, epsilon).
 *   LayerNorm: y = (x - mean) / sqrt(var + epsilon) * g + beta (biased var).
 *   RMSNorm:   y = x / sqrt(mean(x^2) + epsilon) * g; beta is ignored and may
 *              be NULL.
 *   g = 1 + gamma when zero_centered_gamma != 0, else gamma.
 * x: [rows, hidden] of x_dtype (F32 or BF16); gamma, beta: [hidden] of
 * x_dtype. y: [rows, hidden] of y_dtype: F32, BF16 or E4M3. For E4M3 the
 * whole tensor is quantised with current scaling and y_meta (required) gets
 * amax/scale/scale_inv. mu, rsigma: optional [rows] fp32 outputs (mu is not
 * written for RMSNorm). Workspace: te_layernorm_fwd_workspace_size() bytes,
 * 16-byte aligned; empty unless y_dtype is E4M3, when it holds one partial
 * maximum per workgroup of the amax pass (TE_ERR_WORKSPACE_TOO_SMALL if
 * smaller). */
te_status te_layernorm_fwd(const void* x, const void* gamma, const void* beta,
                           int64_t rows, int64_t hidden, te_dtype x_dtype,
                           te_norm_type norm_type, int zero_centered_gamma, float epsilon,
                           void* y, te_dtype y_dtype, const te_fp8_meta* y_meta,
                           float* mu, float* rsigma,
                           void* workspace, size_t workspace_bytes, void* stream);
size_t te_layernorm_fwd_workspace_size(int64_t rows, int64_t hidden, te_dtype x_dtype,
                                       te_dtype y_dtype);

/* te_layernorm_bwd - gradients of the normalisation step ([DENSE]
 * Description: the backward pass gives the gradients of every input, x,
 * gamma and beta among them, from the saved forward context).
 * With xhat = (x - mu) * rsigma (RMSNorm: x * rsigma), g = gamma (1 + gamma
 * when zero_centered_gamma != 0) and dxhat = dy * g:
 *   LayerNorm: dx = rsigma * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat))
 *   RMSNorm:   dx = rsigma * (dxhat - xhat * mean(dxhat * xhat))
 *   dgamma = sum over rows of dy * xhat; dbeta = sum over rows of dy
 *   (LayerNorm only; ignored and not written for RMSNorm).
 * dy, x, dx: [rows, hidden] of dtype (F32 or BF16); gamma: [hidden] of dtype;
 * mu (LayerNorm) and rsigma: [rows] fp32 as te_layernorm_fwd saved them.
 * dgamma, dbeta: optional [hidden] of dparam_dtype (F32 or BF16), summed in
 * fp32 in a fixed order (bitwise reproducible). hidden is at most 16384 (bf16)
 * / 8192 (fp32), else TE_ERR_UNSUPPORTED. rows = 0 zeroes dgamma and dbeta.
 * Workspace (needed with dgamma or dbeta): te_layernorm_bwd_workspace_size(). */
te_status te_layernorm_bwd(const void* dy, const void* x, const float* mu, const float* rsigma,
                           const void* gamma, int64_t rows, int64_t hidden, te_dtype dtype,
                           te_norm_type norm_type, int zero_centered_gamma, void* dx,
                           void* dgamma, void* dbeta, te_dtype dparam_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);
size_t te_layernorm_bwd_workspace_size(int64_t rows, int64_t hidden, te_dtype dtype);

/* te_act_lu - activation forward with optional fp8 output ([ACT]
 * Description: the forward applies the activation with optional
 * quantisation; Outputs: the activated tensor).
 * x: [rows, G*cols] of x_dtype (F32 or BF16), G = 2 for gated types.
 * y: [rows, cols] of y_dtype (F32, BF16 or E4M3). For E4M3, y holds the codes
 * and y_meta (required) the amax/scale/scale_inv of the whole output; the
 * page's dequantised result is te_dequantize() of it. Workspace:
 * te_act_lu_workspace_size() bytes (0 unless y_dtype is E4M3: then it holds
 * one partial maximum per workgroup of the amax pass; workspace may be NULL
 * when the size is 0). */
te_status te_act_lu(const void* x, int64_t rows, int64_t cols, te_dtype x_dtype,
                    te_act_type act_type, void* y, te_dtype y_dtype,
                    const te_fp8_meta* y_meta, void* workspace, size_t workspace_bytes,
                    void* stream);
size_t te_act_lu_workspace_size(int64_t rows, int64_t cols, te_act_type act_type, te_dtype y_dtype);

/* te_dact_dbias - activation backward with the bias-gradient reduction
 * ([ACT] Description: the backward rule computes the activation gradient;
 * [MLP] Description: the fused backward gives the activation gradient and the
 * bias reduction).
 *   dx = grad * act'(x); gated (f, linear) with x = [a | b]:
 *   dx = [grad * b * f'(a) | grad * f(a)].
 *   dbias[j] = sum over rows of dx[:, j], accumulated in fp32 from the fp32
 *   values of dx before they are rounded to `dtype`.
 * grad: [rows, cols]; x: [rows, G*cols] (the saved pre-activation h1);
 * dx: [rows, G*cols]; all of `dtype` (F32 or BF16). dbias: optional
 * [G*cols] of dbias_dtype (F32 or BF16). The reduction order is fixed, so
 * results are bitwise reproducible. Workspace:
 * te_dact_dbias_workspace_size(). */
te_status te_dact_dbias(const void* grad, const void* x, int64_t rows, int64_t cols,
                        te_dtype dtype, te_act_type act_type, void* dx,
                        void* dbias, te_dtype dbias_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);
size_t te_dact_dbias_workspace_size(int64_t rows, int64_t cols, te_act_type act_type);

/* te_dact_dbias_noalloc - te_dact_dbias for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same arguments, results
 * and errors as te_dact_dbias without the workspace: the fp32 column partials
 * of dbias live in a static device buffer of the library,
 * te_dact_dbias_noalloc_scratch_bytes() (32 MiB) per GPU, held from the first
 * call on a device until the process ends; shapes whose partials would not
 * fit return TE_ERR_UNSUPPORTED (no valid shape exceeds it with the shipped
 * kernel configuration). The call allocates nothing. Every call on one GPU
 * shares that GPU's buffer: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * The results are bitwise equal to te_dact_dbias's. */
te_status te_dact_dbias_noalloc(const void* grad, const void* x, int64_t rows, int64_t cols,
                                te_dtype dtype, te_act_type act_type, void* dx,
                                void* dbias, te_dtype dbias_dtype, void* stream);
size_t te_dact_dbias_noalloc_scratch_bytes(void);

/* te_dact_dbias_quantize - the activation backward with the bias reduction
 * and the activation gradient quantised for the fp8 backward GEMMs ([MLP]
 * Description: the fused backward's quantize_dact_dbias step returns the
 * quantised activation gradient together with the bias gradient).
 * dx is computed in fp32 exactly as in te_dact_dbias; with per-tensor current
 * scaling amax = max |dx| over the whole tensor (before any rounding), scale
 * = 448 / amax (1 if amax is 0), dx_codes [rows, G*cols] = E4M3(dx * scale),
 * and dx_meta (required) receives amax, scale and scale_inv. dbias
 * (optional, [G*cols] of dbias_dtype) as in te_dact_dbias. grad and x as in
 * te_dact_dbias. Two passes over grad and x: the scale needs the whole
 * tensor's amax before the first code is written. rows = 0 zeroes dbias and
 * sets dx_meta to amax 0, scale 1, scale_inv 1. Workspace:
 * te_dact_dbias_quantize_workspace_size(). */
te_status te_dact_dbias_quantize(const void* grad, const void* x, int64_t rows, int64_t cols,
                                 te_dtype dtype, te_act_type act_type, uint8_t* dx_codes,
                                 const te_fp8_meta* dx_meta, void* dbias, te_dtype dbias_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);
size_t te_dact_dbias_quantize_workspace_size(int64_t rows, int64_t cols, te_act_type act_type);

/* te_layernorm_dense_fwd - normalisation followed by a dense layer ([DENSE]
 * Description; Outputs: LayerNorm(x) @ kernel + bias). With
 * TE_QUANT_FP8_E4M3_CURRENT the normalised input and the kernel are both
 * quantised to E4M3 before the GEMM (fp32 accumulate).
 * x: [rows, hidden]; kernel: [hidden, out_features]; gamma, beta: [hidden];
 * bias: optional [out_features]; all of `dtype`. y: [rows, out_features] of
 * y_dtype: `dtype`, or TE_F32 for TE_BF16 inputs (the fp32 accumulator plus
 * bias written without the bf16 rounding); any other y_dtype returns
 * TE_ERR_UNSUPPORTED. Workspace: te_layernorm_dense_fwd_workspace_size(). */
te_status te_layernorm_dense_fwd(const void* x, const void* kernel, const void* gamma,
                                 const void* beta, const void* bias,
                                 int64_t rows, int64_t hidden, int64_t out_features,
                                 te_dtype dtype, te_norm_type norm_type,
                                 int zero_centered_gamma, float epsilon, te_quant quant,
                                 void* y, te_dtype y_dtype, void* workspace, size_t workspace_bytes,
                                 void* stream);
size_t te_layernorm_dense_fwd_workspace_size(int64_t rows, int64_t hidden,
                                             int64_t out_features, te_dtype dtype,
                                             te_quant quant);

/* te_layernorm_mlp_fwd - the fused feed-forward sublayer ([MLP] Description:
 * (1) normalisation, (2) GEMM1 with bias1, (3) activation, (4) GEMM2 with
 * bias2; Outputs: LayerNorm(x) -> GEMM1 -> Activation -> GEMM2).
 * x: [rows, hidden]; gamma, beta: [hidden] (beta ignored for RMSNorm);
 * kernel1: [hidden, G*ffn]; bias1: optional [G*ffn]; kernel2: [ffn, hidden];
 * bias2: optional [hidden]; all of `dtype`. y: [rows, hidden] of y_dtype:
 * `dtype`, or TE_F32 for TE_BF16 inputs (GEMM2's fp32 accumulator plus bias2
 * without the bf16 rounding); any other y_dtype returns TE_ERR_UNSUPPORTED.
 * With TE_QUANT_FP8_E4M3_CURRENT (dtype BF16): the normalised input, both
 * kernels and the activation output are quantised per tensor; GEMM1 plus
 * bias1 is rounded to bf16 (h1) and the activation is evaluated from that h1.
 * saved: optional forward context (see te_mlp_saved).
 * Workspace: te_layernorm_mlp_fwd_workspace_size(). */
te_status te_layernorm_mlp_fwd(const void* x, const void* gamma, const void* beta,
                               const void* kernel1, const void* bias1,
                               const void* kernel2, const void* bias2,
                               int64_t rows, int64_t hidden, int64_t ffn,
                               te_dtype dtype, te_norm_type norm_type,
                               int zero_centered_gamma, float epsilon,
                               te_act_type act_type, te_quant quant,
                               void* y, te_dtype y_dtype, const te_mlp_saved* saved,
                               void* workspace, size_t workspace_bytes, void* stream);
size_t te_layernorm_mlp_fwd_workspace_size(int64_t rows, int64_t hidden, int64_t ffn,
                                           te_dtype dtype, te_act_type act_type,
                                           te_quant quant);

/* te_layernorm_mlp_bwd - the backward of the fused feed-forward sublayer
 * ([MLP] Description: the backward pass gives the gradients of every
 * parameter, with the fused activation gradient + bias reduction; [DENSE]
 * Description: gradients for x, kernel, gamma, beta and bias from the
 * saved forward context). With xn the normalised input, act = activation(h1)
 * and grad = dL/dy [rows, hidden]:
 *   dkernel2 = act^T @ grad [ffn, hidden]; dbias2 = sum over rows of grad
 *   dact = grad @ kernel2^T; dh1, dbias1 = te_dact_dbias(dact, h1)
 *   dkernel1 = xn^T @ dh1 [hidden, G*ffn]; dxn = dh1 @ kernel1^T
 *   dx, dgamma, dbeta = te_layernorm_bwd(dxn, x, mu, rsigma, gamma).
 * Inputs are the forward's: x, gamma, beta, kernel1, kernel2, epsilon, and its
 * saved context te_mlp_saved.h1 (pre-activation [rows, G*ffn]), mu (LayerNorm)
 * and rsigma. xn and act are recomputed. dtype TE_BF16 only (else
 * TE_ERR_UNSUPPORTED); all GEMMs accumulate in fp32 and write bf16 (dx,
 * dkernel1, dkernel2); dgamma, dbeta, dbias1, dbias2 are fixed-order fp32
 * sums written as dparam_dtype (F32 or BF16), each optional (NULL skips it;
 * dbeta is ignored for RMSNorm). [rows, features] tensors and the kernels
 * must be smaller than 2 GiB, hidden at most 16384. Workspace:
 * te_layernorm_mlp_bwd_workspace_size(); it holds xn, act, dact, dh1, dxn,
 * a transposed copy of one kernel at a time (the data-gradient GEMMs read
 * kernel2^T and kernel1^T from it) and the fp32 partial sums. */
te_status te_layernorm_mlp_bwd(const void* grad, const void* x, const void* gamma, const void* beta,
                               const void* kernel1, const void* kernel2, const float* mu,
                               const float* rsigma, const void* h1, int64_t rows, int64_t hidden,
                               int64_t ffn, te_dtype dtype, te_norm_type norm_type,
                               int zero_centered_gamma, float epsilon, te_act_type act_type,
                               void* dx, void* dgamma, void* dbeta, void* dkernel1, void* dbias1,
                               void* dkernel2, void* dbias2, te_dtype dparam_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);
size_t te_layernorm_mlp_bwd_workspace_size(int64_t rows, int64_t hidden, int64_t ffn,
                                           te_act_type act_type);

/* te_quantize - the per-tensor fp8 quantiser on its own ([ACT] Inputs:
 * quantizer; [DENSE] Description: the normalised output and the kernel are
 * quantised before the GEMM). x: [n] of x_dtype (F32 or BF16); codes: [n]
 * bytes; meta: required, gets amax/scale/scale_inv. */
te_status te_quantize(const void* x, int64_t n, te_dtype x_dtype, uint8_t* codes,
                      const te_fp8_meta* meta, void* stream);

/* te_dequantize - E4M3(code) * scale_inv back to F32 or BF16 ([ACT]
 * Outputs: the activated tensor is dequantised back to the original
 * precision). scale_inv is read from meta on the device. */
te_status te_dequantize(const uint8_t* codes, int64_t n, const te_fp8_meta* meta,
                        void* y, te_dtype y_dtype, void* stream);

/* te_probe_mfma - a measurement aid, not an operation of the method: the
 * matrix instructions of the GEMMs' main loops with nothing around them, to
 * measure the rate and shader clock the chip sustains on them. Each of
 * `blocks` workgroups (256 threads) runs, per wave, four independent chains
 * of `iters` MFMAs on fixed pseudo-random operands: v_mfma_f32_32x32x16_bf16
 * (bf16 values of magnitude 0.5 to 2), or with fp8 != 0
 * v_mfma_f32_32x32x64_f8f6f4 on E4M3 codes. Work: blocks * 4 waves * iters
 * * 4 * 32768 flops (bf16) or * 131072 (fp8). sink: device, blocks * 256
 * floats, written (one sum per thread, so the loop stays). ticks: device, 2
 * uint64 or NULL: the shader-clock ticks (s_memtime) and 100 MHz
 * reference-clock ticks (s_memrealtime) workgroup 0 spent in its loop.
 * TE_ERR_INVALID_ARGUMENT for blocks or iters < 1 or a NULL sink. */
te_status te_probe_mfma(int fp8, int64_t iters, int blocks, float* sink, uint64_t* ticks, void* stream);

/* Message describing the last failure on the calling thread ("" if none). */
const char* te_last_error(void);

/* Library version string. */
const char* te_version(void);

/* Per-kernel timing, for benchmarks and profiling. When enabled, every
 * kernel the library launches is bracketed by a pair of HIP events recorded
 * on the launch stream. te_timing_collect() waits for the recorded events,
 * adds their durations to per-kernel totals, and returns the number of
 * distinct kernels seen; te_timing_get() reads entry i (name, launch count,
 * total milliseconds). te_timing_reset() clears the totals. Not thread-safe. */
te_status te_timing_enable(int enable);
int te_timing_collect(void);
te_status te_timing_get(int i, const char** name, int64_t* launches, double* total_ms);
void te_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* TE_MI355X_H */
