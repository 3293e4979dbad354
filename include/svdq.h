/*
 * svdq.h — C ABI of the MI355X (gfx950) SVDQuant W4A4 linear layer.
 *
 * The layer of a packed [text | video | audio] video DiT:
 *
 *     Y = X̂·L1·L2 + Q(X̂)·Q(R),    X̂ = X·diag(λ)⁻¹,   W' = diag(λ)·W = L1·L2 + R
 *
 * ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph: outliers absorbed by a
 * 16-bit low-rank branch, 4-bit residual weight, activations quantised at run time;
 * "MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on", sections "Why" and
 * "Calibration": NVFP4 blocks of 16 channels with an FP8 scale, the kernel sees X / λ, λ fed by
 * activation statistics accumulated under a modality mask.)
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - Tensors are DEVICE pointers owned by the caller; the library never keeps them and never
 *    allocates memory.  Host pointers are marked "host".
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - Matrices are row-major with the reduction dimension K contiguous.  X is [M, K] with
 *    leading dimension ldx (elements), W is [N, K] (out, in) with leading dimension ldw.
 *    Channels are in NATURAL order everywhere; any interleaving used by a kernel is private.
 *  - Packed 4-bit codes: two per byte, element 2j in the low nibble of byte j.
 *      NVFP4: sign-magnitude E2M1 codes; scales one E4M3 byte per 16 elements, [rows, K/16];
 *             plus one fp32 tensor scale g (device float[1]).
 *      INT4_G64: two's-complement int4 codes; scales one fp16 per 64 elements, [rows, K/64].
 *  - Shapes: K must be a multiple of 256; N a multiple of 256 for the GEMMs; M >= 1 any value
 *    (ragged tails are masked).  Rank r in [0, 128].  Leading dimensions must keep every row
 *    16-byte aligned, and every device pointer must be 16-byte aligned.
 *  - Streams: every call enqueues on `stream` (a hipStream_t; NULL = the default stream) and
 *    returns without synchronising.  Arguments are validated on the host before anything is
 *    enqueued; an invalid call enqueues nothing.
 *  - Errors: every entry point returns an svdq_status.  svdq_last_error() returns a
 *    thread-local message describing the last failure of the calling thread.  Inputs must be
 *    finite; NaN / Inf inputs give unspecified codes.  Calls that overlap on one stream are
 *    ordered; the library has no global mutable state (it is reentrant).
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* svdq_stream_t; /* same type as hipStream_t */

typedef enum svdq_status {
  SVDQ_OK = 0,
  SVDQ_INVALID_ARG = 1,       /* bad enum, flag or value */
  SVDQ_UNSUPPORTED_SHAPE = 2, /* sizes, leading dimensions or alignment not supported */
  SVDQ_NULL_POINTER = 3,      /* a required pointer is NULL */
  SVDQ_HIP_ERROR = 4,         /* a HIP launch or runtime call failed */
  SVDQ_NOT_IMPLEMENTED = 5
} svdq_status;

typedef enum svdq_format {
  SVDQ_NVFP4 = 0,     /* E2M1 codes, E4M3 scale per 16 along K, fp32 tensor scale */
  SVDQ_INT4_G64 = 1,  /* symmetric int4 codes, fp16 scale per 64 along K */
  SVDQ_MXFP4 = 2,     /* E2M1 codes, E8M0 scale per 32 along K (W4A4 MX variant) */
  SVDQ_MXFP8 = 3      /* E4M3 codes, E8M0 scale per 32 along K (W8A8 MX variant) */
} svdq_format;

/*
 * MX formats ("MiniMax-H3 — MXFP8 (weight-quantized, vLLM-Omni native layout)", section "Quant
 * format": E8M0 block scales per 32, round to nearest, dynamic activations).  Per block of 32
 * along K: a = max|x|; e = floor(log2 a) − emax (emax 2 for E2M1, 8 for E4M3; a == 0 gives
 * −127), clamped to [−127, 127]; scale byte = e + 127; code = element(x · 2^−e), nearest even,
 * saturating, sign bit = sign of x.  MXFP4 codes are packed two per byte (even element in the
 * low nibble, [rows, K/2]); MXFP8 codes are one byte per element ([rows, K]).  Scales are
 * [rows, K/32] bytes.  No tensor scale.
 */

/* Modality bits of a calibration mask (rows are packed text | video | audio). */
#define SVDQ_MOD_TEXT 1u
#define SVDQ_MOD_VIDEO 2u
#define SVDQ_MOD_AUDIO 4u

/* Human-readable name of a status code (static storage). */
const char* svdq_status_string(int status);
/* Message of the calling thread's last failed call ("" if none). */
const char* svdq_last_error(void);
/* ABI version: 1. */
int svdq_abi_version(void);

/*
 * λ calibration reduction ("MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated
 * on", section "Calibration": activation statistics accumulated under a modality mask feed λ;
 * opening section: one λ per input channel shared by all modalities).
 *
 *   ax[μ, k] = max over rows m of modality μ of |X[m, k]|        μ = 0 text, 1 video, 2 audio
 *   aw[k]    = max_n |W[n, k]|                                   (1 when W is NULL)
 *   sel[k]   = max over the modalities set in modality_mask of ax[μ, k]
 *   λ[k]     = sqrt(sel/aw) in fp32 for alpha == 0.5 (sel^α / aw^(1-α) in fp64 otherwise),
 *              1 when sel == 0, aw == 0 or modality_mask == 0
 *   act_amax = max_k fp32(max_μ ax[μ, k] · fp32(1/λ[k]))   (= max |X̂| over ALL rows)
 *
 * seg (host int64[4]) = {0, n_text, n_text + n_video, M}, non-decreasing.
 * accumulate != 0 folds this batch into the running maxima already held in ax / aw
 * (calibration over several batches); accumulate == 0 overwrites them.  λ and act_amax are
 * always recomputed from the (accumulated) ax and aw.
 * Outputs (device, fp32): ax [3, K], aw [K], lambda [K], act_amax [1].  Bit-exact.
 */
svdq_status svdq_calibrate_lambda(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                  const int64_t* seg, const uint16_t* W, int64_t N, int64_t ldw,
                                  uint32_t modality_mask, float alpha, int accumulate, float* ax,
                                  float* aw, float* lambda, float* act_amax,
                                  svdq_stream_t stream);

/*
 * Statistics-only "bits lost" proxy of a smoothing scale, per modality ("MiniMax-H3 NVFP4 —
 * what the smoothing scale should be calibrated on", section "Why": one block scale serves a
 * whole group of channels, so each channel's resolution falls short by the log2 ratio of the
 * group's largest smoothed magnitude to its own, and λ changes these ratios since smoothing comes
 * before quantisation).
 *
 *   c[μ, k] = fp32(ax[μ, k] · fp32(1/λ[k]))                  (lambda may be NULL: λ = 1)
 *   out[μ]  = mean over k with c[μ, k] > 0 of log2(max_{j in k's group} c[μ, j] / c[μ, k])
 *             (fp64; 0 when no channel is live)
 * Groups are `block` consecutive channels: 16 (NVFP4), 32 (MX) or 64 (int4); K % block == 0.
 * ax: device fp32 [3, K] (from svdq_calibrate_lambda); out: device fp64 [3].  Summation order
 * differs from a sequential sum (results agree to fp64 rounding).
 */
svdq_status svdq_bits_lost(const float* ax, const float* lambda, int64_t K, int64_t block,
                           double* out, svdq_stream_t stream);

/*
 * Low-rank factors on the GPU ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening
 * paragraph: a 16-bit rank-r branch absorbs the outliers of the smoothed weight).  The pages give
 * no method; this is a randomized truncated SVD of A = diag(λ)·Wᵀ (K x N):
 *   Y = A Ω, Q = orth(Y); power_iters times: Q = orth(A · orth(Aᵀ Q));  Z = Aᵀ Q
 *   ZᵀZ = U Σ² Uᵀ (ℓ x ℓ);  lora_down = bf16((Q U_r Σ_r)ᵀ) [r, K];  lora_up = bf16(Z U_r Σ_r⁻¹) [N, r]
 * W: bf16 [N, K] with row stride ldw; lambda: fp32 [K] or NULL (λ = 1); omega: fp32 [N, ell]
 * (the caller's random matrix, e.g. Gaussian); 1 <= r <= ell <= min(N, K, 160);
 * 0 <= power_iters <= 8.  Outputs (device): lora_down, lora_up (bf16), sigma (fp32 [r], the
 * estimated singular values in decreasing order; may be NULL).  workspace: device memory of at
 * least svdq_lowrank_workspace_bytes(N, K, ell) bytes, 256-byte aligned, owned by the caller and
 * free again when the stream reaches the end of the call.  Deterministic.  Factors are unique
 * only up to signs and rotations among equal singular values; the product and σ are what the
 * method fixes.
 */
int64_t svdq_lowrank_workspace_bytes(int64_t N, int64_t K, int64_t ell);
svdq_status svdq_lowrank_factors(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                 const float* lambda, const float* omega, int64_t ell, int64_t r,
                                 int power_iters, uint16_t* lora_down, uint16_t* lora_up,
                                 float* sigma, void* workspace, int64_t workspace_bytes,
                                 svdq_stream_t stream);

/*
 * GPTQ rounding of the weight residual ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)",
 * opening paragraph: the residual left by the low-rank branch is GPTQ-rounded; GPTQ as
 * published by Frantar et al. 2022).
 *
 * svdq_gptq_hessian: H [K, K] fp64 row-major (device) = Σ_m x̂_m·x̂_mᵀ over the M rows of X
 * [M, K] bf16, x̂ = fl32(x · fl32(1/λ)) (lambda may be NULL: λ = 1); accumulate != 0 adds to
 * H (calibration batches), else overwrites it.  Symmetric by construction.
 *
 * svdq_gptq_quantize_weight: the codes, scales and (NVFP4) tensor scale of
 * svdq_quantize_weight, same formats and layouts, with the residual R32 (computed exactly as
 * there from W, lambda, lora_down [r, K], lora_up [N, r]) rounded by GPTQ under H: damping
 * H + 0.01·mean(diag H)·I (an all-zero diagonal: H = I), natural column order, each quantiser
 * group's scale fixed when the sweep reaches its first column from the current values, the
 * round-to-nearest element rule applied to fl32 of each fp64 working value; the NVFP4 tensor
 * scale is the round-to-nearest one, max|R32|/2688.  H must be symmetric positive
 * semi-definite (as svdq_gptq_hessian makes it).  N a multiple of 256, K of 256.  workspace:
 * at least svdq_gptq_workspace_bytes(N, K) bytes (about 16·K² + 12·N·K), 256-byte aligned, the
 * caller's.  Deterministic.
 */
svdq_status svdq_gptq_hessian(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                              const float* lambda, int accumulate, double* H,
                              svdq_stream_t stream);
int64_t svdq_gptq_workspace_bytes(int64_t N, int64_t K);
svdq_status svdq_gptq_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K,
                                      int64_t ldw, const float* lambda,
                                      const uint16_t* lora_down, const uint16_t* lora_up,
                                      int64_t r, const double* H, uint8_t* codes, void* scales,
                                      float* tensor_scale, void* workspace,
                                      int64_t workspace_bytes, svdq_stream_t stream);

/*
 * λ grid search against the layer's output error ("MiniMax-H3 NVFP4 — what the smoothing scale
 * should be calibrated on", sections "Calibration": candidate λ scored against the OutputsError
 * objective with a number of low-rank refit iterations each, and "The metric that picks the
 * winner also hides the cost": that objective is the relative L2 against the bf16 layer over a
 * uniform sample of all rows).  For each alphas[i] (host array, each in (0, 1)), in
 * stream order on the device:
 *   λ_i, act_amax_i from the statistics ax [3, K] and aw [K] (as svdq_calibrate_lambda, same
 *   modality_mask); when r > 0 the factors of svdq_lowrank_factors (omega [N, ell], ell,
 *   power_iters); then for iterates t = 0 .. refit_iters:
 *     svdq_quantize_weight; svdq_quant_act_lowrank_down on the n_rows sampled rows X[rows[j], :]
 *     (NVFP4 with the static act_amax_i); svdq_w4a4_gemm;
 *     s_it = sqrt(Σ(Y − Y_ref)²) / sqrt(ΣY_ref²) over those rows, Y_ref = bf16(X·Wᵀ);
 *     unless t is the last iterate, the factors are refit: the rank-r factors (same omega,
 *     power_iters) of E = λ_i·W − deq(Q(R)), what the quantised residual leaves of the
 *     smoothed weight, rounded once to fp32 (the page does not define its refit; this is the
 *     alternating reading);
 *   scores[i] = min over t of s_it (iter_scores[i·(refit_iters+1) + t] = s_it when given)
 * then best_index = the first i of smallest score, best_lambda = λ_best and, when best_down /
 * best_up are given (r > 0), the factors of the best iterate of that candidate ([r, K], [N, r]
 * bf16).  refit_iters > 0 needs r > 0.
 * X [M, K], W [N, K] bf16; rows device int32 [n_rows], each in [0, M) (an index outside reads
 * the nearest row); scores / iter_scores device fp64; best_lambda device fp32 [K]; best_index
 * device int32 [1].  K and N multiples of 256; r as svdq_quantize_weight.  workspace: at least
 * svdq_lambda_search_workspace_bytes(...) bytes (−1: unsupported), 256-byte aligned, the
 * caller's.  The sums behind a score are fp64 atomics, so scores repeat to fp64 rounding; λ is
 * bit-reproducible.
 */
int64_t svdq_lambda_search_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t ell, int64_t r,
                                           int64_t n_rows, int64_t n_alpha, int refit_iters);
svdq_status svdq_lambda_search(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                               const uint16_t* W, int64_t N, int64_t ldw, const float* ax,
                               const float* aw, uint32_t modality_mask, const float* alphas,
                               int64_t n_alpha, int fmt, const float* omega, int64_t ell,
                               int64_t r, int power_iters, int refit_iters, const int32_t* rows,
                               int64_t n_rows, double* scores, double* iter_scores,
                               float* best_lambda, int32_t* best_index, uint16_t* best_down,
                               uint16_t* best_up, void* workspace, int64_t workspace_bytes,
                               svdq_stream_t stream);

/*
 * Weight preparation ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph:
 * low-rank branch plus a 4-bit residual; here rounded to nearest).
 *
 *   R[n, k] = λ_k·W[n, k] − Σ_{i=0..r-1} lora_up[n, i]·lora_down[i, k]   (fp64, i ascending)
 *   R32 = fp32(R), then quantised:
 *     NVFP4: tensor amax = max |R32|; g = amax/2688; per 16-block s = E4M3(max|x| / (6g)),
 *            codes = E2M1(x · 1/(s·g)), round to nearest even, satfinite.
 *     INT4_G64: s = fp16(max|x| / 7); codes = clamp(rint(x · 1/s), −8, 7).
 *     MXFP4 / MXFP8: per 32-block as described at svdq_format.
 * lambda may be NULL (λ = 1).  lora_down [r, K] and lora_up [N, r] are bf16 (ignored when
 * r == 0).  Outputs: codes ([N, K/2], MXFP8 [N, K]); scales ([N, K/16] E4M3 bytes, [N, K/64]
 * fp16, or [N, K/32] E8M0 bytes); tensor_scale (device float[1], g; required for NVFP4,
 * ignored otherwise).  Bit-exact.
 */
svdq_status svdq_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                 const float* lambda, const uint16_t* lora_down,
                                 const uint16_t* lora_up, int64_t r, uint8_t* codes,
                                 void* scales, float* tensor_scale, svdq_stream_t stream);

/*
 * svdq_quantize_weight with a caller workspace (same passage, arguments, results and
 * validation).  NVFP4 needs max|R32| before any code, so without a workspace the residual is
 * formed twice (once for the maximum, once to quantise); here it is formed once, R32 is kept
 * in the workspace (fp32 [N, K]) and the quantising pass reads it back.  Codes, scales and the
 * tensor scale are identical to svdq_quantize_weight's.  workspace: at least
 * svdq_quantize_weight_workspace_bytes(fmt, N, K) bytes (4·N·K for NVFP4, 0 for the
 * single-pass formats, for which the call is svdq_quantize_weight), 256-byte aligned, device
 * memory, the caller's; its contents after the call are unspecified.
 */
int64_t svdq_quantize_weight_workspace_bytes(int fmt, int64_t N, int64_t K);
svdq_status svdq_quantize_weight_ws(int fmt, const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                    const float* lambda, const uint16_t* lora_down,
                                    const uint16_t* lora_up, int64_t r, uint8_t* codes,
                                    void* scales, float* tensor_scale, void* workspace,
                                    int64_t workspace_bytes, svdq_stream_t stream);

/*
 * Activation quantisation fused with the low-rank down-projection (the kernel sees X / λ:
 * "MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on", section "Why").
 *
 *   X̂ = fp32(X) · fp32(1/λ)          (lambda may be NULL: λ = 1)
 *   NVFP4: g_a = act_amax / 2688, blocks of 16 as in svdq_quantize_weight.  act_amax is the
 *          static amax from svdq_calibrate_lambda; NULL selects a dynamic pre-pass computing
 *          max |X̂| over all M rows.  tensor_scale (device float[1]) receives g_a.
 *   INT4_G64: per 64-group scales; tensor_scale and act_amax are ignored.
 *   MXFP4 / MXFP8: per 32-block E8M0 scales (see svdq_format); tensor_scale, act_amax and
 *          sat_count are ignored.
 *   D = bf16(X̂) · lora_downᵀ         [M, r] fp32: products of bf16 operands accumulated in
 *                                     fp32 and NOT rounded to bf16 (D may be NULL iff r == 0)
 * sat_count (nullable, device uint32[1]): the number of NVFP4 blocks whose absmax exceeds the
 * tensor amax is ADDED to it (the caller zeroes it).
 * Outputs: codes [M, K/2] (MXFP8: [M, K]), scales, tensor_scale, D.  Codes and scales
 * bit-exact.  ldx larger than 2^24 elements: SVDQ_UNSUPPORTED_SHAPE.
 */
svdq_status svdq_quant_act_lowrank_down(int fmt, const uint16_t* X, int64_t M, int64_t K,
                                        int64_t ldx, const float* lambda, const float* act_amax,
                                        const uint16_t* lora_down, int64_t r, uint8_t* codes,
                                        void* scales, float* tensor_scale, float* D,
                                        uint32_t* sat_count, svdq_stream_t stream);

/*
 * W4A4 GEMM with the low-rank up-projection, bf16 output ("MiniMax-H3 · SVDQuant W4A4 (int4,
 * rank 32, GPTQ)", opening paragraph: the 4-bit residual product of the quantised activations
 * and weight, plus the 16-bit low-rank branch X̂·L1·L2, is the layer's output; section
 * "Measured": this quantised GEMM is where the layer's time goes).
 *
 *   NVFP4:    Y = bf16( g_a·g_w · Σ_k (c_a·s_a)(c_w·s_w) + D·lora_upᵀ [+ core_out[cube(m)]] )
 *   INT4_G64: Y = bf16( Σ_groups s_a·s_w · Σ_k c_a·c_w + D·lora_upᵀ )
 *   MXFP4 / MXFP8: Y = bf16( Σ_blocks 2^(e_a + e_w) · Σ_k c_a·c_w + D·lora_upᵀ ) on the
 *            hardware block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4)
 * a_codes/a_scales [M, ...] from svdq_quant_act_lowrank_down, w_codes/w_scales [N, ...] from
 * svdq_quantize_weight; g_a / g_w device float[1] (NVFP4 only).  D [M, r] fp32 (from the
 * activation kernel), lora_up [N, r] bf16.
 * core_out (nullable, fp32 [n_cubes, N]) and row_to_cube (int32 [M]) add the DeltaQuant core
 * term ("DeltaQuant on MiniMax-H3"; NVFP4 only; both or neither).  Y [M, N] bf16, leading
 * dimension ldy (a multiple of 8, >= N).  Codes, scales, D, lora_up and Y must be 16-byte
 * aligned; violations return SVDQ_UNSUPPORTED_SHAPE.  fp32 accumulation; results within the
 * layer tolerance of the float64 value.
 */
svdq_status svdq_w4a4_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                           const void* a_scales, const float* g_a, const uint8_t* w_codes,
                           const void* w_scales, const float* g_w, const float* D,
                           const uint16_t* lora_up, int64_t r, const float* core_out,
                           const int32_t* row_to_cube, uint16_t* Y, int64_t ldy,
                           svdq_stream_t stream);

/*
 * DeltaQuant cube geometry, HOST function ("DeltaQuant on MiniMax-H3", sections "The audio win
 * has a mechanism" (1-D cubes of consecutive rows for non-video rows), "Standing configuration"
 * (geometry derived per request, identical across steps) and "Deviations from the paper, and one
 * replication" (uniform cube-64)).
 *
 * Rows are [n_text | T·H·W video in raster (t, h, w) order | n_audio].  A video row belongs to
 * cube (t/ct, h/ch, w/cw) (ragged at the grid edges); text and audio rows form cubes of cube1d
 * consecutive rows of their segment.  Cubes are numbered in order of their first row; members
 * are listed ascending.  Cubes hold at most 64 rows: ct·ch·cw <= 64 and cube1d <= 64
 * (otherwise SVDQ_UNSUPPORTED_SHAPE).  All pointers are HOST pointers: row_to_cube int32 [M],
 * cube_ptr int32 [n_cubes + 1], cube_rows int32 [M], n_cubes int64 [1].  Pass row_to_cube ==
 * NULL to only count: n_cubes is written and nothing else.
 */
svdq_status svdq_cube_geometry(int64_t T, int64_t H, int64_t W, int64_t ct, int64_t ch,
                               int64_t cw, int64_t n_text, int64_t n_audio, int64_t cube1d,
                               int32_t* row_to_cube, int32_t* cube_ptr, int32_t* cube_rows,
                               int64_t* n_cubes);

/*
 * Divisor-aligned cube edges, HOST function ("DeltaQuant on MiniMax-H3", section "Deviations from
 * the paper, and one replication": divisor-aligned cube shapes are an opt-in variant; the page
 * gives no rule).  edges (host int64[3]) = for each of (T, ct), (H, ch), (W, cw) the largest
 * divisor of the grid dimension not above the requested edge (an empty dimension keeps its
 * edge), so that no video cube is ragged and none exceeds the requested shape.  Sizes >= 0,
 * edges >= 1, else SVDQ_INVALID_ARG.
 */
svdq_status svdq_cube_divisor_aligned(int64_t T, int64_t H, int64_t W, int64_t ct, int64_t ch,
                                      int64_t cw, int64_t* edges);

/*
 * Per-step cube schedule lookup, HOST function ("DeltaQuant on MiniMax-H3", section "Deviations
 * from the paper, and one replication": a timestep cube schedule, against uniform cube-64; the
 * page does not print the schedule).  table (host int64 [n_entries][4]) holds rows
 * (first_step, ct, ch, cw) with first_step strictly increasing from 0; edges (host int64[3])
 * receives the (ct, ch, cw) of the last row whose first_step is <= step.  A malformed table or a
 * negative step: SVDQ_INVALID_ARG.  The geometry of the step then comes from svdq_cube_geometry.
 */
svdq_status svdq_cube_schedule(const int64_t* table, int64_t n_entries, int64_t step,
                               int64_t* edges);

/*
 * Work groups of the DeltaQuant activation kernel, HOST function.  Consecutive cubes of the CSR
 * cube_ptr (host int32 [n_cubes + 1], cube_ptr[0] == 0) are packed greedily into groups of at
 * most 64 rows and 16 cubes.  group_ptr (host int32, room for n_cubes + 1 entries; NULL to only
 * count) receives the first cube of every group followed by n_cubes; *n_groups (host) the
 * number of groups.  A cube with no rows or more than 64 rows: SVDQ_UNSUPPORTED_SHAPE.
 */
svdq_status svdq_cube_groups(const int32_t* cube_ptr, int64_t n_cubes, int32_t* group_ptr,
                             int64_t* n_groups);

/*
 * DeltaQuant activations ("DeltaQuant on MiniMax-H3", sections "Why DeltaQuant does not beat
 * SVDQuant here", "The activation scale bound held", "Deviations from the paper, and one
 * replication").  One pass over X:
 *
 *   X̂ = fp32(X)·fp32(1/λ)
 *   core[c, k] = fp32(ascending fp32 sum of X̂ over the cube's rows) / |c|
 *   core codes: E4M3(core · 1/s_c) per core row, s_c = max_k|core[c, k]| / 448 (fp32)
 *   delta = X̂ − core[cube(m)] (fp32, unquantised core), NVFP4 with tensor amax 2·act_amax
 *   D = bf16(X̂)·lora_downᵀ  (fp32, as in svdq_quant_act_lowrank_down)
 * cube_ptr / cube_rows: device int32 CSR from svdq_cube_geometry (or the caller's own, with
 * members ascending); group_ptr: device int32 [n_groups + 1] from svdq_cube_groups over the same
 * cube_ptr (a group the packer would not make gives its cubes a NaN core scale).
 * workspace: at least svdq_delta_workspace_bytes(n_cubes, K) = 4·n_cubes·K bytes of device
 * memory, 256-byte aligned, the caller's (the fp32 cores pass through it).  Outputs: core_codes
 * [n_cubes, K] E4M3 bytes, core_scale fp32 [n_cubes], delta_codes [M, K/2], delta_scales
 * [M, K/16], g_delta float[1], D [M, r] fp32; sat_count (nullable) as in
 * svdq_quant_act_lowrank_down.  Codes and scales bit-exact.
 */
int64_t svdq_delta_workspace_bytes(int64_t n_cubes, int64_t K);
svdq_status svdq_delta_quant_act(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                 const float* lambda, const float* act_amax,
                                 const int32_t* cube_ptr, const int32_t* cube_rows,
                                 int64_t n_cubes, const int32_t* group_ptr, int64_t n_groups,
                                 const uint16_t* lora_down, int64_t r, uint8_t* core_codes,
                                 float* core_scale, uint8_t* delta_codes, uint8_t* delta_scales,
                                 float* g_delta, float* D, uint32_t* sat_count, void* workspace,
                                 int64_t workspace_bytes, svdq_stream_t stream);

/*
 * svdq_delta_quant_act without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and validation as svdq_delta_quant_act; the fp32 cores go through a
 * static device buffer of 128 MiB inside the library instead of a caller workspace (each GPU
 * the library runs on holds one until the process ends).  n_cubes·K·4 above 128 MiB:
 * SVDQ_UNSUPPORTED_SHAPE.  The buffer needs no clearing (every element the kernel reads it
 * wrote earlier in the same call), but all calls on one GPU share it: calls that overlap on a
 * GPU (on different streams, or from several threads without ordering) race and give
 * undefined results.  Allocates nothing.
 */
svdq_status svdq_delta_quant_act_noalloc(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                         const float* lambda, const float* act_amax,
                                         const int32_t* cube_ptr, const int32_t* cube_rows,
                                         int64_t n_cubes, const int32_t* group_ptr,
                                         int64_t n_groups, const uint16_t* lora_down, int64_t r,
                                         uint8_t* core_codes, float* core_scale,
                                         uint8_t* delta_codes, uint8_t* delta_scales,
                                         float* g_delta, float* D, uint32_t* sat_count,
                                         svdq_stream_t stream);

/*
 * DeltaQuant core GEMM on a 16-bit path ("DeltaQuant on MiniMax-H3", section "Deviations from
 * the paper": the core branch does not take the FP4 scaled dot):
 *   core_out[c, n] = s_c · g_w · Σ_k e4m3(core_codes[c, k]) · (c_w·s_w)[n, k]     fp32 [n_cubes, N]
 * w_* are NVFP4 weights from svdq_quantize_weight.
 */
svdq_status svdq_gemm_core(int64_t n_cubes, int64_t N, int64_t K, const uint8_t* core_codes,
                           const float* core_scale, const uint8_t* w_codes,
                           const uint8_t* w_scales, const float* g_w, float* core_out,
                           svdq_stream_t stream);

/*
 * Per-modality relative-L2 sums ("MiniMax-H3 NVFP4 — what the smoothing scale should be
 * calibrated on", section "The metric that picks the winner also hides the cost").
 * For each of the n_rows sampled rows m = rows[i] with group μ = row_group[i] in 0..3
 * (text, video, audio, uniform):
 *   Y_ref[m, :] = bf16(X[m, :] · Wᵀ)   (unsmoothed bf16 X [M, K] and W [N, K], fp32 accumulation)
 *   sums[μ][0] += Σ_n (Y[m, n] − Y_ref[m, n])²,   sums[μ][1] += Σ_n Y_ref[m, n]²   (fp64)
 * sums (device double[8]) is ADDED to (the caller zeroes it).  rows int32, row_group int8.
 */
svdq_status svdq_score_modal_rel_l2(const uint16_t* Y, int64_t ldy, const uint16_t* X,
                                    int64_t ldx, const uint16_t* W, int64_t ldw, int64_t M,
                                    int64_t N, int64_t K, const int32_t* rows,
                                    const int8_t* row_group, int64_t n_rows, double* sums,
                                    svdq_stream_t stream);

/*
 * The scoring above in two parts, for a caller that scores several candidates (λ, formats) of
 * the same batch: the reference rows do not depend on the candidate (same passage as
 * svdq_score_modal_rel_l2).
 *
 * svdq_score_reference_rows: Yref[i, :] = bf16(X[rows[i], :] · Wᵀ) for i < n_rows, fp32
 * accumulation, bf16 Yref [n_rows, N] with row stride ldr (caller-allocated, written).  Bit for
 * bit the reference rows svdq_score_modal_rel_l2 forms internally.  Shape rules as there.
 *
 * svdq_score_modal_rel_l2_ref: for each sampled row i with group μ = row_group[i] in 0..3,
 *   sums[μ][0] += Σ_n (Y[rows[i], n] − Yref[i, n])²,   sums[μ][1] += Σ_n Yref[i, n]²   (fp64)
 * sums (device double[8]) is ADDED to (the caller zeroes it).  N a positive multiple of 8;
 * ldy, ldr >= N and multiples of 8; rows outside [0, M) read row 0 or M - 1.
 */
svdq_status svdq_score_reference_rows(const uint16_t* X, int64_t ldx, const uint16_t* W,
                                      int64_t ldw, int64_t M, int64_t N, int64_t K,
                                      const int32_t* rows, int64_t n_rows, uint16_t* Yref,
                                      int64_t ldr, svdq_stream_t stream);
svdq_status svdq_score_modal_rel_l2_ref(const uint16_t* Y, int64_t ldy, const uint16_t* Yref,
                                        int64_t ldr, int64_t M, int64_t N, const int32_t* rows,
                                        const int8_t* row_group, int64_t n_rows, double* sums,
                                        svdq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
