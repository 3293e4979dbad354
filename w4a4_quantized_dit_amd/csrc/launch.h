// Internal host-side launchers (called by api.cpp after validation).  Each returns the HIP
// error of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

hipError_t launch_calibrate(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                            const int64_t seg[4], const uint16_t* W, int64_t N, int64_t ldw,
                            uint32_t mask, float alpha, int accumulate, float* ax, float* aw,
                            float* lambda, float* act_amax, hipStream_t s);
// λ and the static activation amax from the calibration statistics (the last step of
// launch_calibrate).
hipError_t launch_lambda(const float* ax, const float* aw, int64_t K, uint32_t mask, float alpha,
                         float* lambda, float* act_amax, hipStream_t s);
hipError_t launch_bits_lost(const float* ax, const float* lambda, int64_t K, int block,
                            double* out, hipStream_t s);
int64_t lowrank_workspace_bytes(int64_t N, int64_t K, int64_t ell);
int lowrank_max_ell();
hipError_t launch_lowrank(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                          const float* lambda, const float* omega, int64_t ell, int64_t r,
                          int power_iters, uint16_t* lora_down, uint16_t* lora_up, float* sigma,
                          void* workspace, hipStream_t s);

// The same factors for an fp32 matrix E [N, K] (row stride lde) in place of diag(λ)·Wᵀ's
// transpose: the rank-r approximation of Eᵀ.
hipError_t launch_lowrank_f32(const float* E, int64_t N, int64_t K, int64_t lde,
                              const float* omega, int64_t ell, int64_t r, int power_iters,
                              uint16_t* lora_down, uint16_t* lora_up, float* sigma,
                              void* workspace, hipStream_t s);

hipError_t launch_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                  const float* lambda, const uint16_t* down, const uint16_t* up,
                                  int64_t r, uint8_t* codes, void* scales, float* tensor_scale,
                                  hipStream_t s);

// NVFP4 launch_quantize_weight through R32 [N, K] fp32 scratch (the residual is formed once
// and stored, and the quantising pass reads it back): same codes, scales and tensor scale.
hipError_t launch_quantize_weight_r32(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                      const float* lambda, const uint16_t* down,
                                      const uint16_t* up, int64_t r, uint8_t* codes, void* scales,
                                      float* tensor_scale, float* R32, hipStream_t s);

// R32 = fl32(λ·W − up·down) exactly as launch_quantize_weight forms it, into R32 [N, K]; with
// tensor_scale, also the NVFP4 tensor scale max|R32| / 2688 (1 when the residual is zero).
hipError_t launch_residual_f32(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                               const float* lambda, const uint16_t* down, const uint16_t* up,
                               int64_t r, float* R32, float* tensor_scale, hipStream_t s);

hipError_t launch_quant_act(int fmt, const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                            const float* lambda, const float* act_amax, const uint16_t* down,
                            int64_t r, uint8_t* codes, void* scales, float* tensor_scale,
                            float* D, uint32_t* sat, hipStream_t s);

// LDS bytes (static + dynamic) of the activation kernel for K channels at rank r; a launch
// needs at most 160 KB.
size_t quant_act_lds_bytes(int64_t K, int64_t r);


// Compute units of the current device (cached per device; 0 if the query fails).
int device_cus();

hipError_t launch_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const void* a_scales, const float* g_a, const uint8_t* w_codes,
                       const void* w_scales, const float* g_w, const float* D,
                       const uint16_t* up, int64_t r, const float* core_out,
                       const int32_t* row_to_cube, uint16_t* Y, int64_t ldy, hipStream_t s);

// DeltaQuant activations over host-packed cube groups (group_ptr: cube index of each group's first
// cube, n_groups + 1 entries; at most 64 rows and 16 cubes per group); workspace: fp32
// [n_cubes, K] (delta_workspace_bytes).
int64_t delta_workspace_bytes(int64_t n_cubes, int64_t K);
constexpr int64_t kDeltaGroupRows = 64;
// The allocation-free variant's static scratch (fp32 cores, bytes) and its device address on the
// current device (looked up once per device).
constexpr size_t kDeltaScratchBytes = (size_t)128 << 20;
hipError_t delta_scratch(void** ptr);
constexpr int64_t kDeltaGroupCubes = 16;
hipError_t launch_delta_quant_act(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                  const float* lambda, const float* act_amax,
                                  const int32_t* cube_ptr, const int32_t* cube_rows,
                                  const int32_t* group_ptr, int64_t n_groups,
                                  const uint16_t* down, int64_t r, uint8_t* core_codes,
                                  float* core_scale, uint8_t* delta_codes, uint8_t* delta_scales,
                                  float* g_delta, float* D, uint32_t* sat, void* workspace,
                                  hipStream_t s);

hipError_t launch_gemm_core(int64_t n_cubes, int64_t N, int64_t K, const uint8_t* core_codes,
                            const float* core_scale, const uint8_t* w_codes,
                            const uint8_t* w_scales, const float* g_w, float* core_out,
                            hipStream_t s);

hipError_t launch_score(const uint16_t* Y, int64_t ldy, const uint16_t* X, int64_t ldx,
                        const uint16_t* W, int64_t ldw, int64_t M, int64_t N, int64_t K,
                        const int32_t* rows, const int8_t* grp, int64_t n_rows, double* sums,
                        hipStream_t s);

hipError_t launch_gptq_hessian(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                               const float* lambda, int accumulate, double* H, hipStream_t s);
int64_t gptq_workspace_bytes(int64_t N, int64_t K);
hipError_t launch_gptq_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K,
                                       int64_t ldw, const float* lambda, const uint16_t* down,
                                       const uint16_t* up, int64_t r, const double* H,
                                       uint8_t* codes, void* scales, float* tensor_scale,
                                       void* workspace, hipStream_t s);

// Y_ref = bf16(X·Wᵀ) of the sampled rows (the scoring kernel's reference, fp32 accumulation)
// into Yref [n_rows, N] (row stride ldr).
hipError_t launch_score_ref(const uint16_t* Y, int64_t ldy, const uint16_t* Yref, int64_t ldr,
                            int64_t M, int64_t N, const int32_t* rows, const int8_t* grp,
                            int64_t n_rows, double* sums, hipStream_t s);
hipError_t launch_reference_rows(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                                 int64_t M, int64_t N, int64_t K, const int32_t* rows,
                                 int64_t n_rows, uint16_t* Yref, int64_t ldr, hipStream_t s);

int64_t lambda_search_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t ell, int64_t r,
                                      int64_t n_rows, int64_t n_alpha, int refit_iters);
hipError_t launch_lambda_search(const uint16_t* X, int64_t M, int64_t ldx, const uint16_t* W,
                                int64_t N, int64_t K, int64_t ldw, const float* ax,
                                const float* aw, uint32_t mask, const float* alphas,
                                int64_t n_alpha, int fmt, const float* omega, int64_t ell,
                                int64_t r, int power_iters, int refit_iters,
                                const int32_t* rows, int64_t n_rows, double* scores,
                                double* iter_scores, float* best_lambda, int32_t* best_index,
                                uint16_t* best_down, uint16_t* best_up, void* workspace,
                                hipStream_t s);

}  // namespace svdq
