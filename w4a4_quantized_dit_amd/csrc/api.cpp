// C ABI: argument validation on the host (nothing is enqueued for an invalid call), dispatch to
// the gfx950 kernels, status codes and a thread-local error message.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/svdq.h"
#include "launch.h"

namespace svdq {
int64_t cube_count(int64_t T, int64_t H, int64_t W, int64_t ct, int64_t ch, int64_t cw,
                   int64_t n_text, int64_t n_audio, int64_t c1);
void cube_geometry_fill(int64_t T, int64_t H, int64_t W, int64_t ct, int64_t ch, int64_t cw,
                        int64_t n_text, int64_t n_audio, int64_t c1, int32_t* row_to_cube,
                        int32_t* cube_ptr, int32_t* cube_rows);
int64_t divisor_edge(int64_t n, int64_t e);
int64_t cube_groups(const int32_t* cube_ptr, int64_t n_cubes, int64_t max_rows,
                    int64_t max_cubes, int32_t* group_ptr);
}  // namespace svdq

namespace {

thread_local char g_err[512] = "";

svdq_status fail(svdq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

svdq_status ok() {
  g_err[0] = '\0';
  return SVDQ_OK;
}

svdq_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SVDQ_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                                \
  do {                                                                                \
    if (!(p)) return fail(SVDQ_NULL_POINTER, "%s: '%s' must not be NULL", fn, #p);    \
  } while (0)
#define REQUIRE_ALIGNED(p)                                                                \
  do {                                                                                    \
    if ((p) && !aligned16(p))                                                             \
      return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: '%s' must be 16-byte aligned", fn, #p);    \
  } while (0)

svdq_status check_k(const char* fn, int64_t K) {
  if (K <= 0 || K % 256 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: K=%lld must be a positive multiple of 256", fn,
                (long long)K);
  return SVDQ_OK;
}

svdq_status check_ld(const char* fn, const char* name, int64_t ld, int64_t K) {
  if (ld < K || ld % 8 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE,
                "%s: %s=%lld must be >= K=%lld and a multiple of 8 (16-byte rows)", fn, name,
                (long long)ld, (long long)K);
  return SVDQ_OK;
}

// The activation kernels address the 64 rows of a workgroup with 32-bit byte offsets.
svdq_status check_act_ld(const char* fn, int64_t ldx) {
  if (ldx > ((int64_t)1 << 24))
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: ldx=%lld exceeds 2^24 elements", fn,
                (long long)ldx);
  return SVDQ_OK;
}

// The activation kernel keeps 1/λ for all K channels and the rank-r slice of L1 in LDS.
svdq_status check_act_lds(const char* fn, int64_t K, int64_t r) {
  const size_t need = svdq::quant_act_lds_bytes(K, r);
  if (need > 160 * 1024)
    return fail(SVDQ_UNSUPPORTED_SHAPE,
                "%s: K=%lld at rank %lld needs %zu bytes of LDS, more than the 160 KB of a CU", fn,
                (long long)K, (long long)r, need);
  return SVDQ_OK;
}

svdq_status check_rank(const char* fn, int64_t r) {
  if (r < 0 || r > 128 || r % 8 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: rank r=%lld must be a multiple of 8 in [0, 128]", fn,
                (long long)r);
  return SVDQ_OK;
}

svdq_status check_fmt(const char* fn, int fmt) {
  if (fmt != SVDQ_NVFP4 && fmt != SVDQ_INT4_G64 && fmt != SVDQ_MXFP4 && fmt != SVDQ_MXFP8)
    return fail(SVDQ_INVALID_ARG, "%s: unknown format %d", fn, fmt);
  return SVDQ_OK;
}

#define TRY(x)                      \
  do {                              \
    svdq_status _s = (x);           \
    if (_s != SVDQ_OK) return _s;   \
  } while (0)

}  // namespace

extern "C" {

const char* svdq_status_string(int status) {
  switch (status) {
    case SVDQ_OK: return "SVDQ_OK";
    case SVDQ_INVALID_ARG: return "SVDQ_INVALID_ARG";
    case SVDQ_UNSUPPORTED_SHAPE: return "SVDQ_UNSUPPORTED_SHAPE";
    case SVDQ_NULL_POINTER: return "SVDQ_NULL_POINTER";
    case SVDQ_HIP_ERROR: return "SVDQ_HIP_ERROR";
    case SVDQ_NOT_IMPLEMENTED: return "SVDQ_NOT_IMPLEMENTED";
    default: return "SVDQ_UNKNOWN_STATUS";
  }
}

const char* svdq_last_error(void) { return g_err; }

int svdq_abi_version(void) { return 1; }

svdq_status svdq_calibrate_lambda(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                  const int64_t* seg, const uint16_t* W, int64_t N, int64_t ldw,
                                  uint32_t modality_mask, float alpha, int accumulate, float* ax,
                                  float* aw, float* lambda, float* act_amax,
                                  svdq_stream_t stream) {
  const char* fn = "svdq_calibrate_lambda";
  REQUIRE_PTR(X); REQUIRE_PTR(seg); REQUIRE_PTR(ax); REQUIRE_PTR(aw); REQUIRE_PTR(lambda);
  REQUIRE_PTR(act_amax);
  REQUIRE_ALIGNED(X); REQUIRE_ALIGNED(W);
  if (M < 1) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: M=%lld must be >= 1", fn, (long long)M);
  TRY(check_k(fn, K));
  TRY(check_ld(fn, "ldx", ldx, K));
  if (seg[0] != 0 || seg[3] != M || seg[1] < seg[0] || seg[2] < seg[1] || seg[3] < seg[2])
    return fail(SVDQ_INVALID_ARG, "%s: seg must be non-decreasing {0, n_text, n_text+n_video, M}",
                fn);
  if (modality_mask > 7u) return fail(SVDQ_INVALID_ARG, "%s: modality_mask=%u > 7", fn, modality_mask);
  if (!(alpha > 0.0f && alpha < 1.0f))
    return fail(SVDQ_INVALID_ARG, "%s: alpha must lie in (0, 1)", fn);
  if (W) {
    if (N < 1) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld must be >= 1", fn, (long long)N);
    TRY(check_ld(fn, "ldw", ldw, K));
  }
  return hip_result(svdq::launch_calibrate(X, M, K, ldx, seg, W, N, ldw, modality_mask, alpha,
                                           accumulate, ax, aw, lambda, act_amax,
                                           reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

int64_t svdq_lowrank_workspace_bytes(int64_t N, int64_t K, int64_t ell) {
  if (N < 1 || K < 1 || ell < 1 || ell > svdq::lowrank_max_ell()) return -1;
  return svdq::lowrank_workspace_bytes(N, K, ell);
}

svdq_status svdq_lowrank_factors(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                 const float* lambda, const float* omega, int64_t ell, int64_t r,
                                 int power_iters, uint16_t* lora_down, uint16_t* lora_up,
                                 float* sigma, void* workspace, int64_t workspace_bytes,
                                 svdq_stream_t stream) {
  const char* fn = "svdq_lowrank_factors";
  REQUIRE_PTR(W); REQUIRE_PTR(omega); REQUIRE_PTR(lora_down); REQUIRE_PTR(lora_up);
  REQUIRE_PTR(workspace);
  REQUIRE_ALIGNED(W); REQUIRE_ALIGNED(omega); REQUIRE_ALIGNED(lambda); REQUIRE_ALIGNED(sigma);
  REQUIRE_ALIGNED(lora_down); REQUIRE_ALIGNED(lora_up);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace must be 256-byte aligned", fn);
  if (N < 1 || K < 1)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld, K=%lld must be >= 1", fn, (long long)N,
                (long long)K);
  TRY(check_ld(fn, "ldw", ldw, K));
  const int64_t lim = svdq::lowrank_max_ell();
  if (r < 1 || ell < r || ell > lim || ell > N || ell > K)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: need 1 <= r (%lld) <= ell (%lld) <= min(N, K, %lld)",
                fn, (long long)r, (long long)ell, (long long)lim);
  if (power_iters < 0 || power_iters > 8)
    return fail(SVDQ_INVALID_ARG, "%s: power_iters=%d must lie in [0, 8]", fn, power_iters);
  const int64_t need = svdq::lowrank_workspace_bytes(N, K, ell);
  if (workspace_bytes < need)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace of %lld bytes, needs %lld", fn,
                (long long)workspace_bytes, (long long)need);
  return hip_result(svdq::launch_lowrank(W, N, K, ldw, lambda, omega, ell, r, power_iters,
                                         lora_down, lora_up, sigma, workspace,
                                         reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

svdq_status svdq_gptq_hessian(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                              const float* lambda, int accumulate, double* H,
                              svdq_stream_t stream) {
  const char* fn = "svdq_gptq_hessian";
  REQUIRE_PTR(X); REQUIRE_PTR(H);
  if (M < 1) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: M=%lld must be >= 1", fn, (long long)M);
  TRY(check_k(fn, K));
  TRY(check_ld(fn, "ldx", ldx, K));
  return hip_result(svdq::launch_gptq_hessian(X, M, K, ldx, lambda, accumulate ? 1 : 0, H,
                                              reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

int64_t svdq_gptq_workspace_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return -1;
  return svdq::gptq_workspace_bytes(N, K);
}

svdq_status svdq_gptq_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K,
                                      int64_t ldw, const float* lambda,
                                      const uint16_t* lora_down, const uint16_t* lora_up,
                                      int64_t r, const double* H, uint8_t* codes, void* scales,
                                      float* tensor_scale, void* workspace,
                                      int64_t workspace_bytes, svdq_stream_t stream) {
  const char* fn = "svdq_gptq_quantize_weight";
  TRY(check_fmt(fn, fmt));
  REQUIRE_PTR(W); REQUIRE_PTR(H); REQUIRE_PTR(codes); REQUIRE_PTR(scales); REQUIRE_PTR(workspace);
  REQUIRE_ALIGNED(W); REQUIRE_ALIGNED(codes);
  if (fmt == SVDQ_NVFP4) REQUIRE_PTR(tensor_scale);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace must be 256-byte aligned", fn);
  TRY(check_k(fn, K));
  TRY(check_ld(fn, "ldw", ldw, K));
  if (N < 1 || N % 256 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld must be a positive multiple of 256", fn,
                (long long)N);
  TRY(check_rank(fn, r));
  if (r > 0) { REQUIRE_PTR(lora_down); REQUIRE_PTR(lora_up); }
  const int64_t need = svdq::gptq_workspace_bytes(N, K);
  if (workspace_bytes < need)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace of %lld bytes, needs %lld", fn,
                (long long)workspace_bytes, (long long)need);
  return hip_result(svdq::launch_gptq_quantize_weight(fmt, W, N, K, ldw, lambda, lora_down,
                                                      lora_up, r, H, codes, scales, tensor_scale,
                                                      workspace,
                                                      reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

int64_t svdq_lambda_search_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t ell, int64_t r,
                                           int64_t n_rows, int64_t n_alpha, int refit_iters) {
  if (fmt < 0 || fmt > 3 || N < 1 || K < 1 || n_rows < 1 || n_alpha < 1 || r < 0) return -1;
  if (refit_iters < 0 || (refit_iters > 0 && r == 0)) return -1;
  if (r > 0 && (ell < r || ell > svdq::lowrank_max_ell())) return -1;
  return svdq::lambda_search_workspace_bytes(fmt, N, K, ell, r, n_rows, n_alpha, refit_iters);
}

svdq_status svdq_lambda_search(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                               const uint16_t* W, int64_t N, int64_t ldw, const float* ax,
                               const float* aw, uint32_t modality_mask, const float* alphas,
                               int64_t n_alpha, int fmt, const float* omega, int64_t ell,
                               int64_t r, int power_iters, int refit_iters, const int32_t* rows,
                               int64_t n_rows, double* scores, double* iter_scores,
                               float* best_lambda, int32_t* best_index, uint16_t* best_down,
                               uint16_t* best_up, void* workspace, int64_t workspace_bytes,
                               svdq_stream_t stream) {
  const char* fn = "svdq_lambda_search";
  TRY(check_fmt(fn, fmt));
  REQUIRE_PTR(X); REQUIRE_PTR(W); REQUIRE_PTR(ax); REQUIRE_PTR(aw); REQUIRE_PTR(alphas);
  REQUIRE_PTR(rows); REQUIRE_PTR(scores); REQUIRE_PTR(best_lambda); REQUIRE_PTR(best_index);
  REQUIRE_PTR(workspace);
  REQUIRE_ALIGNED(X); REQUIRE_ALIGNED(W); REQUIRE_ALIGNED(omega);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace must be 256-byte aligned", fn);
  if (M < 1) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: M=%lld must be >= 1", fn, (long long)M);
  TRY(check_k(fn, K));
  TRY(check_ld(fn, "ldx", ldx, K));
  TRY(check_ld(fn, "ldw", ldw, K));
  if (N < 1 || N % 256 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld must be a positive multiple of 256", fn,
                (long long)N);
  if (modality_mask > 7u) return fail(SVDQ_INVALID_ARG, "%s: modality_mask=%u > 7", fn, modality_mask);
  if (n_alpha < 1 || n_alpha > 1024)
    return fail(SVDQ_INVALID_ARG, "%s: n_alpha=%lld must lie in [1, 1024]", fn, (long long)n_alpha);
  for (int64_t i = 0; i < n_alpha; ++i)
    if (!(alphas[i] > 0.0f && alphas[i] < 1.0f))
      return fail(SVDQ_INVALID_ARG, "%s: alphas[%lld] must lie in (0, 1)", fn, (long long)i);
  TRY(check_rank(fn, r));
  if (r > 0) {
    REQUIRE_PTR(omega);
    const int64_t lim = svdq::lowrank_max_ell();
    if (ell < r || ell > lim || ell > N || ell > K)
      return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: need r (%lld) <= ell (%lld) <= min(N, K, %lld)",
                  fn, (long long)r, (long long)ell, (long long)lim);
    if (power_iters < 0 || power_iters > 8)
      return fail(SVDQ_INVALID_ARG, "%s: power_iters=%d must lie in [0, 8]", fn, power_iters);
  }
  if (refit_iters < 0 || refit_iters > 1000)
    return fail(SVDQ_INVALID_ARG, "%s: refit_iters=%d must lie in [0, 1000]", fn, refit_iters);
  if (refit_iters > 0 && r == 0)
    return fail(SVDQ_INVALID_ARG, "%s: refit iterations need a low-rank branch (r > 0)", fn);
  if ((best_down == nullptr) != (best_up == nullptr))
    return fail(SVDQ_NULL_POINTER, "%s: best_down and best_up go together", fn);
  if (best_down != nullptr && r == 0)
    return fail(SVDQ_INVALID_ARG, "%s: best factors need a low-rank branch (r > 0)", fn);
  REQUIRE_ALIGNED(best_down); REQUIRE_ALIGNED(best_up);
  if (n_rows < 1)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: n_rows=%lld must be >= 1", fn, (long long)n_rows);
  TRY(check_act_lds(fn, K, r));
  const int64_t need =
      svdq::lambda_search_workspace_bytes(fmt, N, K, ell, r, n_rows, n_alpha, refit_iters);
  if (workspace_bytes < need)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace of %lld bytes, needs %lld", fn,
                (long long)workspace_bytes, (long long)need);
  return hip_result(
      svdq::launch_lambda_search(X, M, ldx, W, N, K, ldw, ax, aw, modality_mask, alphas, n_alpha,
                                 fmt, omega, ell, r, power_iters, refit_iters, rows, n_rows,
                                 scores, iter_scores, best_lambda, best_index, best_down,
                                 best_up, workspace, reinterpret_cast<hipStream_t>(stream)),
      fn);
}

svdq_status svdq_bits_lost(const float* ax, const float* lambda, int64_t K, int64_t block,
                           double* out, svdq_stream_t stream) {
  const char* fn = "svdq_bits_lost";
  REQUIRE_PTR(ax); REQUIRE_PTR(out);
  if (block != 16 && block != 32 && block != 64)
    return fail(SVDQ_INVALID_ARG, "%s: block=%lld must be 16, 32 or 64", fn, (long long)block);
  if (K < block || K % block != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: K=%lld must be a positive multiple of block=%lld", fn,
                (long long)K, (long long)block);
  return hip_result(svdq::launch_bits_lost(ax, lambda, K, (int)block, out,
                                           reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

namespace {
// (static: inside the extern "C" block an unnamed namespace alone does not make it internal)
static svdq_status check_quantize_weight(const char* fn, int fmt, const uint16_t* W, int64_t N,
                                  int64_t K, int64_t ldw, const uint16_t* lora_down,
                                  const uint16_t* lora_up, int64_t r, uint8_t* codes,
                                  void* scales, float* tensor_scale) {
  TRY(check_fmt(fn, fmt));
  REQUIRE_PTR(W); REQUIRE_PTR(codes); REQUIRE_PTR(scales);
  if (fmt == SVDQ_NVFP4) REQUIRE_PTR(tensor_scale);
  REQUIRE_ALIGNED(W); REQUIRE_ALIGNED(codes); REQUIRE_ALIGNED(lora_down); REQUIRE_ALIGNED(lora_up);
  if (N < 1) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld must be >= 1", fn, (long long)N);
  TRY(check_k(fn, K));
  TRY(check_ld(fn, "ldw", ldw, K));
  TRY(check_rank(fn, r));
  if (r > 0) { REQUIRE_PTR(lora_down); REQUIRE_PTR(lora_up); }
  return ok();
}
}  // namespace

int64_t svdq_quantize_weight_workspace_bytes(int fmt, int64_t N, int64_t K) {
  if (fmt != SVDQ_NVFP4 || N < 1 || K < 1) return 0;
  return 4 * N * K;
}

svdq_status svdq_quantize_weight_ws(int fmt, const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                    const float* lambda, const uint16_t* lora_down,
                                    const uint16_t* lora_up, int64_t r, uint8_t* codes,
                                    void* scales, float* tensor_scale, void* workspace,
                                    int64_t workspace_bytes, svdq_stream_t stream) {
  const char* fn = "svdq_quantize_weight_ws";
  TRY(check_quantize_weight(fn, fmt, W, N, K, ldw, lora_down, lora_up, r, codes, scales,
                            tensor_scale));
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (fmt != SVDQ_NVFP4)  // single-pass formats: the workspace is not needed
    return hip_result(svdq::launch_quantize_weight(fmt, W, N, K, ldw, lambda, lora_down, lora_up,
                                                   r, codes, scales, tensor_scale, s),
                      fn);
  REQUIRE_PTR(workspace);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace must be 256-byte aligned", fn);
  const int64_t need = svdq_quantize_weight_workspace_bytes(fmt, N, K);
  if (workspace_bytes < need)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace of %lld bytes, needs %lld", fn,
                (long long)workspace_bytes, (long long)need);
  return hip_result(svdq::launch_quantize_weight_r32(W, N, K, ldw, lambda, lora_down, lora_up, r,
                                                     codes, scales, tensor_scale,
                                                     static_cast<float*>(workspace), s),
                    fn);
}

svdq_status svdq_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                 const float* lambda, const uint16_t* lora_down,
                                 const uint16_t* lora_up, int64_t r, uint8_t* codes,
                                 void* scales, float* tensor_scale, svdq_stream_t stream) {
  const char* fn = "svdq_quantize_weight";
  TRY(check_quantize_weight(fn, fmt, W, N, K, ldw, lora_down, lora_up, r, codes, scales,
                            tensor_scale));
  return hip_result(svdq::launch_quantize_weight(fmt, W, N, K, ldw, lambda, lora_down, lora_up, r,
                                                 codes, scales, tensor_scale,
                                                 reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

svdq_status svdq_quant_act_lowrank_down(int fmt, const uint16_t* X, int64_t M, int64_t K,
                                        int64_t ldx, const float* lambda, const float* act_amax,
                                        const uint16_t* lora_down, int64_t r, uint8_t* codes,
                                        void* scales, float* tensor_scale, float* D,
                                        uint32_t* sat_count, svdq_stream_t stream) {
  const char* fn = "svdq_quant_act_lowrank_down";
  TRY(check_fmt(fn, fmt));
  REQUIRE_PTR(X); REQUIRE_PTR(codes); REQUIRE_PTR(scales);
  if (fmt == SVDQ_NVFP4) REQUIRE_PTR(tensor_scale);
  REQUIRE_ALIGNED(X); REQUIRE_ALIGNED(codes); REQUIRE_ALIGNED(scales); REQUIRE_ALIGNED(lora_down);
  REQUIRE_ALIGNED(D);
  if (M < 1) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: M=%lld must be >= 1", fn, (long long)M);
  TRY(check_k(fn, K));
  TRY(check_ld(fn, "ldx", ldx, K));
  TRY(check_act_ld(fn, ldx));
  TRY(check_rank(fn, r));
  if (r > 0) { REQUIRE_PTR(lora_down); REQUIRE_PTR(D); }
  TRY(check_act_lds(fn, K, r));
  return hip_result(svdq::launch_quant_act(fmt, X, M, K, ldx, lambda, act_amax, lora_down, r,
                                           codes, scales, tensor_scale, D, sat_count,
                                           reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

svdq_status svdq_w4a4_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                           const void* a_scales, const float* g_a, const uint8_t* w_codes,
                           const void* w_scales, const float* g_w, const float* D,
                           const uint16_t* lora_up, int64_t r, const float* core_out,
                           const int32_t* row_to_cube, uint16_t* Y, int64_t ldy,
                           svdq_stream_t stream) {
  const char* fn = "svdq_w4a4_gemm";
  TRY(check_fmt(fn, fmt));
  REQUIRE_PTR(a_codes); REQUIRE_PTR(a_scales); REQUIRE_PTR(w_codes); REQUIRE_PTR(w_scales);
  REQUIRE_PTR(Y);
  if (fmt == SVDQ_NVFP4) { REQUIRE_PTR(g_a); REQUIRE_PTR(g_w); }
  REQUIRE_ALIGNED(a_codes); REQUIRE_ALIGNED(w_codes); REQUIRE_ALIGNED(D); REQUIRE_ALIGNED(lora_up);
  REQUIRE_ALIGNED(a_scales); REQUIRE_ALIGNED(w_scales); REQUIRE_ALIGNED(Y);
  if (M < 1) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: M=%lld must be >= 1", fn, (long long)M);
  if (N < 1 || N % 256 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld must be a positive multiple of 256", fn,
                (long long)N);
  TRY(check_k(fn, K));
  TRY(check_rank(fn, r));
  if (ldy < N || ldy % 8 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: ldy=%lld must be >= N and a multiple of 8", fn,
                (long long)ldy);
  if (r > 0) { REQUIRE_PTR(D); REQUIRE_PTR(lora_up); }
  if ((core_out == nullptr) != (row_to_cube == nullptr))
    return fail(SVDQ_INVALID_ARG, "%s: core_out and row_to_cube must be given together", fn);
  if (core_out && fmt != SVDQ_NVFP4)
    return fail(SVDQ_INVALID_ARG, "%s: the core term is defined for NVFP4 only", fn);
  return hip_result(svdq::launch_gemm(fmt, M, N, K, a_codes, a_scales, g_a, w_codes, w_scales, g_w,
                                      D, lora_up, r, core_out, row_to_cube, Y, ldy,
                                      reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

svdq_status svdq_cube_geometry(int64_t T, int64_t H, int64_t W, int64_t ct, int64_t ch,
                               int64_t cw, int64_t n_text, int64_t n_audio, int64_t cube1d,
                               int32_t* row_to_cube, int32_t* cube_ptr, int32_t* cube_rows,
                               int64_t* n_cubes) {
  const char* fn = "svdq_cube_geometry";
  REQUIRE_PTR(n_cubes);
  if (T < 0 || H < 0 || W < 0 || n_text < 0 || n_audio < 0)
    return fail(SVDQ_INVALID_ARG, "%s: sizes must be non-negative", fn);
  if (ct < 1 || ch < 1 || cw < 1 || cube1d < 1)
    return fail(SVDQ_INVALID_ARG, "%s: cube sizes must be >= 1", fn);
  if (ct > 64 || ch > 64 || cw > 64 || ct * ch * cw > 64 || cube1d > 64)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: cubes of more than 64 rows are not supported", fn);
  const int64_t M = n_text + T * H * W + n_audio;
  if (M < 1 || M > INT32_MAX) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: bad row count", fn);
  *n_cubes = svdq::cube_count(T, H, W, ct, ch, cw, n_text, n_audio, cube1d);
  if (!row_to_cube) return ok();
  REQUIRE_PTR(cube_ptr); REQUIRE_PTR(cube_rows);
  svdq::cube_geometry_fill(T, H, W, ct, ch, cw, n_text, n_audio, cube1d, row_to_cube, cube_ptr,
                           cube_rows);
  return ok();
}

svdq_status svdq_cube_divisor_aligned(int64_t T, int64_t H, int64_t W, int64_t ct, int64_t ch,
                                      int64_t cw, int64_t* edges) {
  const char* fn = "svdq_cube_divisor_aligned";
  REQUIRE_PTR(edges);
  if (T < 0 || H < 0 || W < 0) return fail(SVDQ_INVALID_ARG, "%s: sizes must be non-negative", fn);
  if (ct < 1 || ch < 1 || cw < 1) return fail(SVDQ_INVALID_ARG, "%s: edges must be >= 1", fn);
  edges[0] = svdq::divisor_edge(T, ct);
  edges[1] = svdq::divisor_edge(H, ch);
  edges[2] = svdq::divisor_edge(W, cw);
  return ok();
}

svdq_status svdq_cube_schedule(const int64_t* table, int64_t n_entries, int64_t step,
                               int64_t* edges) {
  const char* fn = "svdq_cube_schedule";
  REQUIRE_PTR(table); REQUIRE_PTR(edges);
  if (n_entries < 1 || table[0] != 0)
    return fail(SVDQ_INVALID_ARG, "%s: the schedule must start at step 0", fn);
  if (step < 0) return fail(SVDQ_INVALID_ARG, "%s: step=%lld is negative", fn, (long long)step);
  int64_t pick = 0;
  for (int64_t i = 0; i < n_entries; ++i) {
    const int64_t* e = table + 4 * i;
    if (i > 0 && e[0] <= table[4 * (i - 1)])
      return fail(SVDQ_INVALID_ARG, "%s: first steps must increase (entry %lld)", fn,
                  (long long)i);
    if (e[1] < 1 || e[2] < 1 || e[3] < 1)
      return fail(SVDQ_INVALID_ARG, "%s: edges of entry %lld must be >= 1", fn, (long long)i);
    if (e[0] <= step) pick = i;
  }
  edges[0] = table[4 * pick + 1];
  edges[1] = table[4 * pick + 2];
  edges[2] = table[4 * pick + 3];
  return ok();
}

svdq_status svdq_cube_groups(const int32_t* cube_ptr, int64_t n_cubes, int32_t* group_ptr,
                             int64_t* n_groups) {
  const char* fn = "svdq_cube_groups";
  REQUIRE_PTR(cube_ptr); REQUIRE_PTR(n_groups);
  if (n_cubes < 1) return fail(SVDQ_INVALID_ARG, "%s: n_cubes must be >= 1", fn);
  if (cube_ptr[0] != 0) return fail(SVDQ_INVALID_ARG, "%s: cube_ptr[0] must be 0", fn);
  const int64_t g = svdq::cube_groups(cube_ptr, n_cubes, svdq::kDeltaGroupRows,
                                      svdq::kDeltaGroupCubes, nullptr);
  if (g < 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE,
                "%s: every cube must hold between 1 and %lld rows", fn,
                (long long)svdq::kDeltaGroupRows);
  *n_groups = g;
  if (group_ptr) svdq::cube_groups(cube_ptr, n_cubes, svdq::kDeltaGroupRows,
                                   svdq::kDeltaGroupCubes, group_ptr);
  return ok();
}

int64_t svdq_delta_workspace_bytes(int64_t n_cubes, int64_t K) {
  if (n_cubes < 1 || K < 1) return -1;
  return svdq::delta_workspace_bytes(n_cubes, K);
}

}  // extern "C"

namespace {

// Validation shared by the DeltaQuant activation entry points (workspace checked by the caller).
svdq_status check_delta(const char* fn, const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                        const float* act_amax, const int32_t* cube_ptr, const int32_t* cube_rows,
                        int64_t n_cubes, const int32_t* group_ptr, int64_t n_groups,
                        const uint16_t* lora_down, int64_t r, const uint8_t* core_codes,
                        const float* core_scale, const uint8_t* delta_codes,
                        const uint8_t* delta_scales, const float* g_delta, const float* D) {
  REQUIRE_PTR(X); REQUIRE_PTR(act_amax); REQUIRE_PTR(cube_ptr); REQUIRE_PTR(cube_rows);
  REQUIRE_PTR(group_ptr); REQUIRE_PTR(core_codes); REQUIRE_PTR(core_scale);
  REQUIRE_PTR(delta_codes); REQUIRE_PTR(delta_scales); REQUIRE_PTR(g_delta);
  REQUIRE_ALIGNED(X); REQUIRE_ALIGNED(core_codes); REQUIRE_ALIGNED(delta_codes);
  REQUIRE_ALIGNED(delta_scales); REQUIRE_ALIGNED(lora_down); REQUIRE_ALIGNED(D);
  if (M < 1 || M > INT32_MAX)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: M=%lld must lie in [1, 2^31)", fn, (long long)M);
  if (n_cubes < 1 || n_cubes > M) return fail(SVDQ_INVALID_ARG, "%s: bad n_cubes", fn);
  if (n_groups < 1 || n_groups > n_cubes)
    return fail(SVDQ_INVALID_ARG, "%s: n_groups=%lld must lie in [1, n_cubes]", fn,
                (long long)n_groups);
  TRY(check_k(fn, K));
  TRY(check_ld(fn, "ldx", ldx, K));
  TRY(check_rank(fn, r));
  if (r > 0) { REQUIRE_PTR(lora_down); REQUIRE_PTR(D); }
  return SVDQ_OK;
}

}  // namespace

extern "C" {

svdq_status svdq_delta_quant_act(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                 const float* lambda, const float* act_amax,
                                 const int32_t* cube_ptr, const int32_t* cube_rows,
                                 int64_t n_cubes, const int32_t* group_ptr, int64_t n_groups,
                                 const uint16_t* lora_down, int64_t r, uint8_t* core_codes,
                                 float* core_scale, uint8_t* delta_codes, uint8_t* delta_scales,
                                 float* g_delta, float* D, uint32_t* sat_count, void* workspace,
                                 int64_t workspace_bytes, svdq_stream_t stream) {
  const char* fn = "svdq_delta_quant_act";
  TRY(check_delta(fn, X, M, K, ldx, act_amax, cube_ptr, cube_rows, n_cubes, group_ptr, n_groups,
                  lora_down, r, core_codes, core_scale, delta_codes, delta_scales, g_delta, D));
  REQUIRE_PTR(workspace);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace must be 256-byte aligned", fn);
  const int64_t need = svdq::delta_workspace_bytes(n_cubes, K);
  if (workspace_bytes < need)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: workspace of %lld bytes, needs %lld", fn,
                (long long)workspace_bytes, (long long)need);
  return hip_result(svdq::launch_delta_quant_act(X, M, K, ldx, lambda, act_amax, cube_ptr,
                                                 cube_rows, group_ptr, n_groups, lora_down, r,
                                                 core_codes, core_scale, delta_codes,
                                                 delta_scales, g_delta, D, sat_count, workspace,
                                                 reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

svdq_status svdq_delta_quant_act_noalloc(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                         const float* lambda, const float* act_amax,
                                         const int32_t* cube_ptr, const int32_t* cube_rows,
                                         int64_t n_cubes, const int32_t* group_ptr,
                                         int64_t n_groups, const uint16_t* lora_down, int64_t r,
                                         uint8_t* core_codes, float* core_scale,
                                         uint8_t* delta_codes, uint8_t* delta_scales,
                                         float* g_delta, float* D, uint32_t* sat_count,
                                         svdq_stream_t stream) {
  const char* fn = "svdq_delta_quant_act_noalloc";
  TRY(check_delta(fn, X, M, K, ldx, act_amax, cube_ptr, cube_rows, n_cubes, group_ptr, n_groups,
                  lora_down, r, core_codes, core_scale, delta_codes, delta_scales, g_delta, D));
  const int64_t need = svdq::delta_workspace_bytes(n_cubes, K);
  if ((uint64_t)need > svdq::kDeltaScratchBytes)
    return fail(SVDQ_UNSUPPORTED_SHAPE,
                "%s: n_cubes=%lld x K=%lld needs %lld bytes of scratch, more than the %zu of the "
                "static buffer (use svdq_delta_quant_act with a workspace)",
                fn, (long long)n_cubes, (long long)K, (long long)need, svdq::kDeltaScratchBytes);
  void* scratch_ptr = nullptr;
  const hipError_t e = svdq::delta_scratch(&scratch_ptr);
  if (e != hipSuccess)
    return fail(SVDQ_HIP_ERROR, "%s: scratch address: %s", fn, hipGetErrorString(e));
  return hip_result(svdq::launch_delta_quant_act(X, M, K, ldx, lambda, act_amax, cube_ptr,
                                                 cube_rows, group_ptr, n_groups, lora_down, r,
                                                 core_codes, core_scale, delta_codes,
                                                 delta_scales, g_delta, D, sat_count, scratch_ptr,
                                                 reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

svdq_status svdq_gemm_core(int64_t n_cubes, int64_t N, int64_t K, const uint8_t* core_codes,
                           const float* core_scale, const uint8_t* w_codes,
                           const uint8_t* w_scales, const float* g_w, float* core_out,
                           svdq_stream_t stream) {
  const char* fn = "svdq_gemm_core";
  REQUIRE_PTR(core_codes); REQUIRE_PTR(core_scale); REQUIRE_PTR(w_codes); REQUIRE_PTR(w_scales);
  REQUIRE_PTR(g_w); REQUIRE_PTR(core_out);
  REQUIRE_ALIGNED(core_codes); REQUIRE_ALIGNED(w_codes);
  if (n_cubes < 1) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: n_cubes must be >= 1", fn);
  if (N < 1 || N % 256 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld must be a positive multiple of 256", fn,
                (long long)N);
  TRY(check_k(fn, K));
  return hip_result(svdq::launch_gemm_core(n_cubes, N, K, core_codes, core_scale, w_codes,
                                           w_scales, g_w, core_out,
                                           reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

svdq_status svdq_score_modal_rel_l2(const uint16_t* Y, int64_t ldy, const uint16_t* X,
                                    int64_t ldx, const uint16_t* W, int64_t ldw, int64_t M,
                                    int64_t N, int64_t K, const int32_t* rows,
                                    const int8_t* row_group, int64_t n_rows, double* sums,
                                    svdq_stream_t stream) {
  const char* fn = "svdq_score_modal_rel_l2";
  REQUIRE_PTR(Y); REQUIRE_PTR(X); REQUIRE_PTR(W); REQUIRE_PTR(rows); REQUIRE_PTR(row_group);
  REQUIRE_PTR(sums);
  REQUIRE_ALIGNED(X); REQUIRE_ALIGNED(W); REQUIRE_ALIGNED(Y);
  if (M < 1 || n_rows < 0) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: bad M or n_rows", fn);
  if (N < 1 || N % 256 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld must be a positive multiple of 256", fn,
                (long long)N);
  TRY(check_k(fn, K));
  TRY(check_ld(fn, "ldx", ldx, K));
  TRY(check_ld(fn, "ldw", ldw, K));
  if (ldy < N || ldy % 8 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: ldy must be >= N and a multiple of 8", fn);
  if (n_rows == 0) return ok();
  return hip_result(svdq::launch_score(Y, ldy, X, ldx, W, ldw, M, N, K, rows, row_group, n_rows,
                                       sums, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

svdq_status svdq_score_reference_rows(const uint16_t* X, int64_t ldx, const uint16_t* W,
                                      int64_t ldw, int64_t M, int64_t N, int64_t K,
                                      const int32_t* rows, int64_t n_rows, uint16_t* Yref,
                                      int64_t ldr, svdq_stream_t stream) {
  const char* fn = "svdq_score_reference_rows";
  REQUIRE_PTR(X); REQUIRE_PTR(W); REQUIRE_PTR(rows); REQUIRE_PTR(Yref);
  REQUIRE_ALIGNED(X); REQUIRE_ALIGNED(W); REQUIRE_ALIGNED(Yref);
  if (M < 1 || n_rows < 0) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: bad M or n_rows", fn);
  if (N < 1 || N % 256 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld must be a positive multiple of 256", fn,
                (long long)N);
  TRY(check_k(fn, K));
  TRY(check_ld(fn, "ldx", ldx, K));
  TRY(check_ld(fn, "ldw", ldw, K));
  if (ldr < N || ldr % 8 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: ldr must be >= N and a multiple of 8", fn);
  if (n_rows == 0) return ok();
  return hip_result(svdq::launch_reference_rows(X, ldx, W, ldw, M, N, K, rows, n_rows, Yref, ldr,
                                                reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

svdq_status svdq_score_modal_rel_l2_ref(const uint16_t* Y, int64_t ldy, const uint16_t* Yref,
                                        int64_t ldr, int64_t M, int64_t N, const int32_t* rows,
                                        const int8_t* row_group, int64_t n_rows, double* sums,
                                        svdq_stream_t stream) {
  const char* fn = "svdq_score_modal_rel_l2_ref";
  REQUIRE_PTR(Y); REQUIRE_PTR(Yref); REQUIRE_PTR(rows); REQUIRE_PTR(row_group);
  REQUIRE_PTR(sums);
  REQUIRE_ALIGNED(Y); REQUIRE_ALIGNED(Yref);
  if (M < 1 || n_rows < 0) return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: bad M or n_rows", fn);
  if (N < 1 || N % 8 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: N=%lld must be a positive multiple of 8", fn,
                (long long)N);
  if (ldy < N || ldy % 8 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: ldy must be >= N and a multiple of 8", fn);
  if (ldr < N || ldr % 8 != 0)
    return fail(SVDQ_UNSUPPORTED_SHAPE, "%s: ldr must be >= N and a multiple of 8", fn);
  if (n_rows == 0) return ok();
  return hip_result(svdq::launch_score_ref(Y, ldy, Yref, ldr, M, N, rows, row_group, n_rows, sums,
                                           reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
