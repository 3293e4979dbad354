// λ grid search against the layer's output error ("MiniMax-H3 NVFP4 — what the smoothing scale
// should be calibrated on", sections "Calibration" — a grid of candidate λ scored against the
// OutputsError objective — and "The metric that picks the winner also hides the cost" — that
// objective is the relative L2 of the layer's output against the bf16 layer over a uniform sample
// of all rows).  For each α of the grid, entirely on the device and in stream order:
//   λ_α from the calibration statistics; rank-r factors of diag(λ_α)·Wᵀ (randomized SVD);
//   residual weight quantisation; activation quantisation of the sampled rows (static amax of
//   λ_α) with the low-rank down-projection; the W4A4 GEMM; relative L2 against bf16(X·Wᵀ)
// then the first α of smallest error is selected and its λ copied out.
//
// Low-rank refit (the same page, section "Calibration", runs a number of refit iterations of the
// branch against the same objective for every candidate; it does not define them).  Reading: the
// alternating refit, where iterate t + 1 takes the rank-r factors of E_t = λ·W − deq(Q(R_t)),
// what the quantised residual of iterate t leaves of the smoothed weight, so that branch and
// quantised residual are fitted to each other; every iterate is scored like the first, and a
// candidate's score is the smallest over its iterates.  The factors of the best iterate of the
// winning candidate can be copied out.
//
// The per-candidate steps are the library's own launches; this file adds the row gather, the
// refit target and the bookkeeping.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

// Xs[i, :] = X[rows[i], :]  (16 bytes per thread; an index outside [0, M) reads the nearest row)
__global__ __launch_bounds__(256) void k_gather_rows(const uint16_t* __restrict__ X, int64_t M,
                                                     int64_t ldx, const int32_t* __restrict__ rows,
                                                     int64_t n_rows, int64_t K,
                                                     uint16_t* __restrict__ Xs) {
  const int64_t per_row = K / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_rows * per_row) return;
  const int64_t i = t / per_row, c = (t % per_row) * 8;
  int64_t m = rows[i];
  m = m < 0 ? 0 : (m < M ? m : M - 1);
  *reinterpret_cast<u32x4_t*>(Xs + i * K + c) =
      *reinterpret_cast<const u32x4_t*>(X + m * ldx + c);
}

// identity row list and one scoring group (3: the uniform rows) for the gathered rows
__global__ __launch_bounds__(256) void k_rows_setup(int64_t n_rows, int32_t* __restrict__ ids,
                                                    int8_t* __restrict__ grp) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n_rows) {
    ids[t] = (int32_t)t;
    grp[t] = 3;
  }
}

__global__ void k_zero_sums(double* __restrict__ sums) {
  if (threadIdx.x < 8) sums[threadIdx.x] = 0.0;
}

// sums[6] += Σ (Y − Y_ref)², sums[7] += Σ Y_ref² over n elements of bf16 Y and Y_ref (fp64,
// 8 elements per 16-byte load, one atomic pair per workgroup: atomics on one address serialise)
__global__ __launch_bounds__(256) void k_diff_sums(const uint16_t* __restrict__ Y,
                                                   const uint16_t* __restrict__ Yr, int64_t n,
                                                   double* __restrict__ sums) {
  __shared__ double red[2][4];
  double d2 = 0.0, r2 = 0.0;
  const int64_t n8 = n / 8;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n8; t += (int64_t)gridDim.x * 256) {
    const u32x4_t a = reinterpret_cast<const u32x4_t*>(Y)[t];
    const u32x4_t b = reinterpret_cast<const u32x4_t*>(Yr)[t];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double r0 = (double)bf16_lo(b[e]), r1 = (double)bf16_hi(b[e]);
      const double e0 = (double)bf16_lo(a[e]) - r0, e1 = (double)bf16_hi(a[e]) - r1;
      d2 += e0 * e0 + e1 * e1;
      r2 += r0 * r0 + r1 * r1;
    }
  }
  for (int64_t t = n8 * 8 + (int64_t)blockIdx.x * 256 + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * 256) {
    const double y = (double)bf16_to_f32(Y[t]), r = (double)bf16_to_f32(Yr[t]);
    const double d = y - r;
    d2 += d * d;
    r2 += r * r;
  }
  for (int off = 32; off > 0; off >>= 1) {
    d2 += __shfl_xor(d2, off);
    r2 += __shfl_xor(r2, off);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = d2;
    red[1][threadIdx.x >> 6] = r2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double d = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    const double r = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    if (d != 0.0) atomicAdd(sums + 6, d);
    if (r != 0.0) atomicAdd(sums + 7, r);
  }
}

__global__ void k_set_inf(double* __restrict__ v) {
  if (threadIdx.x == 0) *v = __builtin_huge_val();
}

// The score of iterate t of a candidate, sqrt(Σ(Y−Y_ref)²) / sqrt(ΣY_ref²) over group 3 (+inf
// when the reference is all zero), into cur and iter_score (when given); the candidate's score
// is the smallest over its iterates (a NaN is replaced by any later number).
__global__ void k_finish_iter(const double* __restrict__ sums, int t, double* __restrict__ score,
                              double* __restrict__ iter_score, double* __restrict__ cur) {
  if (threadIdx.x == 0) {
    const double d = sums[6], r = sums[7];
    const double v = r > 0.0 ? sqrt(d) / sqrt(r) : __builtin_huge_val();
    *cur = v;
    if (iter_score) *iter_score = v;
    const double old = *score;
    if (t == 0 || v < old || old != old) *score = v;
  }
}

// Factors of an iterate that beats every earlier iterate of every earlier candidate are copied
// out (strictly smaller: the first of equal scores is kept, as in the choice of α) ...
__global__ __launch_bounds__(256) void k_keep_factors(const double* __restrict__ cur,
                                                      const double* __restrict__ best,
                                                      const uint16_t* __restrict__ down,
                                                      const uint16_t* __restrict__ up,
                                                      int64_t n_down, int64_t n_up,
                                                      uint16_t* __restrict__ best_down,
                                                      uint16_t* __restrict__ best_up) {
  if (!(*cur < *best)) return;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n_down) best_down[t] = down[t];
  else if (t < n_down + n_up) best_up[t - n_down] = up[t - n_down];
}

// ... and the running best score follows once the copy has been made.
__global__ void k_commit_best(const double* __restrict__ cur, double* __restrict__ best) {
  if (threadIdx.x == 0 && *cur < *best) *best = *cur;
}

// Refit target of the low-rank branch: E = λ·W − deq(Q(R)), the smoothed weight less the
// dequantised residual, in fp64 (every term exact), rounded once to fp32.  One thread per 16
// consecutive channels of a row.  FMT: 0 NVFP4, 1 int4-g64, 2 MXFP4, 3 MXFP8.
template <int FMT>
__global__ __launch_bounds__(256) void k_refit_target(const uint16_t* __restrict__ W, int64_t N,
                                                      int64_t K, int64_t ldw,
                                                      const float* __restrict__ lambda,
                                                      const uint8_t* __restrict__ codes,
                                                      const void* __restrict__ scales,
                                                      const float* __restrict__ g,
                                                      float* __restrict__ E) {
  const int64_t per_row = K / 16;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N * per_row) return;
  const int64_t n = t / per_row, k0 = (t % per_row) * 16;
  double mult;
  if (FMT == 0) {
    mult = e4m3_value(static_cast<const uint8_t*>(scales)[n * (K / 16) + k0 / 16]) * (double)*g;
  } else if (FMT == 1) {
    const uint16_t h = static_cast<const uint16_t*>(scales)[n * (K / 64) + k0 / 64];
    mult = (double)(float)__builtin_bit_cast(_Float16, h);
  } else {
    mult = ldexp(1.0, (int)static_cast<const uint8_t*>(scales)[n * (K / 32) + k0 / 32] - 127);
  }
  uint8_t b[16];
  if (FMT == 3) {
    *reinterpret_cast<u32x4_t*>(b) = *reinterpret_cast<const u32x4_t*>(codes + n * K + k0);
  } else {
    const uint64_t q = *reinterpret_cast<const uint64_t*>(codes + n * (K / 2) + k0 / 2);
#pragma unroll
    for (int j = 0; j < 16; ++j) b[j] = (uint8_t)((q >> (4 * j)) & 0xFu);
  }
  const uint16_t* wr = W + n * ldw + k0;
  float* er = E + n * K + k0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    double v;
    if (FMT == 3) v = e4m3_value(b[j]);
    else if (FMT == 1) v = (double)((int)b[j] - (b[j] >= 8 ? 16 : 0));
    else v = e2m1_value(b[j]);
    er[j] = (float)((double)lambda[k0 + j] * (double)bf16_to_f32(wr[j]) - v * mult);
  }
}

// first index of the smallest score (NaN never wins); its λ copied to best_lambda
__global__ __launch_bounds__(256) void k_pick(const double* __restrict__ scores, int64_t n,
                                              const float* __restrict__ lam_all, int64_t K,
                                              float* __restrict__ best_lambda,
                                              int32_t* __restrict__ best_index) {
  __shared__ int64_t s_best;
  if (threadIdx.x == 0) {
    int64_t b = 0;
    for (int64_t i = 1; i < n; ++i)
      if (scores[i] < scores[b] || scores[b] != scores[b]) b = i;
    s_best = b;
    *best_index = (int32_t)b;
  }
  __syncthreads();
  for (int64_t k = threadIdx.x; k < K; k += 256) best_lambda[k] = lam_all[s_best * K + k];
}

int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t code_bytes(int fmt, int64_t rows, int64_t K) { return fmt == 3 ? rows * K : rows * K / 2; }
int64_t scale_bytes(int fmt, int64_t rows, int64_t K) {
  return fmt == 0 ? rows * K / 16 : fmt == 1 ? rows * (K / 64) * 2 : rows * K / 32;
}

struct SearchWs {
  float *lam_all, *amax, *g_w, *g_a, *D, *E;
  double *cur, *best;
  uint16_t *down, *up, *xs, *ys, *yref;
  uint8_t *w_codes, *w_scales, *a_codes, *a_scales;
  int32_t* ids;
  int8_t* grp;
  double* sums;
  void* lowrank;
  int64_t bytes;
};

SearchWs carve(void* base, int fmt, int64_t N, int64_t K, int64_t ell, int64_t r, int64_t S,
               int64_t n_alpha, int refit_iters) {
  uint8_t* b = static_cast<uint8_t*>(base);
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    void* p = b ? b + off : nullptr;
    off += align256(bytes > 0 ? bytes : 1);
    return p;
  };
  SearchWs w;
  w.lowrank = r > 0 ? take(lowrank_workspace_bytes(N, K, ell)) : nullptr;
  w.lam_all = static_cast<float*>(take(n_alpha * K * 4));
  w.amax = static_cast<float*>(take(n_alpha * 4));
  w.g_w = static_cast<float*>(take(4));
  w.g_a = static_cast<float*>(take(4));
  w.D = static_cast<float*>(take(S * (r > 0 ? r : 1) * 4));
  w.down = static_cast<uint16_t*>(take((r > 0 ? r : 1) * K * 2));
  w.up = static_cast<uint16_t*>(take(N * (r > 0 ? r : 1) * 2));
  w.xs = static_cast<uint16_t*>(take(S * K * 2));
  w.ys = static_cast<uint16_t*>(take(S * N * 2));
  w.yref = static_cast<uint16_t*>(take(S * N * 2));
  w.w_codes = static_cast<uint8_t*>(take(code_bytes(fmt, N, K)));
  w.w_scales = static_cast<uint8_t*>(take(scale_bytes(fmt, N, K)));
  w.a_codes = static_cast<uint8_t*>(take(code_bytes(fmt, S, K)));
  w.a_scales = static_cast<uint8_t*>(take(scale_bytes(fmt, S, K)));
  w.ids = static_cast<int32_t*>(take(S * 4));
  w.grp = static_cast<int8_t*>(take(S));
  w.sums = static_cast<double*>(take(8 * 8));
  w.cur = static_cast<double*>(take(8));
  w.best = static_cast<double*>(take(8));
  w.E = refit_iters > 0 ? static_cast<float*>(take(N * K * 4)) : nullptr;
  w.bytes = off;
  return w;
}

}  // namespace

int64_t lambda_search_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t ell, int64_t r,
                                      int64_t n_rows, int64_t n_alpha, int refit_iters) {
  return carve(nullptr, fmt, N, K, ell, r, n_rows, n_alpha, refit_iters).bytes;
}

hipError_t launch_lambda_search(const uint16_t* X, int64_t M, int64_t ldx, const uint16_t* W,
                                int64_t N, int64_t K, int64_t ldw, const float* ax,
                                const float* aw, uint32_t mask, const float* alphas,
                                int64_t n_alpha, int fmt, const float* omega, int64_t ell,
                                int64_t r, int power_iters, int refit_iters,
                                const int32_t* rows, int64_t n_rows, double* scores,
                                double* iter_scores, float* best_lambda, int32_t* best_index,
                                uint16_t* best_down, uint16_t* best_up, void* workspace,
                                hipStream_t s) {
  const SearchWs w = carve(workspace, fmt, N, K, ell, r, n_rows, n_alpha, refit_iters);
  hipError_t e;
#define SVDQ_TRY_HIP(x)                    \
  do {                                     \
    if ((e = (x)) != hipSuccess) return e; \
  } while (0)
  k_gather_rows<<<dim3((unsigned)ceil_div(n_rows * (K / 8), 256)), dim3(256), 0, s>>>(
      X, M, ldx, rows, n_rows, K, w.xs);
  SVDQ_TRY_HIP(hipGetLastError());
  k_rows_setup<<<dim3((unsigned)ceil_div(n_rows, 256)), dim3(256), 0, s>>>(n_rows, w.ids, w.grp);
  SVDQ_TRY_HIP(hipGetLastError());
  // the reference rows do not depend on the candidate: once
  SVDQ_TRY_HIP(launch_reference_rows(w.xs, K, W, ldw, n_rows, N, K, w.ids, n_rows, w.yref, N, s));
  const unsigned diff_blocks =
      (unsigned)(ceil_div(n_rows * N, 2048) < 256 ? ceil_div(n_rows * N, 2048) : 256);
  const bool keep = r > 0 && best_down != nullptr;
  if (keep) {
    k_set_inf<<<dim3(1), dim3(64), 0, s>>>(w.best);
    SVDQ_TRY_HIP(hipGetLastError());
  }
  const uint16_t* down = r > 0 ? w.down : nullptr;
  const uint16_t* up = r > 0 ? w.up : nullptr;
  float* D = r > 0 ? w.D : nullptr;
  float* g_w = fmt == 0 ? w.g_w : nullptr;
  const int64_t n_tgt = N * (K / 16);
  for (int64_t i = 0; i < n_alpha; ++i) {
    float* lam = w.lam_all + i * K;
    float* amax = w.amax + i;
    SVDQ_TRY_HIP(launch_lambda(ax, aw, K, mask, alphas[i], lam, amax, s));
    if (r > 0)
      SVDQ_TRY_HIP(launch_lowrank(W, N, K, ldw, lam, omega, ell, r, power_iters, w.down, w.up,
                                  nullptr, w.lowrank, s));
    for (int t = 0; t <= refit_iters; ++t) {
      SVDQ_TRY_HIP(launch_quantize_weight(fmt, W, N, K, ldw, lam, down, up, r, w.w_codes,
                                          w.w_scales, g_w, s));
      SVDQ_TRY_HIP(launch_quant_act(fmt, w.xs, n_rows, K, K, lam, fmt == 0 ? amax : nullptr,
                                    down, r, w.a_codes, w.a_scales, fmt == 0 ? w.g_a : nullptr,
                                    D, nullptr, s));
      SVDQ_TRY_HIP(launch_gemm(fmt, n_rows, N, K, w.a_codes, w.a_scales,
                               fmt == 0 ? w.g_a : nullptr, w.w_codes, w.w_scales, g_w, D, up, r,
                               nullptr, nullptr, w.ys, N, s));
      k_zero_sums<<<dim3(1), dim3(64), 0, s>>>(w.sums);
      SVDQ_TRY_HIP(hipGetLastError());
      k_diff_sums<<<dim3(diff_blocks), dim3(256), 0, s>>>(w.ys, w.yref, n_rows * N, w.sums);
      SVDQ_TRY_HIP(hipGetLastError());
      k_finish_iter<<<dim3(1), dim3(64), 0, s>>>(
          w.sums, t, scores + i,
          iter_scores ? iter_scores + i * (refit_iters + 1) + t : nullptr, w.cur);
      SVDQ_TRY_HIP(hipGetLastError());
      if (keep) {
        k_keep_factors<<<dim3((unsigned)ceil_div(r * K + N * r, 256)), dim3(256), 0, s>>>(
            w.cur, w.best, w.down, w.up, r * K, N * r, best_down, best_up);
        SVDQ_TRY_HIP(hipGetLastError());
        k_commit_best<<<dim3(1), dim3(64), 0, s>>>(w.cur, w.best);
        SVDQ_TRY_HIP(hipGetLastError());
      }
      if (t < refit_iters) {   // refit the branch to what the quantised residual leaves
        const dim3 grid((unsigned)ceil_div(n_tgt, 256));
        if (fmt == 0)
          k_refit_target<0><<<grid, dim3(256), 0, s>>>(W, N, K, ldw, lam, w.w_codes, w.w_scales,
                                                      g_w, w.E);
        else if (fmt == 1)
          k_refit_target<1><<<grid, dim3(256), 0, s>>>(W, N, K, ldw, lam, w.w_codes, w.w_scales,
                                                      g_w, w.E);
        else if (fmt == 2)
          k_refit_target<2><<<grid, dim3(256), 0, s>>>(W, N, K, ldw, lam, w.w_codes, w.w_scales,
                                                      g_w, w.E);
        else
          k_refit_target<3><<<grid, dim3(256), 0, s>>>(W, N, K, ldw, lam, w.w_codes, w.w_scales,
                                                      g_w, w.E);
        SVDQ_TRY_HIP(hipGetLastError());
        SVDQ_TRY_HIP(launch_lowrank_f32(w.E, N, K, K, omega, ell, r, power_iters, w.down, w.up,
                                        nullptr, w.lowrank, s));
      }
    }
  }
  k_pick<<<dim3(1), dim3(256), 0, s>>>(scores, n_alpha, w.lam_all, K, best_lambda, best_index);
  SVDQ_TRY_HIP(hipGetLastError());
#undef SVDQ_TRY_HIP
  return hipSuccess;
}

}  // namespace svdq
