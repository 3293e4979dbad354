// Weight preparation: residual R = diag(λ)·W − L1·L2 in fp64 (i ascending), rounded to fp32 and
// quantised to NVFP4 (dynamic tensor amax max|R32|) or int4-g64 ("MiniMax-H3 · SVDQuant W4A4
// (int4, rank 32, GPTQ)", opening paragraph: 16-bit low-rank branch plus a 4-bit residual).
// Offline step; the residual is recomputed in the quantisation pass instead of being stored.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;

// R32 for the 16 elements W[n, k0 .. k0+16).
__device__ __forceinline__ void residual16(const uint16_t* __restrict__ W, int64_t ldw,
                                           const float* __restrict__ lambda,
                                           const uint16_t* __restrict__ down,
                                           const uint16_t* __restrict__ up, int r, int64_t K,
                                           int64_t n, int64_t k0, float* out) {
  double R[16];
  const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(W + n * ldw + k0);
  u32x4_t w0 = wp[0], w1 = wp[1];
  uint32_t wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float l0 = lambda ? lambda[k0 + 2 * j] : 1.0f;
    const float l1 = lambda ? lambda[k0 + 2 * j + 1] : 1.0f;
    R[2 * j] = (double)l0 * (double)bf16_lo(wv[j]);
    R[2 * j + 1] = (double)l1 * (double)bf16_hi(wv[j]);
  }
  for (int i = 0; i < r; ++i) {
    const uint16_t* upn = up + n * (int64_t)r;
    const double u = (double)bf16_to_f32(upn[i]);
    const u32x4_t* dp = reinterpret_cast<const u32x4_t*>(down + (int64_t)i * K + k0);
    u32x4_t d0 = dp[0], d1 = dp[1];
    uint32_t dv[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      R[2 * j] -= u * (double)bf16_lo(dv[j]);      // product exact in fp64; one rounding
      R[2 * j + 1] -= u * (double)bf16_hi(dv[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) out[j] = (float)R[j];
}

__global__ __launch_bounds__(kThreads) void k_resid_amax(const uint16_t* __restrict__ W,
                                                         int64_t N, int64_t K, int64_t ldw,
                                                         const float* __restrict__ lambda,
                                                         const uint16_t* __restrict__ down,
                                                         const uint16_t* __restrict__ up, int r,
                                                         float* __restrict__ amax) {
  const int64_t nb = K / NVFP4_BLOCK;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  float m = 0.0f;
  if (id < N * nb) {
    const int64_t n = id / nb, k0 = (id % nb) * NVFP4_BLOCK;
    float x[16];
    residual16(W, ldw, lambda, down, up, r, K, n, k0, x);
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(x[j]));
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0 && m > 0.0f) atomic_max_pos(amax, m);
}

__global__ __launch_bounds__(kThreads) void k_resid_nvfp4(
    const uint16_t* __restrict__ W, int64_t N, int64_t K, int64_t ldw,
    const float* __restrict__ lambda, const uint16_t* __restrict__ down,
    const uint16_t* __restrict__ up, int r, const float* __restrict__ amax_p,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nb = K / NVFP4_BLOCK;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= N * nb) return;
  const int64_t n = id / nb, b = id % nb, k0 = b * NVFP4_BLOCK;
  const float amax = amax_p[0];
  const float g = amax == 0.0f ? 1.0f : amax / 2688.0f;
  const float d6 = 6.0f * g;
  float x[16];
  residual16(W, ldw, lambda, down, up, r, K, n, k0, x);
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(x[j]));
  float inv;
  const uint32_t sc = nvfp4_block_scale(a, g, d6, &inv);
  float y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) y[j] = x[j] * inv;
  uint2 packed;
  packed.x = e2m1_pack8(y);
  packed.y = e2m1_pack8(y + 8);
  *reinterpret_cast<uint2*>(codes + n * (K / 2) + k0 / 2) = packed;
  scales[n * nb + b] = (uint8_t)sc;
}

__global__ __launch_bounds__(kThreads) void k_resid_int4(
    const uint16_t* __restrict__ W, int64_t N, int64_t K, int64_t ldw,
    const float* __restrict__ lambda, const uint16_t* __restrict__ down,
    const uint16_t* __restrict__ up, int r, uint8_t* __restrict__ codes,
    __half* __restrict__ scales) {
  const int64_t ng = K / INT4_GROUP;
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= N * ng) return;
  const int64_t n = id / ng, gi = id % ng, k0 = gi * INT4_GROUP;
  float x[64];
#pragma unroll
  for (int q = 0; q < 4; ++q) residual16(W, ldw, lambda, down, up, r, K, n, k0 + 16 * q, x + 16 * q);
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 64; ++j) a = fmaxf(a, fabsf(x[j]));
  const __half s = __float2half_rn(a / 7.0f);
  const float sf = __half2float(s);
  const float inv = sf != 0.0f ? 1.0f / sf : 0.0f;
  uint32_t w[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) v |= int4_code(x[8 * d + j] * inv) << (4 * j);
    w[d] = v;
  }
  u32x4_t* cp = reinterpret_cast<u32x4_t*>(codes + n * (K / 2) + k0 / 2);
  cp[0] = u32x4_t{w[0], w[1], w[2], w[3]};
  cp[1] = u32x4_t{w[4], w[5], w[6], w[7]};
  scales[n * ng + gi] = s;
}

__global__ void k_amax_to_g(float* t) {
  const float a = t[0];
  t[0] = a == 0.0f ? 1.0f : a / 2688.0f;
}

__global__ void k_zero1(float* t) { t[0] = 0.0f; }

}  // namespace

hipError_t launch_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                  const float* lambda, const uint16_t* down, const uint16_t* up,
                                  int64_t r, uint8_t* codes, void* scales, float* tensor_scale,
                                  hipStream_t s) {
  if (fmt == 1) {
    const int64_t n = N * (K / INT4_GROUP);
    k_resid_int4<<<dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(
        W, N, K, ldw, lambda, down, up, (int)r, codes, reinterpret_cast<__half*>(scales));
    return hipGetLastError();
  }
  const int64_t n = N * (K / NVFP4_BLOCK);
  const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
  // tensor_scale holds max|R32| between the passes, then g = amax / 2688.
  k_zero1<<<1, 1, 0, s>>>(tensor_scale);
  k_resid_amax<<<grid, dim3(kThreads), 0, s>>>(W, N, K, ldw, lambda, down, up, (int)r,
                                                tensor_scale);
  k_resid_nvfp4<<<grid, dim3(kThreads), 0, s>>>(W, N, K, ldw, lambda, down, up, (int)r,
                                                 tensor_scale, codes,
                                                 reinterpret_cast<uint8_t*>(scales));
  k_amax_to_g<<<1, 1, 0, s>>>(tensor_scale);
  return hipGetLastError();
}

}  // namespace svdq
