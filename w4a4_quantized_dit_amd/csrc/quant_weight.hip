// Weight preparation: residual R = diag(λ)·W − L1·L2 in fp64 (i ascending), rounded to fp32 and
// quantised to NVFP4 (dynamic tensor amax max|R32|) or int4-g64 ("MiniMax-H3 · SVDQuant W4A4
// (int4, rank 32, GPTQ)", opening paragraph: 16-bit low-rank branch plus a 4-bit residual).
//
// A block owns a tile of 128 weight rows x 128 channels; a thread owns 4 rows x one 16-channel
// block.  The tile's slice of lora_down [r, 128] is staged in LDS as fp32 (exact), the rows of
// lora_up transposed to [r, 128] bf16, and λ as fp32.  For each rank i in ascending order a
// thread converts its 16 lora_down values to fp64 once and applies them to its 4 rows:
// R[n, k] ← fma(−up[n, i], down[i, k], R[n, k]) starting from λ_k·W[n, k] (exact in fp64).
// Every up·down product is exact in fp64, so each fused multiply-add rounds once, exactly as a
// subtract after the multiply.  NVFP4 blocks are quantised from registers; an int4 group of 64
// spans four lanes, which combine their absmax with two shuffles.  NVFP4 needs the tensor amax
// first: a pass computes max|R32| (one atomic per block), then the quantising pass recomputes
// the residual instead of storing it.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 128;       // weight rows per tile
constexpr int kTileCols = 128;       // channels per tile
constexpr int kRowsPerThread = 4;    // rows of one thread (a 16-channel block each)

// MODE 0: max|R32| over the whole weight (one atomic per block)
// MODE 1: NVFP4 codes and scales with g = amax / 2688
// MODE 2: int4-g64 codes and fp16 scales
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_resid(const uint16_t* __restrict__ W, int64_t N,
                                                    int64_t K, int64_t ldw,
                                                    const float* __restrict__ lambda,
                                                    const uint16_t* __restrict__ down,
                                                    const uint16_t* __restrict__ up, int r,
                                                    float* __restrict__ amax_io,
                                                    uint8_t* __restrict__ codes,
                                                    void* __restrict__ scales) {
  // dynamic LDS: lora_down slice fp32 [r][128] | lora_up transposed bf16 [r][128] | λ [128]
  extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
  float* s_down = reinterpret_cast<float*>(s_dyn);
  uint16_t* s_upT = reinterpret_cast<uint16_t*>(s_dyn + (size_t)r * kTileCols * 4);
  float* s_lam = reinterpret_cast<float*>(s_dyn + (size_t)r * kTileCols * 6);
  __shared__ float s_red[kThreads / 64];

  const int tid = threadIdx.x;
  const int64_t tiles_k = K / kTileCols;
  const int64_t n0 = (int64_t)(blockIdx.x / tiles_k) * kTileRows;
  const int64_t c0 = (int64_t)(blockIdx.x % tiles_k) * kTileCols;
  const int cb = tid & 7, rg = tid >> 3;  // 16-channel block, group of 4 rows

  // stage lora_down[:, c0:c0+128] as fp32: piece p = rank p / 16, channels 8·(p % 16) .. +8
  for (int p = tid; p < r * (kTileCols / 8); p += kThreads) {
    const int i = p >> 4, part = p & 15;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(down + (int64_t)i * K + c0 + 8 * part);
    float* dst = s_down + i * kTileCols + 8 * part;
    *reinterpret_cast<f32x4_t*>(dst) =
        f32x4_t{bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1])};
    *reinterpret_cast<f32x4_t*>(dst + 4) =
        f32x4_t{bf16_lo(v[2]), bf16_hi(v[2]), bf16_lo(v[3]), bf16_hi(v[3])};
  }
  // stage lora_up[n0:n0+128, :] transposed: element (row, i) -> s_upT[i][row] (rows past N: 0)
  for (int e = tid; e < kTileRows * r; e += kThreads) {
    const int row = e / r, i = e % r;
    const int64_t n = n0 + row;
    s_upT[i * kTileRows + row] = n < N ? up[n * r + i] : (uint16_t)0;
  }
  if (tid < kTileCols) s_lam[tid] = lambda ? lambda[c0 + tid] : 1.0f;
  __syncthreads();

  // initial values λ_k·W[n, k] (exact in fp64); rows past N read row N-1 and are never used
  double R[kRowsPerThread][16];
  const int64_t kc = c0 + 16 * cb;
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    int64_t n = n0 + kRowsPerThread * rg + j;
    n = n < N ? n : N - 1;
    const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(W + n * ldw + kc);
    const u32x4_t w0 = wp[0], w1 = wp[1];
    const uint32_t w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      R[j][2 * e] = (double)s_lam[16 * cb + 2 * e] * (double)bf16_lo(w[e]);
      R[j][2 * e + 1] = (double)s_lam[16 * cb + 2 * e + 1] * (double)bf16_hi(w[e]);
    }
  }
  // R ← R − up·down, rank by rank in ascending order
  for (int i = 0; i < r; ++i) {
    const f32x4_t* dp = reinterpret_cast<const f32x4_t*>(s_down + i * kTileCols + 16 * cb);
    double d[16];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const f32x4_t v = dp[e4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d[4 * e4 + e] = (double)v[e];
    }
    const uint2 uw = *reinterpret_cast<const uint2*>(s_upT + i * kTileRows + kRowsPerThread * rg);
    const double u[4] = {-(double)bf16_lo(uw.x), -(double)bf16_hi(uw.x), -(double)bf16_lo(uw.y),
                         -(double)bf16_hi(uw.y)};
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) R[j][e] = __builtin_fma(u[j], d[e], R[j][e]);
  }

  if (MODE == 0) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      if (n0 + kRowsPerThread * rg + j < N) {
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf((float)R[j][e]));
      }
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) s_red[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) {
      float b = 0.0f;
      for (int w = 0; w < kThreads / 64; ++w) b = fmaxf(b, s_red[w]);
      if (b > 0.0f) atomic_max_pos(amax_io, b);
    }
  } else if (MODE == 1) {
    const float amax = amax_io[0];
    const float g = amax == 0.0f ? 1.0f : amax / 2688.0f;
    const float d6 = 6.0f * g;
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      const int64_t n = n0 + kRowsPerThread * rg + j;
      float x[16];
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[e] = (float)R[j][e];
        a = fmaxf(a, fabsf(x[e]));
      }
      float inv;
      const uint32_t sc = nvfp4_block_scale(a, g, d6, &inv);
      float y[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] = x[e] * inv;
      if (n < N) {
        *reinterpret_cast<uint2*>(codes + n * (K / 2) + kc / 2) =
            uint2{e2m1_pack8(y), e2m1_pack8(y + 8)};
        reinterpret_cast<uint8_t*>(scales)[n * (K / 16) + kc / 16] = (uint8_t)sc;
      }
    }
  } else {
    // int4-g64: the group's four 16-channel blocks are held by lanes cb = 4g .. 4g+3
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      const int64_t n = n0 + kRowsPerThread * rg + j;
      float x[16];
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[e] = (float)R[j][e];
        a = fmaxf(a, fabsf(x[e]));
      }
      a = fmaxf(a, __shfl_xor(a, 1));
      a = fmaxf(a, __shfl_xor(a, 2));
      const __half s = __float2half_rn(a / 7.0f);
      const float sf = __half2float(s);
      const float inv = sf != 0.0f ? 1.0f / sf : 0.0f;
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        w0 |= int4_code(x[e] * inv) << (4 * e);
        w1 |= int4_code(x[8 + e] * inv) << (4 * e);
      }
      if (n < N) {
        *reinterpret_cast<uint2*>(codes + n * (K / 2) + kc / 2) = uint2{w0, w1};
        if ((cb & 3) == 0) reinterpret_cast<__half*>(scales)[n * (K / 64) + kc / 64] = s;
      }
    }
  }
}

__global__ void k_amax_to_g(float* t) {
  const float a = t[0];
  t[0] = a == 0.0f ? 1.0f : a / 2688.0f;
}

__global__ void k_zero1(float* t) { t[0] = 0.0f; }

size_t lds_bytes(int64_t r) { return (size_t)r * kTileCols * 6 + kTileCols * 4; }

template <int MODE>
hipError_t allow_lds(size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_resid<MODE>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

hipError_t launch_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                  const float* lambda, const uint16_t* down, const uint16_t* up,
                                  int64_t r, uint8_t* codes, void* scales, float* tensor_scale,
                                  hipStream_t s) {
  const int64_t tiles = ((N + kTileRows - 1) / kTileRows) * (K / kTileCols);
  const size_t lds = lds_bytes(r);
  if (fmt == 1) {
    hipError_t e = allow_lds<2>(lds);
    if (e != hipSuccess) return e;
    k_resid<2><<<dim3((unsigned)tiles), dim3(kThreads), lds, s>>>(W, N, K, ldw, lambda, down, up,
                                                                 (int)r, nullptr, codes, scales);
    return hipGetLastError();
  }
  hipError_t e = allow_lds<0>(lds);
  if (e == hipSuccess) e = allow_lds<1>(lds);
  if (e != hipSuccess) return e;
  // tensor_scale holds max|R32| between the passes, then g = amax / 2688.
  k_zero1<<<1, 1, 0, s>>>(tensor_scale);
  k_resid<0><<<dim3((unsigned)tiles), dim3(kThreads), lds, s>>>(W, N, K, ldw, lambda, down, up,
                                                               (int)r, tensor_scale, nullptr,
                                                               nullptr);
  k_resid<1><<<dim3((unsigned)tiles), dim3(kThreads), lds, s>>>(W, N, K, ldw, lambda, down, up,
                                                               (int)r, tensor_scale, codes, scales);
  k_amax_to_g<<<1, 1, 0, s>>>(tensor_scale);
  return hipGetLastError();
}

}  // namespace svdq
