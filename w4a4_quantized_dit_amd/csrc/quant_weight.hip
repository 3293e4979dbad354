// Weight preparation: residual R = diag(λ)·W − L1·L2 in fp64 (i ascending), rounded to fp32 and
// quantised to NVFP4 (dynamic tensor amax max|R32|) or int4-g64 ("MiniMax-H3 · SVDQuant W4A4
// (int4, rank 32, GPTQ)", opening paragraph: 16-bit low-rank branch plus a 4-bit residual).
//
// A block owns a tile of TR weight rows x 256 channels.  The tile's slice of lora_down
// [r, 256], its rows of lora_up [TR, r] and λ[256] are staged in LDS once and shared by all
// threads; each thread forms the fp64 residual of one quantisation block (16 elements for NVFP4,
// 64 for int4).  Every product up·down is exact in fp64, so each step is a fused multiply-add
// with a single rounding — the same value as subtract-after-multiply.  NVFP4 needs the tensor
// amax first: a persistent pass computes max|R32| (one atomic per block), then the quantising
// pass recomputes the residual instead of storing it.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 256;       // channels per tile

template <int BLK>
struct Tile {
  static constexpr int kBlocksPerRow = kCols / BLK;          // 16 (NVFP4) or 4 (int4)
  static constexpr int kRows = kThreads / kBlocksPerRow;     // 16 (NVFP4) or 64 (int4)
};

// Stage lora_down[:, c0:c0+256], lora_up[n0:n0+TR, :] and λ[c0:c0+256] into LDS.
template <int TR>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ down,
                                           const uint16_t* __restrict__ up,
                                           const float* __restrict__ lambda, int r, int64_t N,
                                           int64_t K, int64_t n0, int64_t c0, uint16_t* s_down,
                                           uint16_t* s_up, float* s_lam) {
  // down: r rows x 256 channels = r x 32 chunks of 16 B
  for (int c = threadIdx.x; c < r * (kCols / 8); c += kThreads) {
    const int i = c / (kCols / 8), part = c % (kCols / 8);
    reinterpret_cast<u32x4_t*>(s_down)[c] =
        *reinterpret_cast<const u32x4_t*>(down + (int64_t)i * K + c0 + part * 8);
  }
  for (int c = threadIdx.x; c < TR * r; c += kThreads) {
    const int64_t n = n0 + c / r;
    s_up[c] = n < N ? up[n * r + c % r] : (uint16_t)0;
  }
  for (int c = threadIdx.x; c < kCols; c += kThreads) s_lam[c] = lambda ? lambda[c0 + c] : 1.0f;
}

// fp64 residual of W[n, c0 + j0 .. + NE) with the staged tile; rounded to fp32.
template <int NE>
__device__ __forceinline__ void residual(const uint16_t* __restrict__ W, int64_t ldw, int64_t n,
                                         int64_t c0, int j0, int tr, int r,
                                         const uint16_t* s_down, const uint16_t* s_up,
                                         const float* s_lam, float* out) {
  double R[NE];
  const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(W + n * ldw + c0 + j0);
#pragma unroll
  for (int q = 0; q < NE / 8; ++q) {
    const u32x4_t w = wp[q];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      R[8 * q + 2 * c] = (double)s_lam[j0 + 8 * q + 2 * c] * (double)bf16_lo(w[c]);
      R[8 * q + 2 * c + 1] = (double)s_lam[j0 + 8 * q + 2 * c + 1] * (double)bf16_hi(w[c]);
    }
  }
  for (int i = 0; i < r; ++i) {
    const double u = -(double)bf16_to_f32(s_up[tr * r + i]);
    const u32x4_t* dp = reinterpret_cast<const u32x4_t*>(s_down + i * kCols + j0);
#pragma unroll
    for (int q = 0; q < NE / 8; ++q) {
      const u32x4_t d = dp[q];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        R[8 * q + 2 * c] = __builtin_fma(u, (double)bf16_lo(d[c]), R[8 * q + 2 * c]);
        R[8 * q + 2 * c + 1] = __builtin_fma(u, (double)bf16_hi(d[c]), R[8 * q + 2 * c + 1]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NE; ++j) out[j] = (float)R[j];
}

// MODE 0: max|R32| over the whole weight (persistent grid, one atomic per block)
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
  constexpr int BLK = MODE == 2 ? INT4_GROUP : NVFP4_BLOCK;
  constexpr int TR = Tile<BLK>::kRows;
  constexpr int BPR = Tile<BLK>::kBlocksPerRow;
  // dynamic LDS: lora_down slice [r][256] bf16 | λ [256] | lora_up rows [TR][r] bf16
  extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
  uint16_t* s_down = reinterpret_cast<uint16_t*>(s_dyn);
  float* s_lam = reinterpret_cast<float*>(s_dyn + (size_t)r * kCols * 2);
  uint16_t* s_up = reinterpret_cast<uint16_t*>(s_dyn + (size_t)r * kCols * 2 + kCols * 4);
  __shared__ float s_red[kThreads / 64];

  const int64_t tiles_n = (N + TR - 1) / TR, tiles_k = K / kCols;
  const int64_t ntiles = tiles_n * tiles_k;
  const int tr = threadIdx.x / BPR, jb = threadIdx.x % BPR;
  float g = 1.0f, d6 = 6.0f;
  if (MODE == 1) {
    const float a = amax_io[0];
    g = a == 0.0f ? 1.0f : a / 2688.0f;
    d6 = 6.0f * g;
  }
  float m = 0.0f;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t n0 = (tile / tiles_k) * TR, c0 = (tile % tiles_k) * kCols;
    const int rows = (int)min((int64_t)TR, N - n0);
    __syncthreads();  // the previous tile's LDS reads are done
    stage_tile<TR>(down, up, lambda, r, N, K, n0, c0, s_down, s_up, s_lam);
    __syncthreads();
    if (tr < rows) {
      const int64_t n = n0 + tr;
      float x[BLK];
      residual<BLK>(W, ldw, n, c0, jb * BLK, tr, r, s_down, s_up, s_lam, x);
      if (MODE == 0) {
#pragma unroll
        for (int j = 0; j < BLK; ++j) m = fmaxf(m, fabsf(x[j]));
      } else if (MODE == 1) {
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
        const int64_t k0 = c0 + jb * 16;
        *reinterpret_cast<uint2*>(codes + n * (K / 2) + k0 / 2) = packed;
        reinterpret_cast<uint8_t*>(scales)[n * (K / 16) + k0 / 16] = (uint8_t)sc;
      } else {
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
        const int64_t k0 = c0 + jb * 64;
        u32x4_t* cp = reinterpret_cast<u32x4_t*>(codes + n * (K / 2) + k0 / 2);
        cp[0] = u32x4_t{w[0], w[1], w[2], w[3]};
        cp[1] = u32x4_t{w[4], w[5], w[6], w[7]};
        reinterpret_cast<__half*>(scales)[n * (K / 64) + k0 / 64] = s;
      }
    }
  }
  if (MODE == 0) {
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float b = 0.0f;
      for (int i = 0; i < kThreads / 64; ++i) b = fmaxf(b, s_red[i]);
      if (b > 0.0f) atomic_max_pos(amax_io, b);
    }
  }
}

__global__ void k_amax_to_g(float* t) {
  const float a = t[0];
  t[0] = a == 0.0f ? 1.0f : a / 2688.0f;
}

__global__ void k_zero1(float* t) { t[0] = 0.0f; }

size_t lds_bytes(int64_t r, int tr) { return (size_t)r * kCols * 2 + kCols * 4 + (size_t)tr * r * 2; }

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
  if (fmt == 1) {
    constexpr int TR = Tile<INT4_GROUP>::kRows;
    const int64_t tiles = ((N + TR - 1) / TR) * (K / kCols);
    hipError_t e = allow_lds<2>(lds_bytes(r, TR));
    if (e != hipSuccess) return e;
    k_resid<2><<<dim3((unsigned)tiles), dim3(kThreads), lds_bytes(r, TR), s>>>(
        W, N, K, ldw, lambda, down, up, (int)r, nullptr, codes, scales);
    return hipGetLastError();
  }
  constexpr int TR = Tile<NVFP4_BLOCK>::kRows;
  const int64_t tiles = ((N + TR - 1) / TR) * (K / kCols);
  hipError_t e = allow_lds<0>(lds_bytes(r, TR));
  if (e == hipSuccess) e = allow_lds<1>(lds_bytes(r, TR));
  if (e != hipSuccess) return e;
  // tensor_scale holds max|R32| between the passes, then g = amax / 2688.
  k_zero1<<<1, 1, 0, s>>>(tensor_scale);
  const int64_t persistent = tiles < 1024 ? tiles : 1024;
  k_resid<0><<<dim3((unsigned)persistent), dim3(kThreads), lds_bytes(r, TR), s>>>(
      W, N, K, ldw, lambda, down, up, (int)r, tensor_scale, nullptr, nullptr);
  k_resid<1><<<dim3((unsigned)tiles), dim3(kThreads), lds_bytes(r, TR), s>>>(
      W, N, K, ldw, lambda, down, up, (int)r, tensor_scale, codes, scales);
  k_amax_to_g<<<1, 1, 0, s>>>(tensor_scale);
  return hipGetLastError();
}

}  // namespace svdq
