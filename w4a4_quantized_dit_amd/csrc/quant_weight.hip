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
// the residual instead of storing it; with a caller workspace the residual pass stores R32 with
// its maximum and k_quant_r32 quantises the stored values instead.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 128;  // weight rows per tile
constexpr int kTileCols = 128;  // channels per tile
constexpr int kRankChunk = 32;  // ranks staged in LDS at a time

typedef __attribute__((ext_vector_type(2))) double f64x2_t;

// MODE 0: max|R32| over the whole weight (one atomic per block)
// MODE 1: NVFP4 codes and scales with g = amax / 2688
// MODE 2: int4-g64 codes and fp16 scales
// MODE 3 / 4: MX codes (E2M1 / E4M3) with E8M0 scales per 32 (single pass)
// MODE 5: R32 itself (fp32 [N, K], through `codes`), and max|R32| when amax_io is given
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_resid(const uint16_t* __restrict__ W, int64_t N,
                                                    int64_t K, int64_t ldw,
                                                    const float* __restrict__ lambda,
                                                    const uint16_t* __restrict__ down,
                                                    const uint16_t* __restrict__ up, int r,
                                                    float* __restrict__ amax_io,
                                                    uint8_t* __restrict__ codes,
                                                    void* __restrict__ scales) {
  // dynamic LDS: down fp64 [chunk][128] (pieces rotated) | -up fp64 [chunk][128] | lambda [128]
  extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
  double* s_down = reinterpret_cast<double*>(s_dyn);
  double* s_up = reinterpret_cast<double*>(s_dyn + kRankChunk * kTileCols * 8);
  float* s_lam = reinterpret_cast<float*>(s_dyn + 2 * kRankChunk * kTileCols * 8);
  __shared__ float s_red[kThreads / 64];

  const int tid = threadIdx.x;
  const int64_t tiles_k = K / kTileCols;
  const int64_t n0 = (int64_t)(blockIdx.x / tiles_k) * kTileRows;
  const int64_t c0 = (int64_t)(blockIdx.x % tiles_k) * kTileCols;
  const int cb = tid & 15, rg = tid >> 4;  // channels 8 cb .. 8 cb + 7, rows 8 rg .. 8 rg + 7

  // A rank chunk is staged from 16-byte pieces, two per thread per factor: down piece p = rank
  // p / 16, channels 8 (p % 16) .. +8; up piece p = row p % 128, ranks 8 (p / 128) .. +8.
  // The pieces of the next chunk are loaded into registers while the current one is applied.
  auto load_chunk = [&](int i0, int rc, u32x4_t (&pd)[2], u32x4_t (&pu)[2]) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = tid + kThreads * k;
      pd[k] = u32x4_t{0u, 0u, 0u, 0u};
      pu[k] = u32x4_t{0u, 0u, 0u, 0u};
      if (p < rc * 16)
        pd[k] = *reinterpret_cast<const u32x4_t*>(down + (int64_t)(i0 + p / 16) * K + c0 +
                                                  8 * (p % 16));
      const int row = p % kTileRows, k8 = p / kTileRows;
      if (8 * k8 < rc && n0 + row < N)
        pu[k] = *reinterpret_cast<const u32x4_t*>(up + (n0 + row) * r + i0 + 8 * k8);
    }
  };
  auto store_chunk = [&](int rc, const u32x4_t (&pd)[2], const u32x4_t (&pu)[2]) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = tid + kThreads * k;
      if (p < rc * 16) {
        const int i = p / 16, g = p % 16;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f64x2_t*>(s_down + i * kTileCols + g * 8 + ((q + (g >> 2)) & 3) * 2) =
              f64x2_t{(double)bf16_lo(pd[k][q]), (double)bf16_hi(pd[k][q])};
      }
      const int row = p % kTileRows, k8 = p / kTileRows;
      if (8 * k8 < rc) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s_up[(8 * k8 + 2 * q) * kTileRows + row] = -(double)bf16_lo(pu[k][q]);
          s_up[(8 * k8 + 2 * q + 1) * kTileRows + row] = -(double)bf16_hi(pu[k][q]);
        }
      }
    }
  };

  // W tile and the first chunk in flight together; lambda; then the initial values
  // lambda_k W[n, k] (exact in fp64).  Rows past N read row N-1 and are never stored.
  const int64_t kc = c0 + 8 * cb;
  u32x4_t wt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int64_t n = n0 + 8 * rg + j;
    n = n < N ? n : N - 1;
    wt[j] = *reinterpret_cast<const u32x4_t*>(W + n * ldw + kc);
  }
  u32x4_t pd[2], pu[2];
  int rc = r < kRankChunk ? r : kRankChunk;
  if (r > 0) load_chunk(0, rc, pd, pu);
  if (tid < kTileCols) s_lam[tid] = lambda ? lambda[c0 + tid] : 1.0f;
  if (r > 0) store_chunk(rc, pd, pu);
  __syncthreads();
  double R[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      R[j][2 * e] = (double)s_lam[8 * cb + 2 * e] * (double)bf16_lo(wt[j][e]);
      R[j][2 * e + 1] = (double)s_lam[8 * cb + 2 * e + 1] * (double)bf16_hi(wt[j][e]);
    }
  }

  // R <- R - up·down, rank by rank in ascending order.  The thread's 16-byte piece q of a
  // staged down row sits at piece (q + cb / 4) % 4 of its 64 bytes.
  const int rot = cb >> 2;
  for (int i0 = 0; i0 < r; i0 += kRankChunk) {
    const int next = i0 + kRankChunk;
    const int rn = r - next < kRankChunk ? r - next : kRankChunk;
    if (next < r) load_chunk(next, rn, pd, pu);
#pragma unroll 4
    for (int i = 0; i < rc; ++i) {  // unrolled: the next ranks' LDS reads overlap these FMAs
      const double* dp = s_down + i * kTileCols + cb * 8;
      const double* upp = s_up + i * kTileRows + rg * 8;
      double d[8], u[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f64x2_t v = *reinterpret_cast<const f64x2_t*>(dp + ((q + rot) & 3) * 2);
        d[2 * q] = v[0];
        d[2 * q + 1] = v[1];
        const f64x2_t w = *reinterpret_cast<const f64x2_t*>(upp + 2 * q);
        u[2 * q] = w[0];
        u[2 * q + 1] = w[1];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) R[j][e] = __builtin_fma(u[j], d[e], R[j][e]);
    }
    if (next < r) {
      __syncthreads();  // every thread is done with this chunk
      store_chunk(rn, pd, pu);
      __syncthreads();
      rc = rn;
    }
  }

  if (MODE == 0 || MODE == 5) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + 8 * rg + j;
      if (n < N) {
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)R[j][e]));
        if (MODE == 5) {
          float* dst = reinterpret_cast<float*>(codes) + n * K + kc;
          reinterpret_cast<f32x4_t*>(dst)[0] =
              f32x4_t{(float)R[j][0], (float)R[j][1], (float)R[j][2], (float)R[j][3]};
          reinterpret_cast<f32x4_t*>(dst)[1] =
              f32x4_t{(float)R[j][4], (float)R[j][5], (float)R[j][6], (float)R[j][7]};
        }
      }
    }
    if (amax_io) {
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      if ((tid & 63) == 0) s_red[tid >> 6] = m;
      __syncthreads();
      if (tid == 0) {
        float b = 0.0f;
        for (int w = 0; w < kThreads / 64; ++w) b = fmaxf(b, s_red[w]);
        if (b > 0.0f) atomic_max_pos(amax_io, b);
      }
    }
  } else if (MODE == 1) {
    // an NVFP4 block of 16 channels is held by lanes cb = 2b, 2b + 1
    const float amax = amax_io[0];
    const float g = amax == 0.0f ? 1.0f : amax / 2688.0f;
    const float d6 = 6.0f * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + 8 * rg + j;
      float x[8];
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = (float)R[j][e];
        a = fmaxf(a, fabsf(x[e]));
      }
      a = fmaxf(a, __shfl_xor(a, 1));
      float inv;
      const uint32_t sc = nvfp4_block_scale(a, g, d6, &inv);
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[e] * inv;
      if (n < N) {
        *reinterpret_cast<uint32_t*>(codes + n * (K / 2) + kc / 2) = e2m1_pack8(y);
        if ((cb & 1) == 0) reinterpret_cast<uint8_t*>(scales)[n * (K / 16) + kc / 16] = (uint8_t)sc;
      }
    }
  } else if (MODE == 3 || MODE == 4) {
    // an MX block of 32 channels is held by lanes cb = 4b .. 4b + 3: E8M0 exponent from the
    // block maximum, codes of x · 2^-e, E2M1 (MODE 3) or E4M3 (MODE 4)
    constexpr int kEmax = MODE == 3 ? 2 : 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + 8 * rg + j;
      float x[8];
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = (float)R[j][e];
        a = fmaxf(a, fabsf(x[e]));
      }
      a = fmaxf(a, __shfl_xor(a, 1));
      a = fmaxf(a, __shfl_xor(a, 2));
      const int ex = mx_exponent(a, kEmax);
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = __builtin_ldexpf(x[e], -ex);
      if (n < N) {
        if (MODE == 3) {
          *reinterpret_cast<uint32_t*>(codes + n * (K / 2) + kc / 2) = e2m1_pack8(y);
        } else {
          const uint32_t w0 = e4m3_pack4(y[0], y[1], y[2], y[3]);
          const uint32_t w1 = e4m3_pack4(y[4], y[5], y[6], y[7]);
          *reinterpret_cast<uint2*>(codes + n * K + kc) = uint2{w0, w1};
        }
        if ((cb & 3) == 0) reinterpret_cast<uint8_t*>(scales)[n * (K / 32) + kc / 32] = (uint8_t)(ex + 127);
      }
    }
  } else {
    // an int4-g64 group is held by lanes cb = 8g .. 8g + 7
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + 8 * rg + j;
      float x[8];
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = (float)R[j][e];
        a = fmaxf(a, fabsf(x[e]));
      }
      a = fmaxf(a, __shfl_xor(a, 1));
      a = fmaxf(a, __shfl_xor(a, 2));
      a = fmaxf(a, __shfl_xor(a, 4));
      const __half s = __float2half_rn(a / 7.0f);
      const float sf = __half2float(s);
      const float inv = sf != 0.0f ? 1.0f / sf : 0.0f;
      uint32_t w0 = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) w0 |= int4_code(x[e] * inv) << (4 * e);
      if (n < N) {
        *reinterpret_cast<uint32_t*>(codes + n * (K / 2) + kc / 2) = w0;
        if ((cb & 7) == 0) reinterpret_cast<__half*>(scales)[n * (K / 64) + kc / 64] = s;
      }
    }
  }
}

// NVFP4 codes and scales of R32 [N, K] (fp32, from the residual pass) with the tensor amax in
// amax_p, the arithmetic of the quantising residual pass (MODE 1) on the same fp32 values.  R32
// is read in 1 KB pieces, lane l of a wave holding bytes [16 l, 16 l + 16) of a piece, so every
// load instruction covers 8 whole cache lines (one thread per 64-byte block made each
// instruction touch 32 lines, every line four times).  Four lanes hold one 16-block: their
// maxima combine with two lane exchanges, each computes the block scale, and lane l writes the
// two code bytes of its four values (128 contiguous bytes per piece) and lane 4b the scale byte
// of block b.  A wave takes kPieces consecutive pieces per round.
constexpr int kPieces = 4;
__global__ __launch_bounds__(256) void k_quant_r32(const float* __restrict__ R32, int64_t npiece,
                                                   const float* __restrict__ amax_p,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales) {
  const float amax = amax_p[0];
  const float g = amax == 0.0f ? 1.0f : amax / 2688.0f;
  const float d6 = 6.0f * g;
  const int lane = threadIdx.x & 63;
  const int64_t nwave = (int64_t)gridDim.x * 4;
  for (int64_t p0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kPieces; p0 < npiece;
       p0 += nwave * kPieces) {
    f32x4_t x[kPieces];
#pragma unroll
    for (int u = 0; u < kPieces; ++u)
      if (p0 + u < npiece)
        x[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(R32 + (p0 + u) * 256) + lane);
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      if (p0 + u >= npiece) break;
      float a = fmaxf(fmaxf(fabsf(x[u][0]), fabsf(x[u][1])), fmaxf(fabsf(x[u][2]), fabsf(x[u][3])));
      a = fmaxf(a, __shfl_xor(a, 1));
      a = fmaxf(a, __shfl_xor(a, 2));
      float inv;
      const uint32_t sc = nvfp4_block_scale(a, g, d6, &inv);
      uint32_t w = e2m1_pack2<0>(0u, x[u][0] * inv, x[u][1] * inv);
      w = e2m1_pack2<1>(w, x[u][2] * inv, x[u][3] * inv);
      *reinterpret_cast<uint16_t*>(codes + (p0 + u) * 128 + 2 * lane) = (uint16_t)w;
      if ((lane & 3) == 0) scales[(p0 + u) * 16 + (lane >> 2)] = (uint8_t)sc;
    }
  }
}

__global__ void k_amax_to_g(float* t) {
  const float a = t[0];
  t[0] = a == 0.0f ? 1.0f : a / 2688.0f;
}

__global__ void k_zero1(float* t) { t[0] = 0.0f; }

// fixed layout: a full rank chunk of down and up values (fp64), then lambda
size_t lds_bytes(int64_t) { return (size_t)kRankChunk * kTileCols * 16 + kTileCols * 4; }

template <int MODE>
hipError_t allow_lds(size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_resid<MODE>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

hipError_t launch_residual_f32(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                               const float* lambda, const uint16_t* down, const uint16_t* up,
                               int64_t r, float* R32, float* tensor_scale, hipStream_t s) {
  const int64_t tiles = ((N + kTileRows - 1) / kTileRows) * (K / kTileCols);
  const size_t lds = lds_bytes(r);
  hipError_t e = allow_lds<5>(lds);
  if (e != hipSuccess) return e;
  if (tensor_scale) k_zero1<<<1, 1, 0, s>>>(tensor_scale);
  k_resid<5><<<dim3((unsigned)tiles), dim3(kThreads), lds, s>>>(
      W, N, K, ldw, lambda, down, up, (int)r, tensor_scale, reinterpret_cast<uint8_t*>(R32),
      nullptr);
  if (tensor_scale) k_amax_to_g<<<1, 1, 0, s>>>(tensor_scale);
  return hipGetLastError();
}

hipError_t launch_quantize_weight_r32(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                      const float* lambda, const uint16_t* down,
                                      const uint16_t* up, int64_t r, uint8_t* codes, void* scales,
                                      float* tensor_scale, float* R32, hipStream_t s) {
  const int64_t tiles = ((N + kTileRows - 1) / kTileRows) * (K / kTileCols);
  const size_t lds = lds_bytes(r);
  hipError_t e = allow_lds<5>(lds);
  if (e != hipSuccess) return e;
  // R32 and its max|R32| in one residual pass; the codes from R32; then g = amax / 2688
  k_zero1<<<1, 1, 0, s>>>(tensor_scale);
  k_resid<5><<<dim3((unsigned)tiles), dim3(kThreads), lds, s>>>(
      W, N, K, ldw, lambda, down, up, (int)r, tensor_scale, reinterpret_cast<uint8_t*>(R32),
      nullptr);
  const int64_t npiece = N * (K / 256);  // 1 KB pieces of R32 (K % 256 == 0)
  const int64_t waves = (npiece + kPieces - 1) / kPieces;
  const int64_t grid = (waves + 3) / 4 < 2048 ? (waves + 3) / 4 : 2048;
  k_quant_r32<<<dim3((unsigned)grid), dim3(256), 0, s>>>(R32, npiece, tensor_scale, codes,
                                                         reinterpret_cast<uint8_t*>(scales));
  k_amax_to_g<<<1, 1, 0, s>>>(tensor_scale);
  return hipGetLastError();
}

hipError_t launch_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                                  const float* lambda, const uint16_t* down, const uint16_t* up,
                                  int64_t r, uint8_t* codes, void* scales, float* tensor_scale,
                                  hipStream_t s) {
  const int64_t tiles = ((N + kTileRows - 1) / kTileRows) * (K / kTileCols);
  const size_t lds = lds_bytes(r);
  if (fmt == 2 || fmt == 3) {  // MX: one pass, no tensor scale
    hipError_t e = fmt == 2 ? allow_lds<3>(lds) : allow_lds<4>(lds);
    if (e != hipSuccess) return e;
    if (fmt == 2)
      k_resid<3><<<dim3((unsigned)tiles), dim3(kThreads), lds, s>>>(W, N, K, ldw, lambda, down, up,
                                                                   (int)r, nullptr, codes, scales);
    else
      k_resid<4><<<dim3((unsigned)tiles), dim3(kThreads), lds, s>>>(W, N, K, ldw, lambda, down, up,
                                                                   (int)r, nullptr, codes, scales);
    return hipGetLastError();
  }
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
