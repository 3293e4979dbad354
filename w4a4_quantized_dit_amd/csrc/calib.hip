// λ calibration reduction ("MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated
// on", section "Calibration": per-channel activation absmax accumulated under a modality mask
// feeds λ).  HBM-bound: one streaming read of X (and of W), order-free max reductions.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kAbsmaxWaves = 4;
constexpr int kAbsmaxThreads = 64 * kAbsmaxWaves;  // a block covers 512 channels (8 per lane)
constexpr int kAbsmaxRows = 512;                    // rows per block (never straddling a segment)
constexpr int kUnroll = 16;                         // loads in flight per lane

// Row chunks of one launch: X's three modality segments, then (optionally) W as a fourth.
struct SegChunks {
  int64_t seg[5];     // {0, n_text, n_text + n_video, M, M + N}: X rows, then W rows
  int64_t cstart[5];  // first chunk of each segment (cumulative), cstart[4] = total
};

__global__ void k_fill2(float* __restrict__ p, int64_t n, float v, float* __restrict__ q,
                        int64_t nq, float vq) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
  if (q && i < nq) q[i] = vq;
}

typedef __attribute__((ext_vector_type(8))) uint16_t u16x8;

// ax[mu*K + k] = max(ax, max over the chunk's rows of |X[row, k]|) for the three modality
// segments, and aw[k] = max(aw, max |W[row, k]|) for the fourth (W's rows).  bf16 magnitudes
// compare as unsigned 15-bit patterns, so the max is taken on integers; the four waves of a
// block take interleaved rows and combine through LDS before one atomic per channel.  The rows
// are streamed once: nontemporal loads.
__global__ __launch_bounds__(kAbsmaxThreads) void k_absmax(const uint16_t* __restrict__ X,
                                                           int64_t ldx,
                                                           const uint16_t* __restrict__ W,
                                                           int64_t ldw, int64_t K, SegChunks sc,
                                                           float* __restrict__ ax,
                                                           float* __restrict__ aw) {
  __shared__ u16x8 red[kAbsmaxWaves][64];
  const int64_t chunk = blockIdx.y;
  const int mu = (chunk >= sc.cstart[1]) + (chunk >= sc.cstart[2]) + (chunk >= sc.cstart[3]);
  int64_t r0 = sc.seg[mu] + (chunk - sc.cstart[mu]) * kAbsmaxRows;
  int64_t r1 = min(r0 + (int64_t)kAbsmaxRows, sc.seg[mu + 1]);
  const uint16_t* base = X;
  int64_t ld = ldx;
  if (mu == 3) {  // W rows
    base = W;
    ld = ldw;
    r0 -= sc.seg[3];
    r1 -= sc.seg[3];
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t col = ((int64_t)blockIdx.x * 64 + lane) * 8;
  const u16x8 mask = (u16x8)(0x7FFF);
  u16x8 m = (u16x8)(0);
  if (col < K) {
    const uint16_t* p = base + col;
    int64_t r = r0 + wave;
    for (; r + (kUnroll - 1) * kAbsmaxWaves < r1; r += kUnroll * kAbsmaxWaves) {
      u16x8 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = __builtin_nontemporal_load((const u16x8*)(p + (r + u * kAbsmaxWaves) * ld));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) m = __builtin_elementwise_max(m, v[u] & mask);
    }
    for (; r < r1; r += kAbsmaxWaves) m = __builtin_elementwise_max(m, *(const u16x8*)(p + r * ld) & mask);
  }
  red[wave][lane] = m;
  __syncthreads();
  if (wave == 0 && col < K) {
#pragma unroll
    for (int w = 1; w < kAbsmaxWaves; ++w) m = __builtin_elementwise_max(m, red[w][lane]);
    float* o = (mu == 3 ? aw : ax + (int64_t)mu * K) + col;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (m[j]) atomic_max_pos(o + j, bf16_to_f32(m[j]));
  }
}

// λ from the (accumulated) maxima, and the static activation amax max_k ax_all[k]·(1/λ[k]).
__global__ __launch_bounds__(1024) void k_lambda(const float* __restrict__ ax,
                                                 const float* __restrict__ aw, int64_t K,
                                                 uint32_t mask, float alpha,
                                                 float* __restrict__ lam,
                                                 float* __restrict__ act_amax) {
  __shared__ float red[16];
  float local = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += blockDim.x) {
    const float a0 = ax[k], a1 = ax[K + k], a2 = ax[2 * K + k];
    float sel = 0.0f;
    if (mask & 1u) sel = fmaxf(sel, a0);
    if (mask & 2u) sel = fmaxf(sel, a1);
    if (mask & 4u) sel = fmaxf(sel, a2);
    const float w = aw[k];
    float l = 1.0f;
    if (mask != 0u && sel != 0.0f && w != 0.0f) {
      if (alpha == 0.5f) {
        l = __builtin_sqrtf(sel / w);
      } else {
        l = (float)(pow((double)sel, (double)alpha) / pow((double)w, 1.0 - (double)alpha));
      }
    }
    lam[k] = l;
    const float inv = 1.0f / l;
    local = fmaxf(local, fmaxf(fmaxf(a0, a1), a2) * inv);
  }
  for (int off = 32; off > 0; off >>= 1) local = fmaxf(local, __shfl_xor(local, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = local;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = 0.0f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
    act_amax[0] = m;
  }
}

SegChunks make_chunks(const int64_t seg[4], int64_t n_w) {
  SegChunks sc;
  for (int i = 0; i < 4; ++i) sc.seg[i] = seg[i];
  sc.seg[4] = seg[3] + n_w;
  sc.cstart[0] = 0;
  for (int i = 0; i < 4; ++i)
    sc.cstart[i + 1] = sc.cstart[i] + (sc.seg[i + 1] - sc.seg[i] + kAbsmaxRows - 1) / kAbsmaxRows;
  return sc;
}

// Bits-lost proxy ("MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on",
// section "Why"): one workgroup per modality, a thread per group of `block` channels at a time.
// The smoothed channel maximum is fp32(ax · fp32(1/λ)) as in the activation kernel (correctly
// rounded reciprocal, no contraction); each live channel adds log2(group max / its max) in fp64.
constexpr int kBitsThreads = 256;
__global__ __launch_bounds__(kBitsThreads) void k_bits_lost(const float* __restrict__ ax,
                                                            const float* __restrict__ lambda,
                                                            int64_t K, int block,
                                                            double* __restrict__ out) {
  const float* a = ax + (int64_t)blockIdx.x * K;
  double sum = 0.0;
  int64_t live = 0;
  for (int64_t g = threadIdx.x; g < K / block; g += kBitsThreads) {
    const int64_t k0 = g * block;
    float gmax = 0.0f;
    for (int j = 0; j < block; ++j) {
      const float c = a[k0 + j] * (lambda ? 1.0f / lambda[k0 + j] : 1.0f);
      gmax = fmaxf(gmax, c);
    }
    for (int j = 0; j < block; ++j) {
      const float c = a[k0 + j] * (lambda ? 1.0f / lambda[k0 + j] : 1.0f);
      if (c > 0.0f) {
        sum += log2((double)gmax / (double)c);
        ++live;
      }
    }
  }
  __shared__ double s_sum[kBitsThreads];
  __shared__ int64_t s_live[kBitsThreads];
  s_sum[threadIdx.x] = sum;
  s_live[threadIdx.x] = live;
  __syncthreads();
  for (int w = kBitsThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s_sum[threadIdx.x] += s_sum[threadIdx.x + w];
      s_live[threadIdx.x] += s_live[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = s_live[0] ? s_sum[0] / (double)s_live[0] : 0.0;
}

}  // namespace

hipError_t launch_calibrate(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                            const int64_t seg[4], const uint16_t* W, int64_t N, int64_t ldw,
                            uint32_t mask, float alpha, int accumulate, float* ax, float* aw,
                            float* lambda, float* act_amax, hipStream_t s) {
  hipError_t e;
  // one fill launch: clears ax (unless accumulating) and sets aw (0 before a max over W, or 1
  // without W)
  if (!accumulate || !W) {
    float* p = accumulate ? nullptr : ax;
    float* q = (!accumulate || !W) ? aw : nullptr;
    const int64_t n = 3 * K;
    k_fill2<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(
        p ? p : aw, p ? n : 0, 0.0f, q, q ? K : 0, W ? 0.0f : 1.0f);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // one launch over X's modality segments and W's rows
  const SegChunks sc = make_chunks(seg, W ? N : 0);
  if (sc.cstart[4] > 0) {
    const dim3 grid((unsigned)((K / 8 + 63) / 64), (unsigned)sc.cstart[4]);
    k_absmax<<<grid, dim3(kAbsmaxThreads), 0, s>>>(X, ldx, W, ldw, K, sc, ax, aw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  k_lambda<<<dim3(1), dim3(1024), 0, s>>>(ax, aw, K, mask, alpha, lambda, act_amax);
  return hipGetLastError();
}

hipError_t launch_lambda(const float* ax, const float* aw, int64_t K, uint32_t mask, float alpha,
                         float* lambda, float* act_amax, hipStream_t s) {
  k_lambda<<<dim3(1), dim3(1024), 0, s>>>(ax, aw, K, mask, alpha, lambda, act_amax);
  return hipGetLastError();
}

hipError_t launch_bits_lost(const float* ax, const float* lambda, int64_t K, int block,
                            double* out, hipStream_t s) {
  k_bits_lost<<<dim3(3), dim3(kBitsThreads), 0, s>>>(ax, lambda, K, block, out);
  return hipGetLastError();
}

}  // namespace svdq
