// Per-modality relative-L2 scoring against the unquantised bf16 layer ("MiniMax-H3 NVFP4 — what
// the smoothing scale should be calibrated on", section "The metric that picks the winner also
// hides the cost": relative L2 on rows drawn uniformly and on rows sampled per modality).
//
// For the sampled rows, Y_ref = bf16(X·Wᵀ) is recomputed on bf16 MFMA (fp32 accumulation) with
// the X rows gathered by index; the epilogue forms (Y − Y_ref)² and Y_ref² per element and
// accumulates them per row group in fp64, then adds each wave's eight sums to `sums`.
// Workgroup tile 128 sampled rows x 128 columns, 4 waves of 64 x 64 (2 x 2 MFMA 32x32 tiles).
// The same kernel can instead store Y_ref of the sampled rows (a sweep over several λ computes
// them once per batch: they do not depend on λ), and k_score_ref then scores against them.
// K mapping: in a 64-element chunk, lane (row = lane % 32, h = lane / 32) holds elements
// [32h, 32h + 32) of its row; MFMA step t takes [8t, 8t + 8) of them, for X and W alike.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;

// WRITE: instead of the sums, Y_ref of sampled row i is stored at Y[i * ldy + n] (bf16).
template <bool WRITE>
__global__ __launch_bounds__(kThreads) void k_score(uint16_t* __restrict__ Y, int64_t ldy,
                                                    const uint16_t* __restrict__ X, int64_t ldx,
                                                    const uint16_t* __restrict__ W, int64_t ldw,
                                                    int64_t M, int64_t N, int64_t K,
                                                    const int32_t* __restrict__ rows,
                                                    const int8_t* __restrict__ grp,
                                                    int64_t n_rows, double* __restrict__ sums) {
  constexpr int FM = 2, FN = 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t i_base = (int64_t)blockIdx.y * 128 + wm * 64;   // sampled-row index
  const int64_t n_base = (int64_t)blockIdx.x * 128 + wn * 64;
  const int r32 = lane & 31, h = lane >> 5;

  const uint16_t* pa[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    int64_t idx = i_base + 32 * i + r32;
    idx = idx < n_rows ? idx : n_rows - 1;
    int64_t m = rows[idx];
    m = m < 0 ? 0 : (m < M ? m : M - 1);  // an out-of-range index reads a valid row
    pa[i] = X + m * ldx + 32 * h;
  }
  const uint16_t* pb[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) pb[j] = W + (n_base + 32 * j + r32) * ldw + 32 * h;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // the operands of chunk k0 + 64 are loaded while chunk k0 is multiplied (two register sets)
  u32x4_t a[2][FM][4], b[2][FN][4];
  auto load = [&](int buf, int64_t k0) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) a[buf][i][t] = reinterpret_cast<const u32x4_t*>(pa[i] + k0)[t];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) b[buf][j][t] = reinterpret_cast<const u32x4_t*>(pb[j] + k0)[t];
  };
  auto mul = [&](int buf) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a[buf][i][t]), __builtin_bit_cast(bf16x8_t, b[buf][j][t]),
              acc[i][j], 0, 0, 0);
  };
  load(0, 0);
  for (int64_t k0 = 0; k0 < K; k0 += 128) {
    if (k0 + 64 < K) load(1, k0 + 64);
    mul(0);
    if (k0 + 64 < K) {
      if (k0 + 128 < K) load(0, k0 + 128);
      mul(1);
    }
  }

  // 32x32 accumulator layout: lane holds column r32 and rows (e/4)*8 + 4h + e%4
  if (WRITE) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t idx = i_base + 32 * i + (e >> 2) * 8 + 4 * h + (e & 3);
        if (idx < n_rows) {
#pragma unroll
          for (int j = 0; j < FN; ++j) Y[idx * ldy + n_base + 32 * j + r32] = f32_to_bf16(acc[i][j][e]);
        }
      }
    return;
  }
  double sd[4] = {0.0, 0.0, 0.0, 0.0}, sr[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t idx = i_base + 32 * i + (e >> 2) * 8 + 4 * h + (e & 3);
      if (idx < n_rows) {
        int64_t m = rows[idx];
        m = m < 0 ? 0 : (m < M ? m : M - 1);
        const int gsel = grp[idx];
        double d2 = 0.0, r2 = 0.0;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float yref = bf16_to_f32(f32_to_bf16(acc[i][j][e]));
          const float y = bf16_to_f32(Y[m * ldy + n_base + 32 * j + r32]);
          const double d = (double)y - (double)yref;
          d2 += d * d;
          r2 += (double)yref * (double)yref;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          sd[g] += gsel == g ? d2 : 0.0;
          sr[g] += gsel == g ? r2 : 0.0;
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    for (int off = 32; off > 0; off >>= 1) {
      sd[g] += __shfl_xor(sd[g], off);
      sr[g] += __shfl_xor(sr[g], off);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (sd[g] != 0.0) atomicAdd(sums + 2 * g, sd[g]);
      if (sr[g] != 0.0) atomicAdd(sums + 2 * g + 1, sr[g]);
    }
  }
}

// Sums against stored reference rows: sampled row i compares Y[rows[i], :] with Yref[i, :].  A
// wave takes one sampled row at a time (grid-stride over rows), its lanes 16-byte pieces of the
// two rows; each lane keeps fp64 sums per row group, the workgroup combines them in LDS and adds
// one value per (group, quantity) to `sums`.
__global__ __launch_bounds__(256) void k_score_ref(const uint16_t* __restrict__ Y, int64_t ldy,
                                                   const uint16_t* __restrict__ Yr, int64_t ldr,
                                                   int64_t M, int64_t N,
                                                   const int32_t* __restrict__ rows,
                                                   const int8_t* __restrict__ grp, int64_t n_rows,
                                                   double* __restrict__ sums) {
  __shared__ double red[4][8];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};  // [group][d2, r2]
  const int64_t n8 = N / 8;
  for (int64_t i = (int64_t)blockIdx.x * 4 + wave; i < n_rows; i += (int64_t)gridDim.x * 4) {
    int64_t m = rows[i];
    m = m < 0 ? 0 : (m < M ? m : M - 1);  // an out-of-range index reads a valid row
    const int g = grp[i];
    const u32x4_t* py = reinterpret_cast<const u32x4_t*>(Y + m * ldy);
    const u32x4_t* pr = reinterpret_cast<const u32x4_t*>(Yr + i * ldr);
    double d2 = 0.0, r2 = 0.0;
    for (int64_t p = lane; p < n8; p += 64) {
      const u32x4_t a = py[p], b = pr[p];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double r0 = (double)bf16_lo(b[e]), r1 = (double)bf16_hi(b[e]);
        const double e0 = (double)bf16_lo(a[e]) - r0, e1 = (double)bf16_hi(a[e]) - r1;
        d2 += e0 * e0 + e1 * e1;
        r2 += r0 * r0 + r1 * r1;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += q == g ? d2 : 0.0;
      acc[2 * q + 1] += q == g ? r2 : 0.0;
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    for (int off = 32; off > 0; off >>= 1) acc[q] += __shfl_xor(acc[q], off);
    if (lane == 0) red[wave][q] = acc[q];
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int q = threadIdx.x;
    const double v = (red[0][q] + red[1][q]) + (red[2][q] + red[3][q]);
    if (v != 0.0) atomicAdd(sums + q, v);
  }
}

}  // namespace

hipError_t launch_score_ref(const uint16_t* Y, int64_t ldy, const uint16_t* Yref, int64_t ldr,
                            int64_t M, int64_t N, const int32_t* rows, const int8_t* grp,
                            int64_t n_rows, double* sums, hipStream_t s) {
  int64_t blocks = (n_rows + 3) / 4;
  blocks = blocks < 2048 ? blocks : 2048;
  k_score_ref<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(Y, ldy, Yref, ldr, M, N, rows, grp,
                                                           n_rows, sums);
  return hipGetLastError();
}

hipError_t launch_score(const uint16_t* Y, int64_t ldy, const uint16_t* X, int64_t ldx,
                        const uint16_t* W, int64_t ldw, int64_t M, int64_t N, int64_t K,
                        const int32_t* rows, const int8_t* grp, int64_t n_rows, double* sums,
                        hipStream_t s) {
  const dim3 grid((unsigned)(N / 128), (unsigned)((n_rows + 127) / 128));
  k_score<false><<<grid, dim3(kThreads), 0, s>>>(const_cast<uint16_t*>(Y), ldy, X, ldx, W, ldw, M,
                                                  N, K, rows, grp, n_rows, sums);
  return hipGetLastError();
}

hipError_t launch_reference_rows(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                                 int64_t M, int64_t N, int64_t K, const int32_t* rows,
                                 int64_t n_rows, uint16_t* Yref, int64_t ldr, hipStream_t s) {
  const dim3 grid((unsigned)(N / 128), (unsigned)((n_rows + 127) / 128));
  k_score<true><<<grid, dim3(kThreads), 0, s>>>(Yref, ldr, X, ldx, W, ldw, M, N, K, rows,
                                                 nullptr, n_rows, nullptr);
  return hipGetLastError();
}

}  // namespace svdq
