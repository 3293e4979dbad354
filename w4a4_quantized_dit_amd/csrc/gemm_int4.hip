// int4-g64 W4A4 GEMM: exact integer-code MFMA per 64-group with fp32 rescaling.
//   Y = bf16( Σ_groups s_a[m,g]·s_w[n,g] · Σ_{k∈g} c_a·c_w  +  D·L2 )
// ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)": int4 codes for weights and per-token
// activations; the per-group fp16 scales of the int4 workload.)
//
// Codes are expanded to int8 with a shift (a nibble in the high half of a byte is 16·c as a
// signed byte), so one v_mfma_i32_32x32x32_i8 pair covers a 64-group of one 32x32 tile with
// 256·Σ c_a·c_w, exact in int32.  The group result is converted once and accumulated with its
// scale product, s_a·s_w/256, in fp32.  The accumulator row of an element is not the lane's
// own operand row, so each wave publishes its rows' activation scales through LDS.
// K mapping: in a 64-group, lane (row = lane % 32, h = lane / 32) holds elements
// [32h, 32h + 32); the weight operand uses the same lane/byte mapping.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;

// 8 int4 nibbles -> two dwords of int8 (16·c): even elements, odd elements.
__device__ __forceinline__ void expand8(uint32_t w, uint32_t& even, uint32_t& odd) {
  even = (w << 4) & 0xF0F0F0F0u;
  odd = w & 0xF0F0F0F0u;
}

template <int FM, int FN>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_int4(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
    const __half* __restrict__ As, const uint8_t* __restrict__ B,
    const __half* __restrict__ Bs, const float* __restrict__ D,
    const uint16_t* __restrict__ up, int r, uint16_t* __restrict__ Y, int64_t ldy) {
  __shared__ float s_sa[4][2][32 * FM];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m_base = (int64_t)blockIdx.y * (64 * FM) + wm * (32 * FM);
  const int64_t n_base = (int64_t)blockIdx.x * (64 * FN) + wn * (32 * FN);
  if (m_base >= M) return;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2, ng = K / 64;

  int64_t arow[FM];
  const uint8_t* pa[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    int64_t row = m_base + 32 * i + r32;
    arow[i] = row < M ? row : M - 1;
    pa[i] = A + arow[i] * kb + 16 * h;
  }
  const uint8_t* pb[FN];
  int64_t bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    bcol[j] = n_base + 32 * j + r32;
    pb[j] = B + bcol[j] * kb + 16 * h;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  u32x4_t ca[FM], cb[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) ca[i] = *reinterpret_cast<const u32x4_t*>(pa[i]);
#pragma unroll
  for (int j = 0; j < FN; ++j) cb[j] = *reinterpret_cast<const u32x4_t*>(pb[j]);

  for (int64_t g = 0; g < ng; ++g) {
    u32x4_t ca_cur[FM], cb_cur[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) ca_cur[i] = ca[i];
#pragma unroll
    for (int j = 0; j < FN; ++j) cb_cur[j] = cb[j];
    if (g + 1 < ng) {
#pragma unroll
      for (int i = 0; i < FM; ++i) ca[i] = *reinterpret_cast<const u32x4_t*>(pa[i] + (g + 1) * 32);
#pragma unroll
      for (int j = 0; j < FN; ++j) cb[j] = *reinterpret_cast<const u32x4_t*>(pb[j] + (g + 1) * 32);
    }
    // publish this wave's activation-row scales of group g, read the ones of the accumulator rows
    float* slot = s_sa[wave][g & 1];
    if (h == 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i) slot[32 * i + r32] = __half2float(As[arow[i] * ng + g]);
    }
    float sw[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) sw[j] = __half2float(Bs[bcol[j] * ng + g]) * 0.00390625f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    uint32_t a8[FM][8], b8[FN][8];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) expand8(ca_cur[i][d], a8[i][2 * d], a8[i][2 * d + 1]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int d = 0; d < 4; ++d) expand8(cb_cur[j][d], b8[j][2 * d], b8[j][2 * d + 1]);

#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float sa[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) sa[e] = slot[32 * i + (e >> 2) * 8 + 4 * h + (e & 3)];
      const i32x4_t a_lo = {(int)a8[i][0], (int)a8[i][1], (int)a8[i][2], (int)a8[i][3]};
      const i32x4_t a_hi = {(int)a8[i][4], (int)a8[i][5], (int)a8[i][6], (int)a8[i][7]};
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const i32x4_t b_lo = {(int)b8[j][0], (int)b8[j][1], (int)b8[j][2], (int)b8[j][3]};
        const i32x4_t b_hi = {(int)b8[j][4], (int)b8[j][5], (int)b8[j][6], (int)b8[j][7]};
        i32x16_t p = {};
        p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_lo, b_lo, p, 0, 0, 0);
        p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_hi, b_hi, p, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] += (float)p[e] * (sa[e] * sw[j]);
      }
    }
  }

  for (int t = 0; 16 * t < r; ++t) {
    const int k0 = 16 * t + 8 * h;
    bf16x8_t d_hi[FM], d_lo[FM], u_op[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) lowrank_operand(D + arow[i] * r + k0, k0 < r, 1.0f, d_hi[i], d_lo[i]);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (k0 < r) v = *reinterpret_cast<const u32x4_t*>(up + bcol[j] * r + k0);
      u_op[j] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
      {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(d_hi[i], u_op[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(d_lo[i], u_op[j], acc[i][j], 0, 0, 0);
      }
  }

#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = m_base + 32 * i + (e >> 2) * 8 + 4 * h + (e & 3);
      if (row < M) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          Y[row * ldy + n_base + 32 * j + r32] = f32_to_bf16(acc[i][j][e]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_int4(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const void* a_scales, const uint8_t* w_codes, const void* w_scales,
                            const float* D, const uint16_t* up, int64_t r, uint16_t* Y,
                            int64_t ldy, hipStream_t s) {
  constexpr int FM = 4, FN = 2;
  const dim3 grid((unsigned)(N / (64 * FN)), (unsigned)((M + 64 * FM - 1) / (64 * FM)));
  k_gemm_int4<FM, FN><<<grid, dim3(kThreads), 0, s>>>(
      M, N, K, a_codes, reinterpret_cast<const __half*>(a_scales), w_codes,
      reinterpret_cast<const __half*>(w_scales), D, up, (int)r, Y, ldy);
  return hipGetLastError();
}

}  // namespace svdq
