// W4A4 GEMM on gfx950 MFMA with the low-rank up-projection folded into the accumulators before
// the bf16 store:  Y = bf16( g_a·g_w · Σ_k A_deq·W_deq + D·L2 [+ core_out[cube(m)]] )
// ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph; DeltaQuant core term:
// "DeltaQuant on MiniMax-H3").
//
// NVFP4 operands (E2M1 code × E4M3 block scale) need at most 6 significant bits and lie in
// [2^-10, 2688], so they are EXACT in fp16.  The kernel dequantises both operands to fp16 in
// registers (v_cvt_scalef32_pk_f16_fp4 with unit scale, then a packed fp16 multiply by the
// block scale) and runs v_mfma_f32_32x32x16_f16; every product is exact in the fp32
// accumulator, and the two tensor scales are applied once in the epilogue.  The hardware
// block-scaled FP4 MFMA takes power-of-two (E8M0) scales per 32 elements, which cannot carry an
// E4M3 scale per 16 exactly, so it is not used for this format.
//
// K mapping: within a 64-element chunk, lane (row = lane % 32, h = lane / 32) holds elements
// [32h, 32h + 32) of its row (16 contiguous bytes of codes).  MFMA step t (0..3) takes the lane's
// elements [8t, 8t + 8) as its k-slots; the weight operand uses the identical mapping, so every
// product pairs equal K indices.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;  // 4 waves, 2 x 2 over the workgroup tile

__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 0u)
    v = (float)m * 0.001953125f;
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (_Float16)v;  // exact: every E4M3 value is an fp16 value
}

// 8 E2M1 codes (one dword, element i in nibble i) times a block scale -> 8 exact fp16 values.
__device__ __forceinline__ f16x8_t dequant8(uint32_t codes, f16x2_t s2) {
  f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
  f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  f16x8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

template <int FM, int FN>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_nvfp4(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
    const uint8_t* __restrict__ As, const float* __restrict__ g_a,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs,
    const float* __restrict__ g_w, const float* __restrict__ D,
    const uint16_t* __restrict__ up, int r, const float* __restrict__ core_out,
    const int32_t* __restrict__ row_to_cube, uint16_t* __restrict__ Y, int64_t ldy) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m_base = (int64_t)blockIdx.y * (64 * FM) + wm * (32 * FM);
  const int64_t n_base = (int64_t)blockIdx.x * (64 * FN) + wn * (32 * FN);
  if (m_base >= M) return;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2, ks = K / 16;

  const uint8_t* pa[FM];
  const uint8_t* psa[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    int64_t row = m_base + 32 * i + r32;
    row = row < M ? row : M - 1;  // rows past M load valid data whose outputs are discarded
    pa[i] = A + row * kb + 16 * h;
    psa[i] = As + row * ks;
  }
  const uint8_t* pb[FN];
  const uint8_t* psb[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = n_base + 32 * j + r32;
    pb[j] = B + col * kb + 16 * h;
    psb[j] = Bs + col * ks;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int64_t nchunk = K / 64;
  u32x4_t ca[FM], cb[FN];
  uint32_t sa[FM], sb[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    ca[i] = *reinterpret_cast<const u32x4_t*>(pa[i]);
    sa[i] = *reinterpret_cast<const uint32_t*>(psa[i]);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    cb[j] = *reinterpret_cast<const u32x4_t*>(pb[j]);
    sb[j] = *reinterpret_cast<const uint32_t*>(psb[j]);
  }

  for (int64_t c = 0; c < nchunk; ++c) {
    u32x4_t ca_cur[FM], cb_cur[FN];
    uint32_t sa_cur[FM], sb_cur[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) { ca_cur[i] = ca[i]; sa_cur[i] = sa[i]; }
#pragma unroll
    for (int j = 0; j < FN; ++j) { cb_cur[j] = cb[j]; sb_cur[j] = sb[j]; }
    if (c + 1 < nchunk) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        ca[i] = *reinterpret_cast<const u32x4_t*>(pa[i] + (c + 1) * 32);
        sa[i] = *reinterpret_cast<const uint32_t*>(psa[i] + (c + 1) * 4);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        cb[j] = *reinterpret_cast<const u32x4_t*>(pb[j] + (c + 1) * 32);
        sb[j] = *reinterpret_cast<const uint32_t*>(psb[j] + (c + 1) * 4);
      }
    }
    // block scales of this lane: elements 0..15 -> block 2h, 16..31 -> block 2h + 1
    f16x2_t sA[FM][2], sB[FN][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const _Float16 v = e4m3_to_f16((sa_cur[i] >> (8 * (2 * h + u))) & 0xFFu);
        sA[i][u] = f16x2_t{v, v};
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const _Float16 v = e4m3_to_f16((sb_cur[j] >> (8 * (2 * h + u))) & 0xFFu);
        sB[j][u] = f16x2_t{v, v};
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8_t a_op[FM], b_op[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a_op[i] = dequant8(ca_cur[i][t], sA[i][t >> 1]);
#pragma unroll
      for (int j = 0; j < FN; ++j) b_op[j] = dequant8(cb_cur[j][t], sB[j][t >> 1]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_op[i], b_op[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: tensor scales, DeltaQuant core, low-rank up-projection, bf16 store ----
  const float gsc = g_a[0] * g_w[0];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] *= gsc;

  if (core_out) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int64_t row = m_base + 32 * i + (e >> 2) * 8 + 4 * h + (e & 3);
        row = row < M ? row : M - 1;
        const float* co = core_out + (int64_t)row_to_cube[row] * N;
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j][e] += co[n_base + 32 * j + r32];
      }
    }
  }

  for (int t = 0; 16 * t < r; ++t) {
    const int k0 = 16 * t + 8 * h;
    bf16x8_t d_hi[FM], d_lo[FM], u_op[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      int64_t row = m_base + 32 * i + r32;
      row = row < M ? row : M - 1;
      lowrank_operand(D + row * r + k0, k0 < r, d_hi[i], d_lo[i]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n_base + 32 * j + r32;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (k0 < r) v = *reinterpret_cast<const u32x4_t*>(up + col * r + k0);
      u_op[j] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(d_hi[i], u_op[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(d_lo[i], u_op[j], acc[i][j], 0, 0, 0);
      }
  }

  // 32x32 accumulator layout: lane holds column r32 and rows (e/4)*8 + 4h + e%4.
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
                            int64_t ldy, hipStream_t s);

hipError_t launch_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const void* a_scales, const float* g_a, const uint8_t* w_codes,
                       const void* w_scales, const float* g_w, const float* D,
                       const uint16_t* up, int64_t r, const float* core_out,
                       const int32_t* row_to_cube, uint16_t* Y, int64_t ldy, hipStream_t s) {
  if (fmt == 1)
    return launch_gemm_int4(M, N, K, a_codes, a_scales, w_codes, w_scales, D, up, r, Y, ldy, s);
  constexpr int FM = 4, FN = 2;
  const dim3 grid((unsigned)(N / (64 * FN)), (unsigned)((M + 64 * FM - 1) / (64 * FM)));
  k_gemm_nvfp4<FM, FN><<<grid, dim3(kThreads), 0, s>>>(
      M, N, K, a_codes, reinterpret_cast<const uint8_t*>(a_scales), g_a, w_codes,
      reinterpret_cast<const uint8_t*>(w_scales), g_w, D, up, (int)r, core_out, row_to_cube, Y,
      ldy);
  return hipGetLastError();
}

}  // namespace svdq
