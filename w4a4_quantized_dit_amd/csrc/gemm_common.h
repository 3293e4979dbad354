// Pieces shared by the W4A4 GEMM kernels: the epilogue (low-rank up-projection, tensor scales,
// DeltaQuant core term, bf16 store) and the XCD-grouped workgroup-to-tile mapping.
#pragma once

#include "device.h"

namespace svdq {

// Workgroup -> output tile.  The hardware hands consecutive workgroup ids to the 8 XCDs in
// turn; each XCD is given a contiguous run of the tile sequence, and the sequence walks groups
// of kGroupM tile rows column by column, so the workgroups resident on one XCD at a time cover a
// compact block of tiles and share their A rows and W columns in that XCD's L2.  Returns false
// for the few padding workgroups of the last run.
constexpr int kGroupM = 8;
__device__ __forceinline__ bool tile_of_block(int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                              int64_t& tn) {
  const int64_t total = tiles_m * tiles_n;
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t L = blockIdx.x;
  const int64_t seq = (L % 8) * per_xcd + L / 8;
  if (seq >= total) return false;
  const int64_t span = (int64_t)kGroupM * tiles_n;
  const int64_t first = (seq / span) * kGroupM;
  const int64_t rows = tiles_m - first < kGroupM ? tiles_m - first : kGroupM;
  const int64_t w = seq % span;
  tm = first + w % rows;
  tn = w / rows;
  return true;
}

inline unsigned grid_of_tiles(int64_t tiles_m, int64_t tiles_n) {
  return (unsigned)(((tiles_m * tiles_n + 7) / 8) * 8);
}

// Epilogue: low-rank up-projection, tensor scales, DeltaQuant core term, bf16 store.
// The accumulators hold Σ A'·W' without the tensor scales gsc = g_a·g_w; the low-rank term is
// folded in before the scaling as (D/gsc)·L2 so the accumulators stay with the MFMA unit, and
// y = gsc·acc (+ core_out[cube(m)]) is formed element by element at the store.  fp32 D/gsc is
// split into an exact-to-2^-16 bf16 pair for the bf16 MFMA.
// 32x32 accumulator layout: lane holds column r32 and rows (e/4)*8 + 4h + e%4.
template <int FM, int FN>
__device__ __forceinline__ void gemm_epilogue(f32x16_t (&acc)[FM][FN], float gsc, int64_t M,
                                              int64_t N, int64_t m_base, int64_t n_base, int r32,
                                              int h, const float* __restrict__ D,
                                              const uint16_t* __restrict__ up, int r,
                                              const float* __restrict__ core_out,
                                              const int32_t* __restrict__ row_to_cube,
                                              uint16_t* __restrict__ Y, int64_t ldy) {
  const float inv_gsc = 1.0f / gsc;
  for (int t = 0; 16 * t < r; ++t) {
    const int k0 = 16 * t + 8 * h;
    bf16x8_t u_op[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n_base + 32 * j + r32;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (k0 < r) v = *reinterpret_cast<const u32x4_t*>(up + col * r + k0);
      u_op[j] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      int64_t row = m_base + 32 * i + r32;
      row = row < M ? row : M - 1;
      bf16x8_t d_hi, d_lo;
      lowrank_operand(D + row * r + k0, k0 < r, inv_gsc, d_hi, d_lo);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(d_hi, u_op[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(d_lo, u_op[j], acc[i][j], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = m_base + 32 * i + (e >> 2) * 8 + 4 * h + (e & 3);
      if (row < M) {
        const float* co = core_out ? core_out + (int64_t)row_to_cube[row] * N : nullptr;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t col = n_base + 32 * j + r32;
          float v = acc[i][j][e] * gsc;
          if (co) v += co[col];
          Y[row * ldy + col] = f32_to_bf16(v);
        }
      }
    }
  }
}

}  // namespace svdq
