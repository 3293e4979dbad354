// Pieces shared by the W4A4 GEMM kernels: the low-rank up-projection (the accumulators' starting
// value), the store (tensor scales, DeltaQuant core term, bf16 through LDS) and the XCD-grouped
// workgroup-to-tile mapping.
#pragma once

#include "device.h"

namespace svdq {

// Workgroup -> output tile.  The hardware hands consecutive workgroup ids to the 8 XCDs in
// turn; each XCD is given a contiguous run of the tile sequence, and the sequence walks groups
// of kGroupM tile rows column by column, so the workgroups resident on one XCD at a time cover a
// compact block of tiles and share their A rows and W columns in that XCD's L2.  Returns false
// for the few padding workgroups of the last run.
constexpr int kGroupM = 8;
__device__ __forceinline__ void tile_of_seq32(int seq, int tiles_m, int tiles_n, int& tm,
                                              int& tn) {
  const int span = kGroupM * tiles_n;
  const int first = (seq / span) * kGroupM;
  const int rows = tiles_m - first < kGroupM ? tiles_m - first : kGroupM;
  const int w = seq % span;
  tm = first + w % rows;
  tn = w / rows;
}

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

// Low-rank term as the accumulators' starting value.  The accumulators hold Σ A'·W' without the
// tensor scales gsc = g_a·g_w, so the term enters as (D/gsc)·L2 and y = gsc·acc at the store.
// It is computed before the main loop, where its D and L2 loads overlap the first stage loads
// instead of standing alone after the loop.  fp32 D/gsc is split into an exact-to-2^-16 bf16
// pair for the bf16 MFMA.
// 32x32 accumulator layout: lane holds column r32 and rows (e/4)*8 + 4h + e%4.
template <int FM, int FN>
__device__ __forceinline__ void gemm_lowrank_init(f32x16_t (&acc)[FM][FN], float inv_gsc,
                                                  int64_t M, int64_t m_base, int64_t n_base,
                                                  int r32, int h, const float* __restrict__ D,
                                                  const uint16_t* __restrict__ up, int r) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
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
}

// Bytes of LDS a wave needs to stage its (32 FM) x (32 FN) bf16 output tile.
template <int FM, int FN>
constexpr int gemm_store_bytes() {
  return FM * 32 * FN * 64;
}

// Store y = bf16(gsc·acc (+ core_out[cube(m)][n])) of the wave's tile at (m_base, n_base).  The
// elements go one by one, in the accumulator layout, into the wave's own LDS region (row-major,
// 64 FN bytes per row), and come back as 16-byte row pieces that are written to Y with
// full-width stores, 4 FN lanes per row segment.  Piece c of staged row R sits at
// c ^ (4 ((R >> 2) & 1)), so the two half-waves of one element write (rows 4 apart) use
// different banks.  Rows past M are not stored.  Y rows must be 16-byte aligned (ldy % 8 == 0).
template <int FM, int FN>
__device__ __forceinline__ void gemm_store(const f32x16_t (&acc)[FM][FN], float gsc,
                                           uint8_t* region, int lane, int64_t M, int64_t N,
                                           int64_t m_base, int64_t n_base,
                                           const float* __restrict__ core_out,
                                           const int32_t* __restrict__ row_to_cube,
                                           uint16_t* __restrict__ Y, int64_t ldy) {
  static_assert(FN >= 2, "the piece swizzle needs at least 8 pieces per staged row");
  static_assert(FM == 4, "the cube-id lookup covers 128 rows per wave");
  constexpr int kRowB = FN * 64;
  const int r32 = lane & 31, h = lane >> 5;
  // DeltaQuant core term: the cube ids of the wave's 128 rows are fetched once (lane l holds
  // rows l and 64 + l) and handed out with lane permutes; each row tile's 16·FN core values
  // are then requested together, so the gather costs a few memory round trips per tile
  // instead of one dependent pair of loads per row.
  int cube_lo = 0, cube_hi = 0;
  if (core_out) {
    int64_t r0 = m_base + lane, r1 = m_base + 64 + lane;
    cube_lo = row_to_cube[r0 < M ? r0 : M - 1];
    cube_hi = row_to_cube[r1 < M ? r1 : M - 1];
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    float cv[16][FN];
    if (core_out) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 32 * i + (e >> 2) * 8 + 4 * h + (e & 3);
        const int cube = __shfl(i < 2 ? cube_lo : cube_hi, row & 63);
        const float* co = core_out + (int64_t)cube * N + n_base;
#pragma unroll
        for (int j = 0; j < FN; ++j) cv[e][j] = co[32 * j + r32];
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 32 * i + (e >> 2) * 8 + 4 * h + (e & 3);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = 32 * j + r32;
        float v = acc[i][j][e] * gsc;
        if (core_out) v += cv[e][j];
        const int piece = (col >> 3) ^ (((row >> 2) & 1) << 2);
        *reinterpret_cast<uint16_t*>(region + row * kRowB + piece * 16 + (col & 7) * 2) =
            f32_to_bf16(v);
      }
    }
  }
  // the pieces are read back by other lanes of this wave
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int kPieces = FM * 32 * (kRowB / 16);
#pragma unroll
  for (int it = 0; it < kPieces / 64; ++it) {
    const int c = it * 64 + lane;
    const int row = c / (kRowB / 16), piece = c % (kRowB / 16);
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
        region + row * kRowB + (piece ^ (((row >> 2) & 1) << 2)) * 16);
    const int64_t grow = m_base + row;
    if (grow < M) *reinterpret_cast<u32x4_t*>(Y + grow * ldy + n_base + piece * 8) = v;
  }
}

}  // namespace svdq
