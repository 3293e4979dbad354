// MX variant of the layer's GEMM on gfx950's hardware block-scaled MFMA:
//   Y = bf16( Σ_blocks 2^(e_a + e_w) · Σ_{k in block} c_a·c_w  +  D·L2 )
// with E2M1 (MXFP4, W4A4) or E4M3 (MXFP8, W8A8) codes and one E8M0 exponent per 32 along K
// ("MiniMax-H3 — MXFP8 (weight-quantized, vLLM-Omni native layout)", section "Quant format";
// the layer: "MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph).
//
// This is the scale layout v_mfma_scale_f32_32x32x64_f8f6f4 takes natively: one MFMA covers 64
// elements of K, i.e. two scale blocks per row, and each lane supplies the E8M0 byte of its
// (row, block).  The codes go from global memory straight into LDS (global_load_lds) and from
// LDS into the MFMA with no conversion at all.  Operand layout (measured): lane (row = lane % 32,
// h = lane / 32) holds, for FP4, elements [32h, 32h + 32) of the 64 in dwords 0..3 (element 8d
// + j in nibble j of dword d); for FP8, dwords 0..3 hold elements [16h, 16h + 16) of block 0 and
// dwords 4..7 the same positions of block 1, with lane h supplying block h's scale.  Inside a
// block the element order only has to agree between A and W.
//
// Tiling: workgroup 256 x 256, 8 waves (two per SIMD) of 128 x 64 (4 x 2 tiles of 32x32),
// XCD-grouped tile order; K advances 128 elements per stage (two MFMA steps), staged through a
// ring of LDS buffers (four for FP4, two for FP8), with one LDS-only barrier per stage.  A row's
// 16-byte code chunk c of a stage is stored at chunk c ^ f(row) (f = (row >> 2) & 3 for 4 chunks
// per row, (row >> 1) & 7 for 8), which keeps the fragment reads (32 consecutive rows, one
// chunk) free of bank conflicts.  The E8M0 bytes of a row's four blocks of the stage are one
// dword.  The low-rank term and the LDS-staged bf16 store are the ones of the NVFP4 GEMM.
#include "device.h"
#include "gemm_common.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 512;
constexpr int kBM = 256, kBN = 256, kBK = 128;

template <int FP8>
struct MxCfg {
  static constexpr int kRowBytes = FP8 ? 128 : 64;       // codes of a row per stage
  static constexpr int kChunks = kRowBytes / 16;         // 16-byte chunks per row per stage
  static constexpr int kStages = FP8 ? 2 : 4;
  static constexpr int kCodeBuf = kBM * kRowBytes;       // one operand, one stage
  static constexpr int kScaleBuf = kBM * 4;              // four E8M0 bytes per row per stage
  static constexpr int kStageBytes = 2 * kCodeBuf + 2 * kScaleBuf;
  static constexpr int kPerWave = kBM * kChunks / 64 / 8;  // 16-byte loads per wave per operand
  static constexpr int kLoads = 2 * kPerWave + 1;          // direct loads per wave per stage
};

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

template <int FP8>
__device__ __forceinline__ int chunk_swz(int row) {
  return FP8 ? (row >> 1) & 7 : (row >> 2) & 3;
}

// Workgroup barrier ordering LDS accesses only; the stage loads are completed with explicit
// vmcnt waits before it, so it must not drain the stages still in flight, which a full
// __syncthreads() fence would do.  (The memory clobber keeps the compiler from moving memory
// accesses across it.)
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(n) (other counters untouched), gfx9 encoding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// This wave's share of one stage: code chunks (chunk id c of an operand: row c / kChunks, stored
// part c % kChunks holding logical part (c % kChunks) ^ f(row)); then the scale dwords of 64 rows
// (waves 0..3: A, 4..7: W).  Rows of A past M read row M-1 (never stored).
template <int FP8>
__device__ __forceinline__ void stage_issue(uint8_t* buf, const uint8_t* __restrict__ A,
                                            const uint8_t* __restrict__ As,
                                            const uint8_t* __restrict__ B,
                                            const uint8_t* __restrict__ Bs, int64_t M, int64_t m0,
                                            int64_t n0, int64_t kb, int64_t ks, int64_t stage,
                                            int wave, int lane) {
  using C = MxCfg<FP8>;
#pragma unroll
  for (int q = 0; q < C::kPerWave; ++q) {
    const int c = (wave * C::kPerWave + q) * 64 + lane;
    const int row = c / C::kChunks, part = (c % C::kChunks) ^ chunk_swz<FP8>(row);
    int64_t ar = m0 + row;
    ar = ar < M ? ar : M - 1;
    __builtin_amdgcn_global_load_lds(
        (gvoid_t*)(A + ar * kb + stage * C::kRowBytes + part * 16),
        (lvoid_t*)(buf + (wave * C::kPerWave + q) * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(
        (gvoid_t*)(B + (n0 + row) * kb + stage * C::kRowBytes + part * 16),
        (lvoid_t*)(buf + C::kCodeBuf + (wave * C::kPerWave + q) * 1024), 16, 0, 0);
  }
  const int srow = (wave & 3) * 64 + lane;
  int64_t sr = (wave < 4 ? m0 : n0) + srow;
  if (wave < 4) sr = sr < M ? sr : M - 1;
  __builtin_amdgcn_global_load_lds(
      (gvoid_t*)((wave < 4 ? As : Bs) + sr * ks + stage * (kBK / 32)),
      (lvoid_t*)(buf + 2 * C::kCodeBuf + (wave < 4 ? 0 : C::kScaleBuf) + (wave & 3) * 256), 4, 0,
      0);
}

template <int FP8>
__global__ __launch_bounds__(kThreads) void k_gemm_mx(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
    const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const float* __restrict__ D,
    const uint16_t* __restrict__ up, int r, uint16_t* __restrict__ Y, int64_t ldy) {
  using C = MxCfg<FP8>;
  constexpr int FM = 4, FN = 2;
  constexpr int kFmt = FP8 ? 0 : 4;  // MFMA operand format: 0 E4M3, 4 E2M1
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kStages * C::kStageBytes];
  int64_t tm, tn;
  if (!tile_of_block((M + kBM - 1) / kBM, N / kBN, tm, tn)) return;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t m_base = m0 + wm * 128, n_base = n0 + wn * 64;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = FP8 ? K : K / 2, ks = K / 32;
  const int64_t nstage = K / kBK;

  // the lane's fragment rows share their low 5 bits with r32, hence one swizzle for all
  const int sw = chunk_swz<FP8>(r32);
  int a_row[FM], b_row[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_row[i] = (wm * 128 + 32 * i + r32);
#pragma unroll
  for (int j = 0; j < FN; ++j) b_row[j] = (wn * 64 + 32 * j + r32);

  f32x16_t acc[FM][FN];
  gemm_lowrank_init<FM, FN>(acc, 1.0f, M, m_base, n_base, r32, h, D, up, r);

  // prologue: stages 0 .. S-2 in flight, stage 0 landed
#pragma unroll
  for (int p = 0; p < C::kStages - 1; ++p)
    if (p < nstage)
      stage_issue<FP8>(lds + p * C::kStageBytes, A, As, B, Bs, M, m0, n0, kb, ks, p, wave, lane);
  if (nstage >= C::kStages - 1)
    wait_vmcnt<(C::kStages - 2) * C::kLoads>();
  else
    wait_vmcnt<0>();
  barrier_lds();

  for (int64_t s = 0; s < nstage; ++s) {
    // stage s+S-1 into the buffer computed in the previous iteration (all waves passed the
    // barrier after it)
    if (s + C::kStages - 1 < nstage)
      stage_issue<FP8>(lds + ((s + C::kStages - 1) % C::kStages) * C::kStageBytes, A, As, B, Bs,
                       M, m0, n0, kb, ks, s + C::kStages - 1, wave, lane);
    const uint8_t* buf = lds + (s % C::kStages) * C::kStageBytes;
    // E8M0 bytes of the fragments' rows for the stage's four blocks; step t, lane h uses block
    // 2t + h
    uint32_t sa[FM], sb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      sa[i] = *reinterpret_cast<const uint32_t*>(buf + 2 * C::kCodeBuf + a_row[i] * 4) >> (8 * h);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      sb[j] = *reinterpret_cast<const uint32_t*>(buf + 2 * C::kCodeBuf + C::kScaleBuf +
                                                 b_row[j] * 4) >> (8 * h);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      i32x8_t a_op[FM], b_op[FN];
      auto frag = [&](int base, int row) {
        i32x8_t v;
        if (FP8) {
          const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(
              buf + base + row * C::kRowBytes + 16 * ((4 * t + h) ^ sw));
          const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(
              buf + base + row * C::kRowBytes + 16 * ((4 * t + 2 + h) ^ sw));
          v = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else {
          const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(
              buf + base + row * C::kRowBytes + 16 * ((2 * t + h) ^ sw));
          v = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
        }
        return v;
      };
#pragma unroll
      for (int i = 0; i < FM; ++i) a_op[i] = frag(0, a_row[i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) b_op[j] = frag(C::kCodeBuf, b_row[j]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a_op[i], b_op[j], acc[i][j], kFmt, kFmt, 0, (int)((sa[i] >> (16 * t)) & 0xFFu), 0,
              (int)((sb[j] >> (16 * t)) & 0xFFu));
    }
    // the next iteration reads stage s+1: it must have landed (in every wave) before the
    // barrier; only the stages issued after it may still be in flight
    if (s + C::kStages - 1 < nstage)
      wait_vmcnt<(C::kStages - 2) * C::kLoads>();
    else
      wait_vmcnt<0>();
    barrier_lds();
  }

  // every wave passed the last barrier after its final reads: the ring is free for the output
  // staging (each wave its own 16 KB)
  static_assert(8 * gemm_store_bytes<FM, FN>() <= C::kStages * C::kStageBytes,
                "output staging fits the LDS");
  gemm_store<FM, FN>(acc, 1.0f, lds + wave * gemm_store_bytes<FM, FN>(), lane, M, N, m_base,
                     n_base, nullptr, nullptr, Y, ldy);
}

}  // namespace

hipError_t launch_gemm_mx(int fp8, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                          const uint8_t* a_scales, const uint8_t* w_codes,
                          const uint8_t* w_scales, const float* D, const uint16_t* up, int64_t r,
                          uint16_t* Y, int64_t ldy, hipStream_t s) {
  const dim3 grid(grid_of_tiles((M + kBM - 1) / kBM, N / kBN));
  if (fp8)
    k_gemm_mx<1><<<grid, dim3(kThreads), 0, s>>>(M, N, K, a_codes, a_scales, w_codes, w_scales, D,
                                                 up, (int)r, Y, ldy);
  else
    k_gemm_mx<0><<<grid, dim3(kThreads), 0, s>>>(M, N, K, a_codes, a_scales, w_codes, w_scales, D,
                                                 up, (int)r, Y, ldy);
  return hipGetLastError();
}

}  // namespace svdq
