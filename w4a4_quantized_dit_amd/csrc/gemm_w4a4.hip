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
// K mapping: within each 64-element half of a stage, lane (row = lane % 32, h = lane / 32) holds
// elements [32h, 32h + 32) of its row (16 contiguous bytes of codes).  MFMA step t (0..3) takes the lane's
// elements [8t, 8t + 8) as its k-slots; the weight operand uses the identical mapping, so every
// product pairs equal K indices.
#include "device.h"
#include "gemm_common.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 512;  // 8 waves, 2 x 4 over the workgroup tile (two per SIMD)

// Workgroup tile 256 x 256, 8 waves in 2 x 4 (two per SIMD), each wave 128 x 64 (4 x 2 MFMA
// tiles of 32x32), tiles assigned in XCD-grouped order.  The second wave on a SIMD issues its
// MFMAs while the other one waits on its conversion chain, which is what keeps the matrix unit
// busy: each wave's fp4 -> fp16 conversions (v_cvt_scalef32_pk_f16_fp4, then the block-scale
// multiply) depend on each other, and a single wave cannot hide that latency.
//
// K advances 128 elements per stage.  Raw codes and scales go from global memory straight into
// a ring of four LDS stage buffers (global_load_lds: no registers, no LDS store instructions),
// three stages ahead.  Code rows are 64 bytes without padding; the 16-byte chunk p of row R
// sits at chunk p ^ ((R >> 2) & 3), so the fragment reads (consecutive rows) spread over the
// banks.  A lane reads its 16 code bytes of a fragment once per 64-element sub-stage (four
// steps), one sub-stage ahead.
constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kRowBytes = kBK / 2;          // 64 bytes of codes per row per stage
constexpr int kStages = 4;
constexpr int kCodeBuf = kBM * kRowBytes;   // per operand per stage
constexpr int kScaleBuf = kBM * (kBK / 16); // 8 scale bytes per row per stage
constexpr int kStageBytes = 2 * kCodeBuf + 2 * kScaleBuf;
constexpr int kLoadsPerStage = 6;           // direct-load instructions per wave per stage

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

__device__ __forceinline__ int swz(int row, int part) { return part ^ ((row >> 2) & 3); }

// This wave's share of one stage: codes as 16-byte chunks (chunk c of an operand: row c / 4,
// stored part c % 4, loaded part swz(row, c % 4)), scales as 4-byte pieces (piece c: row c / 2,
// half c % 2).  Rows of A past M read row M-1 (never stored).
__device__ __forceinline__ void stage_issue(uint8_t* buf, const uint8_t* __restrict__ A,
                                            const uint8_t* __restrict__ As,
                                            const uint8_t* __restrict__ B,
                                            const uint8_t* __restrict__ Bs, int64_t M,
                                            int64_t m0, int64_t n0, int64_t kb, int64_t ks,
                                            int64_t stage, int wave, int lane) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = (wave * 2 + q) * 64 + lane;
    const int row = c >> 2, part = swz(row, c & 3);
    int64_t ar = m0 + row;
    ar = ar < M ? ar : M - 1;
    __builtin_amdgcn_global_load_lds((gvoid_t*)(A + ar * kb + stage * kRowBytes + part * 16),
                                     (lvoid_t*)(buf + (wave * 2 + q) * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(
        (gvoid_t*)(B + (n0 + row) * kb + stage * kRowBytes + part * 16),
        (lvoid_t*)(buf + kCodeBuf + (wave * 2 + q) * 1024), 16, 0, 0);
  }
  const int c = wave * 64 + lane;
  const int row = c >> 1, half = c & 1;
  int64_t ar = m0 + row;
  ar = ar < M ? ar : M - 1;
  __builtin_amdgcn_global_load_lds((gvoid_t*)(As + ar * ks + stage * (kBK / 16) + 4 * half),
                                   (lvoid_t*)(buf + 2 * kCodeBuf + wave * 256), 4, 0, 0);
  __builtin_amdgcn_global_load_lds((gvoid_t*)(Bs + (n0 + row) * ks + stage * (kBK / 16) + 4 * half),
                                   (lvoid_t*)(buf + 2 * kCodeBuf + kScaleBuf + wave * 256), 4, 0,
                                   0);
}

// Workgroup barrier ordering LDS accesses only.  The stage loads are completed explicitly with
// wait_vmcnt before it, so the barrier must not wait for the stages still in flight, which a full
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

__global__ __launch_bounds__(kThreads) void k_gemm_nvfp4(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
    const uint8_t* __restrict__ As, const float* __restrict__ g_a,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs,
    const float* __restrict__ g_w, const float* __restrict__ D,
    const uint16_t* __restrict__ up, int r, const float* __restrict__ core_out,
    const int32_t* __restrict__ row_to_cube, uint16_t* __restrict__ Y, int64_t ldy) {
  constexpr int FM = 4, FN = 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStageBytes];
  int64_t tm, tn;
  if (!tile_of_block((M + kBM - 1) / kBM, N / kBN, tm, tn)) return;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t m_base = m0 + wm * 128, n_base = n0 + wn * 64;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2, ks = K / 16;
  const int64_t nstage = K / kBK;

  // Per-fragment offsets inside a stage buffer: the lane's 16 code bytes of sub-stage `sub`
  // (logical chunk 2 sub + h, swizzled) and its two scale bytes.
  int a_code[2][FM], b_code[2][FN], a_sc[FM], b_sc[FN];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * 128 + 32 * i + r32;
      a_code[sub][i] = row * kRowBytes + 16 * swz(row, 2 * sub + h);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn * 64 + 32 * j + r32;
      b_code[sub][j] = kCodeBuf + row * kRowBytes + 16 * swz(row, 2 * sub + h);
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) a_sc[i] = 2 * kCodeBuf + (wm * 128 + 32 * i + r32) * 8 + 2 * h;
#pragma unroll
  for (int j = 0; j < FN; ++j)
    b_sc[j] = 2 * kCodeBuf + kScaleBuf + (wn * 64 + 32 * j + r32) * 8 + 2 * h;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // prologue: stages 0, 1, 2 in flight; stages 0 and 1 must land (iteration s reads ahead into
  // stage s+1)
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < nstage) stage_issue(lds + p * kStageBytes, A, As, B, Bs, M, m0, n0, kb, ks, p, wave, lane);
  if (nstage >= 3)
    wait_vmcnt<kLoadsPerStage>();
  else
    wait_vmcnt<0>();
  barrier_lds();

  // Raw fragments of one 64-element sub-stage: 16 code bytes (four steps) and the packed pair
  // of block scales per fragment.
  u32x4_t ca[FM], cb[FN];
  f16x2_t sa[FM], sb[FN];
  auto read_sub = [&](const uint8_t* buf, int sub, u32x4_t (&xa)[FM], u32x4_t (&xb)[FN],
                      f16x2_t (&ya)[FM], f16x2_t (&yb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      xa[i] = *reinterpret_cast<const u32x4_t*>(buf + a_code[sub][i]);
      ya[i] = e4m3x2_to_f16x2(*reinterpret_cast<const uint16_t*>(buf + a_sc[i] + 4 * sub));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      xb[j] = *reinterpret_cast<const u32x4_t*>(buf + b_code[sub][j]);
      yb[j] = e4m3x2_to_f16x2(*reinterpret_cast<const uint16_t*>(buf + b_sc[j] + 4 * sub));
    }
  };
  read_sub(lds, 0, ca, cb, sa, sb);
  f16x8_t a_op[FM], b_op[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_op[i] = dequant8(ca[i][0], f16x2_t{sa[i][0], sa[i][0]});
#pragma unroll
  for (int j = 0; j < FN; ++j) b_op[j] = dequant8(cb[j][0], f16x2_t{sb[j][0], sb[j][0]});

  for (int64_t s = 0; s < nstage; ++s) {
    // stage s+3 into the buffer computed in the previous iteration (all waves passed the
    // barrier after it)
    if (s + 3 < nstage)
      stage_issue(lds + ((s + 3) % kStages) * kStageBytes, A, As, B, Bs, M, m0, n0, kb, ks, s + 3,
                  wave, lane);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // raw fragments of the next sub-stage (past the end: this one again, never used)
      u32x4_t na[FM], nb[FN];
      f16x2_t nsa[FM], nsb[FN];
      const bool more = sub == 0 || s + 1 < nstage;
      const uint8_t* nbuf = lds + ((sub == 0 || !more ? s : s + 1) % kStages) * kStageBytes;
      read_sub(nbuf, more ? sub ^ 1 : sub, na, nb, nsa, nsb);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_op[i], b_op[j], acc[i][j], 0, 0, 0);
        // operands of the next step
        if (t < 3) {
          const int hi = (t + 1) >> 1;
#pragma unroll
          for (int i = 0; i < FM; ++i)
            a_op[i] = dequant8(ca[i][t + 1], hi ? f16x2_t{sa[i][1], sa[i][1]} : f16x2_t{sa[i][0], sa[i][0]});
#pragma unroll
          for (int j = 0; j < FN; ++j)
            b_op[j] = dequant8(cb[j][t + 1], hi ? f16x2_t{sb[j][1], sb[j][1]} : f16x2_t{sb[j][0], sb[j][0]});
        } else {
#pragma unroll
          for (int i = 0; i < FM; ++i) a_op[i] = dequant8(na[i][0], f16x2_t{nsa[i][0], nsa[i][0]});
#pragma unroll
          for (int j = 0; j < FN; ++j) b_op[j] = dequant8(nb[j][0], f16x2_t{nsb[j][0], nsb[j][0]});
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        ca[i] = na[i];
        sa[i] = nsa[i];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        cb[j] = nb[j];
        sb[j] = nsb[j];
      }
    }
    // iteration s+1 reads ahead into stage s+2: it must have landed (in every wave) before the
    // barrier; only the loads of stage s+3 may still be in flight
    if (s + 3 < nstage)
      wait_vmcnt<kLoadsPerStage>();
    else
      wait_vmcnt<0>();
    barrier_lds();
  }

  gemm_epilogue<FM, FN>(acc, g_a[0] * g_w[0], M, N, m_base, n_base, r32, h, D, up, r, core_out,
                        row_to_cube, Y, ldy);
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
  const dim3 grid(grid_of_tiles((M + kBM - 1) / kBM, N / kBN));
  k_gemm_nvfp4<<<grid, dim3(kThreads), 0, s>>>(
      M, N, K, a_codes, reinterpret_cast<const uint8_t*>(a_scales), g_a, w_codes,
      reinterpret_cast<const uint8_t*>(w_scales), g_w, D, up, (int)r, core_out, row_to_cube, Y,
      ldy);
  return hipGetLastError();
}

}  // namespace svdq
