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

constexpr int kThreads = 256;  // 4 waves, 2 x 2 over the workgroup tile
#ifndef SVDQ_GEMM_VALU_PER_MFMA
#define SVDQ_GEMM_VALU_PER_MFMA 4   // scheduling hint: dequantisation VALU ops between MFMAs
#endif

// Workgroup tile 256 x 256, 4 waves in 2 x 2, each wave 128 x 128 (4 x 4 MFMA tiles of 32x32),
// tiles assigned in XCD-grouped order.  K advances 128 elements per stage.  Raw codes and scales are staged global -> registers ->
// LDS through three LDS buffers (the loads for stage s+3 are in flight while stage s is
// computed); each wave dequantises its own fragments from LDS.
constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kRowBytes = kBK / 2;          // 64 bytes of codes per row per stage
constexpr int kRowPitch = kRowBytes + 16;   // padded pitch: conflict-free 16-byte reads
constexpr int kStages = 3;
constexpr int kCodeBuf = kBM * kRowPitch;   // per operand per stage
constexpr int kScaleBuf = kBM * (kBK / 16); // 8 scale bytes per row per stage
constexpr int kStageBytes = 2 * kCodeBuf + 2 * kScaleBuf;

struct StageRegs {
  u32x4_t a[4], b[4];  // 4 x 16 B of codes per operand per thread
  uint2 sa, sb;        // threads 0..255: 8 scale bytes of one row (A and W)
};

__device__ __forceinline__ void stage_load(StageRegs& g, const uint8_t* __restrict__ A,
                                           const uint8_t* __restrict__ As,
                                           const uint8_t* __restrict__ B,
                                           const uint8_t* __restrict__ Bs, int64_t M,
                                           int64_t m0, int64_t n0, int64_t kb, int64_t ks,
                                           int64_t stage, int tid) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;            // chunk id: row = c / 4, part = c % 4
    const int row = c >> 2, part = c & 3;
    int64_t ar = m0 + row;
    ar = ar < M ? ar : M - 1;
    g.a[j] = *reinterpret_cast<const u32x4_t*>(A + ar * kb + stage * kRowBytes + part * 16);
    g.b[j] = *reinterpret_cast<const u32x4_t*>(B + (n0 + row) * kb + stage * kRowBytes + part * 16);
  }
  int64_t ar = m0 + tid;
  ar = ar < M ? ar : M - 1;
  g.sa = *reinterpret_cast<const uint2*>(As + ar * ks + stage * (kBK / 16));
  g.sb = *reinterpret_cast<const uint2*>(Bs + (n0 + tid) * ks + stage * (kBK / 16));
}

__device__ __forceinline__ void stage_store(const StageRegs& g, uint8_t* lds, int tid) {
  uint8_t* la = lds;
  uint8_t* lb = lds + kCodeBuf;
  uint8_t* lsa = lds + 2 * kCodeBuf;
  uint8_t* lsb = lsa + kScaleBuf;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;
    const int row = c >> 2, part = c & 3;
    *reinterpret_cast<u32x4_t*>(la + row * kRowPitch + part * 16) = g.a[j];
    *reinterpret_cast<u32x4_t*>(lb + row * kRowPitch + part * 16) = g.b[j];
  }
  *reinterpret_cast<uint2*>(lsa + tid * 8) = g.sa;
  *reinterpret_cast<uint2*>(lsb + tid * 8) = g.sb;
}

// Raw operand fragments of one 64-element sub-stage: per MFMA tile row / column, 16 B of codes
// (32 elements of the lane's row) and the two E4M3 block scales as broadcast fp16 pairs.
template <int F>
struct Frags {
  u32x4_t c[F];
  f16x2_t s[F][2];
};

template <int F>
__device__ __forceinline__ void read_frags(Frags<F>& f, const uint8_t* codes,
                                           const uint8_t* scales, int sub) {
#pragma unroll
  for (int i = 0; i < F; ++i) {
    f.c[i] = *reinterpret_cast<const u32x4_t*>(codes + i * 32 * kRowPitch + 32 * sub);
    const uint32_t sc = *reinterpret_cast<const uint16_t*>(scales + i * 32 * 8 + 4 * sub);
    const f16x2_t p = e4m3x2_to_f16x2(sc);
    f.s[i][0] = f16x2_t{p[0], p[0]};
    f.s[i][1] = f16x2_t{p[1], p[1]};
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_nvfp4(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
    const uint8_t* __restrict__ As, const float* __restrict__ g_a,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs,
    const float* __restrict__ g_w, const float* __restrict__ D,
    const uint16_t* __restrict__ up, int r, const float* __restrict__ core_out,
    const int32_t* __restrict__ row_to_cube, uint16_t* __restrict__ Y, int64_t ldy) {
  constexpr int FM = 4, FN = 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStageBytes];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  int64_t tm, tn;
  if (!tile_of_block((M + kBM - 1) / kBM, N / kBN, tm, tn)) return;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int64_t m_base = m0 + wm * 128, n_base = n0 + wn * 128;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2, ks = K / 16;
  const int64_t nstage = K / kBK;
  // this lane's fragment rows within a stage buffer
  const int a_off = (wm * 128 + r32) * kRowPitch + 16 * h;
  const int b_off = kCodeBuf + (wn * 128 + r32) * kRowPitch + 16 * h;
  const int sa_off = 2 * kCodeBuf + (wm * 128 + r32) * 8 + 2 * h;
  const int sb_off = 2 * kCodeBuf + kScaleBuf + (wn * 128 + r32) * 8 + 2 * h;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  StageRegs g;
  // prologue: stages 0 and 1 into LDS, stage 2 in registers
  stage_load(g, A, As, B, Bs, M, m0, n0, kb, ks, 0, tid);
  stage_store(g, lds, tid);
  if (nstage > 1) {
    stage_load(g, A, As, B, Bs, M, m0, n0, kb, ks, 1, tid);
    stage_store(g, lds + kStageBytes, tid);
  }
  if (nstage > 2) stage_load(g, A, As, B, Bs, M, m0, n0, kb, ks, 2, tid);
  __syncthreads();

  // Software pipeline over K16 steps: while the 16 MFMAs of one step run, the operands of the
  // next step are dequantised (VALU) and, at the last step of a sub-stage, the next sub-stage's
  // raw fragments are read from LDS.  Stage s+1 is already complete in its LDS buffer while
  // stage s is computed (three buffers), so the look-ahead never waits on a barrier.
  Frags<FM> fa;
  Frags<FN> fb;
  read_frags(fa, lds + a_off, lds + sa_off, 0);
  read_frags(fb, lds + b_off, lds + sb_off, 0);
  f16x8_t a_op[FM], b_op[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_op[i] = dequant8(fa.c[i][0], fa.s[i][0]);
#pragma unroll
  for (int j = 0; j < FN; ++j) b_op[j] = dequant8(fb.c[j][0], fb.s[j][0]);

  for (int64_t s = 0; s < nstage; ++s) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      Frags<FM> na;
      Frags<FN> nb;
      const bool more = sub == 0 || s + 1 < nstage;
      if (more) {
        const uint8_t* nbuf = lds + ((sub == 0 ? s : s + 1) % kStages) * kStageBytes;
        read_frags(na, nbuf + a_off, nbuf + sa_off, sub ^ 1);
        read_frags(nb, nbuf + b_off, nbuf + sb_off, sub ^ 1);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f16x8_t a_nx[FM], b_nx[FN];
        if (t < 3) {
#pragma unroll
          for (int i = 0; i < FM; ++i) a_nx[i] = dequant8(fa.c[i][t + 1], fa.s[i][(t + 1) >> 1]);
#pragma unroll
          for (int j = 0; j < FN; ++j) b_nx[j] = dequant8(fb.c[j][t + 1], fb.s[j][(t + 1) >> 1]);
        } else if (more) {
#pragma unroll
          for (int i = 0; i < FM; ++i) a_nx[i] = dequant8(na.c[i][0], na.s[i][0]);
#pragma unroll
          for (int j = 0; j < FN; ++j) b_nx[j] = dequant8(nb.c[j][0], nb.s[j][0]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_op[i], b_op[j], acc[i][j], 0, 0, 0);
        // interleave: one MFMA, then a few VALU instructions of the next step's dequantisation
#if SVDQ_GEMM_VALU_PER_MFMA > 0
#pragma unroll
        for (int k = 0; k < FM * FN; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, SVDQ_GEMM_VALU_PER_MFMA, 0);
        }
#endif
#pragma unroll
        for (int i = 0; i < FM; ++i) a_op[i] = a_nx[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) b_op[j] = b_nx[j];
      }
      fa = na;
      fb = nb;
    }
    if (s + 2 < nstage) stage_store(g, lds + ((s + 2) % kStages) * kStageBytes, tid);
    if (s + 3 < nstage) stage_load(g, A, As, B, Bs, M, m0, n0, kb, ks, s + 3, tid);
    __syncthreads();
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
