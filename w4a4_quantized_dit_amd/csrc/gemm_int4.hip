// int4-g64 W4A4 GEMM: exact integer-code MFMA per 64-group with fp32 rescaling.
//   Y = bf16( Σ_groups s_a[m,g]·s_w[n,g] · Σ_{k∈g} c_a·c_w  +  D·L2 )
// ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)": int4 codes for weights and per-token
// activations; the per-group fp16 scales of the int4 workload.)
//
// Codes are expanded to int8 with a shift (a nibble in the high half of a byte is 16·c as a
// signed byte), so one v_mfma_i32_32x32x32_i8 pair covers a 64-group of one 32x32 tile with
// 256·Σ c_a·c_w, exact in int32.  Each group result is converted once and accumulated with its
// scale product s_a·s_w/256 in fp32: three VALU operations per output element and group, which
// is more issue time than the two MFMAs take, so the kernel is built to keep the VALU busy.
//
// Workgroup tile 256 x 256 with 8 waves (2 per SIMD, so one wave's VALU work overlaps the
// other's MFMA and memory waits), each wave 128 x 64 (4 x 2 tiles of 32x32), fp32 accumulators
// in VGPRs.  K advances two groups per stage; codes and scales go global -> registers -> LDS
// through three LDS buffers (one barrier per stage).  The fp16 scales are converted to fp32
// once, when a stage is written to LDS, with the weight scale pre-multiplied by 1/256.
// K mapping: in a 64-group, lane (row = lane % 32, h = lane / 32) holds elements
// [32h, 32h + 32) of its row (16 bytes of codes); the weight operand uses the same mapping, so
// every byte of an A operand meets the byte of equal K in the W operand.
#include "device.h"
#include "gemm_common.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 512;
constexpr int kBM = 256, kBN = 256;
constexpr int kGroupsPerStage = 2;                 // K = 128 per stage
constexpr int kRowBytes = kGroupsPerStage * 32;    // 64 bytes of codes per row per stage
constexpr int kRowPitch = kRowBytes + 16;          // padded pitch: conflict-free 16-byte reads
constexpr int kStages = 3;
constexpr int kCodeBuf = kBM * kRowPitch;          // per operand per stage
constexpr int kScaleBuf = kGroupsPerStage * kBM * 4;  // fp32 scales per operand per stage
constexpr int kStageBytes = 2 * kCodeBuf + 2 * kScaleBuf;

struct StageRegs {
  u32x4_t a[2], b[2];  // 2 x 16 B of codes per operand per thread
  uint32_t s;          // two fp16 scales: threads 0..255 of an A row, 256..511 of a W row
};

__device__ __forceinline__ void stage_load(StageRegs& g, const uint8_t* __restrict__ A,
                                           const __half* __restrict__ As,
                                           const uint8_t* __restrict__ B,
                                           const __half* __restrict__ Bs, int64_t M, int64_t m0,
                                           int64_t n0, int64_t kb, int64_t ng, int64_t stage,
                                           int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + kThreads * j;  // chunk id: row = c / 4, part = c % 4
    const int row = c >> 2, part = c & 3;
    int64_t ar = m0 + row;
    ar = ar < M ? ar : M - 1;
    g.a[j] = *reinterpret_cast<const u32x4_t*>(A + ar * kb + stage * kRowBytes + part * 16);
    g.b[j] = *reinterpret_cast<const u32x4_t*>(B + (n0 + row) * kb + stage * kRowBytes + part * 16);
  }
  const int64_t g0 = stage * kGroupsPerStage;
  if (tid < kBM) {
    int64_t ar = m0 + tid;
    ar = ar < M ? ar : M - 1;
    g.s = *reinterpret_cast<const uint32_t*>(As + ar * ng + g0);
  } else {
    g.s = *reinterpret_cast<const uint32_t*>(Bs + (n0 + tid - kBM) * ng + g0);
  }
}

__device__ __forceinline__ void stage_store(const StageRegs& g, uint8_t* lds, int tid) {
  uint8_t* la = lds;
  uint8_t* lb = lds + kCodeBuf;
  float* ls = reinterpret_cast<float*>(lds + 2 * kCodeBuf);  // [operand][group][row]
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + kThreads * j;
    const int row = c >> 2, part = c & 3;
    *reinterpret_cast<u32x4_t*>(la + row * kRowPitch + part * 16) = g.a[j];
    *reinterpret_cast<u32x4_t*>(lb + row * kRowPitch + part * 16) = g.b[j];
  }
  const bool w = tid >= kBM;
  const int row = w ? tid - kBM : tid;
  const float mul = w ? 0.00390625f : 1.0f;  // 1/256 undoes the two x16 code shifts
  const __half lo = __ushort_as_half((unsigned short)(g.s & 0xFFFFu));
  const __half hi = __ushort_as_half((unsigned short)(g.s >> 16));
  float* dst = ls + (w ? kGroupsPerStage * kBM : 0) + row;
  dst[0] = __half2float(lo) * mul;
  dst[kBM] = __half2float(hi) * mul;
}

// 8 int4 nibbles -> two dwords of int8 (16·c): even elements, odd elements.
__device__ __forceinline__ void expand8(uint32_t w, uint32_t& even, uint32_t& odd) {
  even = (w << 4) & 0xF0F0F0F0u;
  odd = w & 0xF0F0F0F0u;
}

struct Operand {
  i32x4_t lo, hi;  // k-slots of the two MFMAs of a group
};

__device__ __forceinline__ Operand expand_operand(u32x4_t raw) {
  uint32_t v[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) expand8(raw[d], v[2 * d], v[2 * d + 1]);
  Operand o;
  o.lo = i32x4_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
  o.hi = i32x4_t{(int)v[4], (int)v[5], (int)v[6], (int)v[7]};
  return o;
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_int4(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
    const __half* __restrict__ As, const uint8_t* __restrict__ B,
    const __half* __restrict__ Bs, const float* __restrict__ D,
    const uint16_t* __restrict__ up, int r, uint16_t* __restrict__ Y, int64_t ldy) {
  constexpr int FM = 4, FN = 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStageBytes];
  const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = N / kBN;
  int64_t tm, tn;
  if (!tile_of_block(tiles_m, tiles_n, tm, tn)) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves over the 256 x 256 tile
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int64_t m_base = m0 + wm * 128, n_base = n0 + wn * 64;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2, ng = K / 64;
  const int64_t nstage = K / (64 * kGroupsPerStage);
  const int a_off = (wm * 128 + r32) * kRowPitch + 16 * h;
  const int b_off = kCodeBuf + (wn * 64 + r32) * kRowPitch + 16 * h;
  const int sa_off = wm * 128 + 4 * h;                      // float index in the A scale block
  const int sw_off = kGroupsPerStage * kBM + wn * 64 + r32;  // float index of the W scales

  StageRegs g;
  stage_load(g, A, As, B, Bs, M, m0, n0, kb, ng, 0, tid);
  f32x16_t acc[FM][FN];
  gemm_lowrank_init<FM, FN>(acc, 1.0f, M, m_base, n_base, r32, h, D, up, r);
  stage_store(g, lds, tid);
  if (nstage > 1) {
    stage_load(g, A, As, B, Bs, M, m0, n0, kb, ng, 1, tid);
    stage_store(g, lds + kStageBytes, tid);
  }
  if (nstage > 2) stage_load(g, A, As, B, Bs, M, m0, n0, kb, ng, 2, tid);
  __syncthreads();

  for (int64_t s = 0; s < nstage; ++s) {
    const uint8_t* buf = lds + (s % kStages) * kStageBytes;
    const float* ls = reinterpret_cast<const float*>(buf + 2 * kCodeBuf);
#pragma unroll 1
    for (int gg = 0; gg < kGroupsPerStage; ++gg) {
      Operand bop[FN];
      float sw[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        bop[j] = expand_operand(
            *reinterpret_cast<const u32x4_t*>(buf + b_off + j * 32 * kRowPitch + 32 * gg));
        sw[j] = ls[sw_off + gg * kBM + 32 * j];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const Operand aop = expand_operand(
            *reinterpret_cast<const u32x4_t*>(buf + a_off + i * 32 * kRowPitch + 32 * gg));
        // activation scales of the accumulator rows (e/4)*8 + 4h + e%4 of this tile row
        float sa[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4_t v =
              *reinterpret_cast<const f32x4_t*>(ls + gg * kBM + sa_off + 32 * i + 8 * q);
#pragma unroll
          for (int t = 0; t < 4; ++t) sa[4 * q + t] = v[t];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          i32x16_t p = {};
          p = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop.lo, bop[j].lo, p, 0, 0, 0);
          p = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop.hi, bop[j].hi, p, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 16; ++e)
            acc[i][j][e] = __builtin_fmaf((float)p[e], sa[e] * sw[j], acc[i][j][e]);
        }
      }
    }
    if (s + 2 < nstage) stage_store(g, lds + ((s + 2) % kStages) * kStageBytes, tid);
    if (s + 3 < nstage) stage_load(g, A, As, B, Bs, M, m0, n0, kb, ng, s + 3, tid);
    __syncthreads();
  }

  // the loop ended with a barrier after the last LDS reads: the stage buffers are free for the
  // output staging (each wave its own 16 KB)
  static_assert(8 * gemm_store_bytes<FM, FN>() <= kStages * kStageBytes, "output staging fits");
  gemm_store<FM, FN>(acc, 1.0f, lds + wave * gemm_store_bytes<FM, FN>(), lane, M, N, m_base,
                     n_base, nullptr, nullptr, Y, ldy);
}

}  // namespace

hipError_t launch_gemm_int4(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const void* a_scales, const uint8_t* w_codes, const void* w_scales,
                            const float* D, const uint16_t* up, int64_t r, uint16_t* Y,
                            int64_t ldy, hipStream_t s) {
  const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = N / kBN;
  k_gemm_int4<<<dim3(grid_of_tiles(tiles_m, tiles_n)), dim3(kThreads), 0, s>>>(
      M, N, K, a_codes, reinterpret_cast<const __half*>(a_scales), w_codes,
      reinterpret_cast<const __half*>(w_scales), D, up, (int)r, Y, ldy);
  return hipGetLastError();
}

}  // namespace svdq
