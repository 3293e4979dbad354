// DeltaQuant variant ("DeltaQuant on MiniMax-H3": a cube of tokens is represented by one core
// plus per-token deltas; the delta's NVFP4 tensor scale comes from the bound
// |x − core| ≤ 2·max|x| ("The activation scale bound held"); the core branch stays on a 16-bit
// path ("Deviations from the paper")).
//
// k_delta_act: one workgroup per cube (persistent over cubes).  The cube's rows are smoothed
// (X̂ = X · 1/λ), summed in ascending row order in fp32 and divided by the member count; the
// core row is kept in LDS, quantised to E4M3 with a per-row scale amax/448, and every member's
// delta X̂ − core (unquantised core) is quantised to NVFP4 with tensor amax 2·act_amax.  Finally
// the members' low-rank activations D = bf16(X̂)·L1 are formed on MFMA with the member rows as
// the 16 row slots of v_mfma_f32_16x16x32_bf16.
//
// k_gemm_core: core_out[c, n] = s_c · g_w · Σ_k e4m3(core[c, k]) · (c_w·s_w)[n, k] on fp16 MFMA:
// E4M3 values and the NVFP4 weight products are exact in fp16.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxCube = 16;

__global__ __launch_bounds__(kThreads) void k_delta_act(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ lambda, const float* __restrict__ act_amax,
    const int32_t* __restrict__ cube_ptr, const int32_t* __restrict__ cube_rows, int64_t n_cubes,
    const uint16_t* __restrict__ down, int r, uint8_t* __restrict__ core_codes,
    float* __restrict__ core_scale, uint8_t* __restrict__ dcodes, uint8_t* __restrict__ dscales,
    float* __restrict__ g_delta, float* __restrict__ D, uint32_t* __restrict__ sat) {
  extern __shared__ float s_dyn[];
  float* s_inv = s_dyn;       // [K]
  float* s_core = s_dyn + K;  // [K]
  __shared__ float s_red[kThreads / 64];
  __shared__ int s_rows[kMaxCube];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int64_t k = tid; k < K; k += kThreads) s_inv[k] = lambda ? 1.0f / lambda[k] : 1.0f;
  const float amax_t = 2.0f * act_amax[0];
  const float g = amax_t == 0.0f ? 1.0f : amax_t / 2688.0f;
  const float d6 = 6.0f * g;
  if (blockIdx.x == 0 && tid == 0) g_delta[0] = g;
  uint32_t nsat = 0;

  for (int64_t c = blockIdx.x; c < n_cubes; c += gridDim.x) {
    const int p0 = cube_ptr[c];
    int n = cube_ptr[c + 1] - p0;
    n = n < 0 ? 0 : (n > kMaxCube ? kMaxCube : n);
    __syncthreads();  // the previous cube's LDS readers are done (and s_inv is complete)
    if (n == 0) continue;  // uniform across the block
    if (tid < n) {
      int m = cube_rows[p0 + tid];
      s_rows[tid] = m < 0 ? 0 : (m < M ? m : (int)M - 1);
    }
    __syncthreads();

    // core: ascending fp32 sum of the members' X̂, divided by the count; row amax
    float amax = 0.0f;
    for (int64_t k = 8 * tid; k < K; k += 8 * kThreads) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < n; ++j) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(X + (int64_t)s_rows[j] * ldx + k);
#pragma unroll
        for (int c2 = 0; c2 < 4; ++c2) {
          acc[2 * c2] += bf16_lo(v[c2]) * s_inv[k + 2 * c2];
          acc[2 * c2 + 1] += bf16_hi(v[c2]) * s_inv[k + 2 * c2 + 1];
        }
      }
      const float fn = (float)n;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float cv = acc[e] / fn;
        s_core[k + e] = cv;
        amax = fmaxf(amax, fabsf(cv));
      }
    }
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (lane == 0) s_red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float sc = amax / 448.0f;
    const float inv_c = sc != 0.0f ? 1.0f / sc : 0.0f;
    if (tid == 0) core_scale[c] = sc;

    // FP8 core codes: sign | E4M3(|core| · 1/s_c)
    for (int64_t k = 8 * tid; k < K; k += 8 * kThreads) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = s_core[k + e];
        float val;
        const uint32_t code = e4m3_encode_pos(fabsf(v) * inv_c, &val) | (__builtin_signbit(v) ? 0x80u : 0u);
        if (e < 4)
          lo |= code << (8 * e);
        else
          hi |= code << (8 * (e - 4));
      }
      *reinterpret_cast<uint2*>(core_codes + c * K + k) = uint2{lo, hi};
    }

    // deltas: one NVFP4 block (16 channels of one member) per task
    const int64_t nblk = K / NVFP4_BLOCK;
    for (int64_t task = tid; task < (int64_t)n * nblk; task += kThreads) {
      const int j = (int)(task / nblk);
      const int64_t b = task % nblk, k0 = b * NVFP4_BLOCK;
      const int64_t m = s_rows[j];
      const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(X + m * ldx + k0);
      const u32x4_t v0 = xp[0], v1 = xp[1];
      const uint32_t w[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      float d[16];
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        d[2 * e] = bf16_lo(w[e]) * s_inv[k0 + 2 * e] - s_core[k0 + 2 * e];
        d[2 * e + 1] = bf16_hi(w[e]) * s_inv[k0 + 2 * e + 1] - s_core[k0 + 2 * e + 1];
        a = fmaxf(a, fmaxf(fabsf(d[2 * e]), fabsf(d[2 * e + 1])));
      }
      nsat += a > amax_t ? 1u : 0u;
      float inv;
      const uint32_t scode = nvfp4_block_scale(a, g, d6, &inv);
      float y[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] = d[e] * inv;
      *reinterpret_cast<uint2*>(dcodes + m * (K / 2) + k0 / 2) = uint2{e2m1_pack8(y), e2m1_pack8(y + 8)};
      dscales[m * nblk + b] = (uint8_t)scode;
    }

    // low-rank activations of the members: D = bf16(X̂)·L1, rank tiles split over the waves
    if (r > 0) {
      const int slot = lane & 15, q = lane >> 4;
      const bool live = slot < n;
      const int64_t xm = s_rows[live ? slot : 0];
      const int ntile = (r + 15) / 16;
      for (int j = wave; j < ntile; j += kThreads / 64) {
        const int rank = 16 * j + slot;
        const uint16_t* dp = down + (int64_t)(rank < r ? rank : r - 1) * K;
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int nk = (int)(K / 32);  // a multiple of 8

        for (int it = 0; it < nk; ++it) {
          const int64_t kk = (int64_t)it * 32 + 8 * q;
          const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(X + xm * ldx + kk);
          u32x4_t av;
#pragma unroll
          for (int c2 = 0; c2 < 4; ++c2) {
            const float x0 = live ? bf16_lo(xv[c2]) * s_inv[kk + 2 * c2] : 0.0f;
            const float x1 = live ? bf16_hi(xv[c2]) * s_inv[kk + 2 * c2 + 1] : 0.0f;
            av[c2] = pack_bf16x2(x0, x1);
          }
          u32x4_t bv = *reinterpret_cast<const u32x4_t*>(dp + kk);
          bv = rank < r ? bv : u32x4_t{0u, 0u, 0u, 0u};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                        __builtin_bit_cast(bf16x8_t, bv), acc, 0,
                                                        0, 0);
        }
        // 16x16 output: lane holds rank column 16j + slot and member slots 4q .. 4q+3
        if (rank < r) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ms = 4 * q + i;
            if (ms < n) D[(int64_t)s_rows[ms] * r + rank] = acc[i];
          }
        }
      }
    }
  }
  if (sat) {
    for (int off = 32; off > 0; off >>= 1) nsat += __shfl_xor(nsat, off);
    if (lane == 0 && nsat) atomicAdd(sat, nsat);
  }
}

// core_out GEMM: workgroup tile 128 cubes x 128 columns, 4 waves of 64 x 64 (2 x 2 tiles of
// 32x32).  K mapping: in a 64-element chunk, lane (row = lane % 32, h = lane / 32) holds elements
// [32h, 32h + 32); MFMA step t takes [8t, 8t + 8), for the core and the weight alike.
__global__ __launch_bounds__(kThreads) void k_gemm_core(
    int64_t n_cubes, int64_t N, int64_t K, const uint8_t* __restrict__ cc,
    const float* __restrict__ cs, const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs,
    const float* __restrict__ g_w, float* __restrict__ out) {
  constexpr int FM = 2, FN = 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t c_base = (int64_t)blockIdx.y * 128 + wm * 64;
  const int64_t n_base = (int64_t)blockIdx.x * 128 + wn * 64;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2, ks = K / 16;
  const uint8_t* pa[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    int64_t c = c_base + 32 * i + r32;
    c = c < n_cubes ? c : n_cubes - 1;
    pa[i] = cc + c * K + 32 * h;
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

  for (int64_t c0 = 0; c0 < K / 64; ++c0) {
    u32x4_t ca[FM][2], cbv[FN];
    uint32_t sbv[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      ca[i][0] = reinterpret_cast<const u32x4_t*>(pa[i] + c0 * 64)[0];
      ca[i][1] = reinterpret_cast<const u32x4_t*>(pa[i] + c0 * 64)[1];
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      cbv[j] = *reinterpret_cast<const u32x4_t*>(pb[j] + c0 * 32);
      sbv[j] = *reinterpret_cast<const uint32_t*>(psb[j] + c0 * 4);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8_t a_op[FM], b_op[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        // elements 8t .. 8t+7 of the lane's 32 E4M3 bytes: dwords 2t, 2t+1
        const uint32_t w0 = ca[i][t >> 1][2 * (t & 1)], w1 = ca[i][t >> 1][2 * (t & 1) + 1];
        const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
        const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
        const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
        const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
        a_op[i] = f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint32_t s2 = (sbv[j] >> (16 * h)) & 0xFFFFu;  // blocks 2h, 2h+1 of the chunk
        const f16x2_t p = e4m3x2_to_f16x2(s2);
        b_op[j] = dequant8(cbv[j][t], (t >> 1) ? f16x2_t{p[1], p[1]} : f16x2_t{p[0], p[0]});
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_op[i], b_op[j], acc[i][j], 0, 0, 0);
    }
  }
  const float gw = g_w[0];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t c = c_base + 32 * i + (e >> 2) * 8 + 4 * h + (e & 3);
      if (c < n_cubes) {
        const float f = cs[c] * gw;
#pragma unroll
        for (int j = 0; j < FN; ++j) out[c * N + n_base + 32 * j + r32] = acc[i][j][e] * f;
      }
    }
  }
}

}  // namespace

hipError_t launch_delta_quant_act(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                  const float* lambda, const float* act_amax,
                                  const int32_t* cube_ptr, const int32_t* cube_rows,
                                  int64_t n_cubes, const uint16_t* down, int64_t r,
                                  uint8_t* core_codes, float* core_scale, uint8_t* delta_codes,
                                  uint8_t* delta_scales, float* g_delta, float* D, uint32_t* sat,
                                  hipStream_t s) {
  const size_t lds = (size_t)2 * K * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_delta_act),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = n_cubes < 2048 ? n_cubes : 2048;
  k_delta_act<<<dim3((unsigned)blocks), dim3(kThreads), lds, s>>>(
      X, M, K, ldx, lambda, act_amax, cube_ptr, cube_rows, n_cubes, down, (int)r, core_codes,
      core_scale, delta_codes, delta_scales, g_delta, D, sat);
  return hipGetLastError();
}

hipError_t launch_gemm_core(int64_t n_cubes, int64_t N, int64_t K, const uint8_t* core_codes,
                            const float* core_scale, const uint8_t* w_codes,
                            const uint8_t* w_scales, const float* g_w, float* core_out,
                            hipStream_t s) {
  const dim3 grid((unsigned)(N / 128), (unsigned)((n_cubes + 127) / 128));
  k_gemm_core<<<grid, dim3(kThreads), 0, s>>>(n_cubes, N, K, core_codes, core_scale, w_codes,
                                               w_scales, g_w, core_out);
  return hipGetLastError();
}

}  // namespace svdq
