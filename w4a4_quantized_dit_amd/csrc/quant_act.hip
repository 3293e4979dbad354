// Fused activation kernel: smoothing (X̂ = X · 1/λ), per-block absmax, NVFP4 (E2M1 + E4M3 block
// scale) or int4-g64 rounding with nibble packing, and the low-rank down-projection
// D = bf16(X̂)·L1 (fp32) on MFMA — one streaming read of X ("MiniMax-H3 NVFP4 — what the smoothing
// scale should be calibrated on", section "Why": the kernel sees X / λ, 16 channels per FP8
// scale; "MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)": activations quantised at run time).
//
// Work split: a block of kWaves waves owns 16 rows per wave and walks K in 256-channel
// chunks.  X is read with coalesced 16-byte loads (one load instruction covers two whole rows of
// the chunk) and re-laid through LDS so that lane (row = lane % 16, q = lane / 16) holds 64
// contiguous channels [k0 + 64q, k0 + 64q + 64): four whole NVFP4 blocks or one whole int4
// group, so every block absmax is lane-local (no cross-lane reduction).  The same registers feed
// v_mfma_f32_16x16x32_bf16: in MFMA step t the lane's k-slots 8q..8q+7 carry channels
// k0 + 64q + 8t .. +8, and the block stages the matching slice of L1 (lora_down[:, k0:k0+256])
// in LDS once for its waves.  X is prefetched one or two chunks ahead of the one processed,
// and two K groups of waves walk alternate chunks of the same rows.
// FMT 0 is NVFP4, FMT 1 int4-g64; FMT 3 / 4 are the MX formats (E8M0 scale per 32 with E2M1
// / E4M3 elements: "MiniMax-H3 — MXFP8 (weight-quantized, vLLM-Omni native layout)", section
// "Quant format"), each lane's 64 channels being two whole blocks.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

#ifndef SVDQ_QA_WAVES
#define SVDQ_QA_WAVES 4    // row waves (16 rows each) per block
#endif
constexpr int kWaves = SVDQ_QA_WAVES;
constexpr int kGroupThreads = 64 * kWaves;      // threads of one K group
constexpr int kRowsPerBlock = 16 * kWaves;
constexpr int kChunk = 256;
constexpr int kPitch = kChunk + 8;   // bf16 elements per LDS row: 528 B, conflict-free reads

// K group ks of a block processes chunks ks, ks + SPLIT, ks + 2 SPLIT, ... of its rows, so a CU
// streams SPLIT chunks of X at once; the groups' partial D are added in group order at the end
// (the quantisation blocks never straddle chunks).
template <int FMT, int NT, int SPLIT>
__global__ __launch_bounds__(kGroupThreads * SPLIT) void k_quant_act(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ lambda, const float* __restrict__ amax_p,
    const uint16_t* __restrict__ down, int r, uint8_t* __restrict__ codes,
    void* __restrict__ scales, float* __restrict__ tensor_scale, int write_g,
    float* __restrict__ D, uint32_t* __restrict__ sat) {
  constexpr int NTc = NT > 0 ? NT : 1;
  constexpr int kSplit = SPLIT;
  constexpr int kThreads = kGroupThreads * SPLIT;
  constexpr int kLPieces = NT * 16 * (kChunk / 8) / kGroupThreads;  // 16-B L1 pieces per thread
  // 1/λ for all K channels, 4 floats of padding after every 64: the four lane groups of a row
  // (64 channels apart) then read different banks instead of one
  extern __shared__ float s_inv[];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kWaves * kSplit][16 * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t s_l[kSplit][NTc * 16 * kPitch];

  float amax = 0.0f, g = 1.0f, d6 = 6.0f;
  if (FMT == 0) {
    amax = amax_p[0];
    g = amax == 0.0f ? 1.0f : amax / 2688.0f;
    d6 = 6.0f * g;
    if (write_g && blockIdx.x == 0 && threadIdx.x == 0) tensor_scale[0] = g;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rw = wave % kWaves, ks = wave / kWaves;   // row wave, K group
  const int gtid = threadIdx.x % kGroupThreads;       // thread index within the K group
  const int64_t row0 = (int64_t)blockIdx.x * kRowsPerBlock + 16 * rw;
  const int rl = lane & 15, q = lane >> 4;
  const int64_t row = row0 + rl;
  const bool valid = row < M;
  const int64_t nchunk = K / kChunk;
  const int64_t nloop = (nchunk + kSplit - 1) / kSplit;

  // coalesced X loads: instruction i covers rows 2i, 2i+1 of the wave, lane piece = lane % 32
  // (rows past M read row M-1; their results are never stored).  Byte offsets from the block's
  // first row stay below 2^31: 64 rows of at most ldx elements each, and the entry points refuse
  // ldx above 2^24.
  const int64_t blk_row = (int64_t)blockIdx.x * kRowsPerBlock;
  const int64_t blk_rows = M - blk_row < kRowsPerBlock ? M - blk_row : kRowsPerBlock;
  const __amdgpu_buffer_rsrc_t x_rsrc =
      raw_rsrc(X + blk_row * ldx, (uint32_t)(((blk_rows - 1) * ldx + K) * 2));
  uint32_t xo[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t xrow = row0 + 2 * i + (lane >> 5);
    xrow = xrow < M ? xrow : M - 1;
    xo[i] = (uint32_t)(((xrow - blk_row) * ldx + 8 * (lane & 31)) * 2);
  }
  // L1 staging within the K group: piece p = rank p / 32, channels 8 * (p % 32) .. +8 (ranks
  // past r read rank r-1 and are zeroed)
  const __amdgpu_buffer_rsrc_t l_rsrc = raw_rsrc(down, (uint32_t)(r > 0 ? r * K * 2 : 0));
  uint32_t lo[kLPieces > 0 ? kLPieces : 1];
#pragma unroll
  for (int u = 0; u < kLPieces; ++u) {
    const int p = gtid + kGroupThreads * u;
    const int n = p >> 5;
    lo[u] = (uint32_t)(((n < r ? n : r - 1) * K + 8 * (p & 31)) * 2);
  }

  f32x4_t acc[NTc];
#pragma unroll
  for (int j = 0; j < NTc; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t nsat = 0;

  // X of the group's next kAhead chunks is in flight while a chunk is processed (E2M1 formats:
  // two register sets used alternately; int4 and MXFP8, whose quantisers need more registers,
  // measured no faster with the second set); the L1 slice one chunk ahead.  The L1 loads are
  // issued before the X loads they are consumed with, because loads complete in issue order for
  // the wait counter: waiting for the L1 slice then leaves the younger X prefetch in flight.
  // Look-ahead loads past the last chunk are still issued, out of the buffers' range (zeros, no
  // memory access), so that every iteration issues the same loads and the compiler can count
  // them across the loop instead of draining the look-ahead at the loop head.
  constexpr int kAhead = (FMT == 0 || FMT == 3) ? 2 : 1;
  u32x4_t xa[8], xb[8], lr[kLPieces > 0 ? kLPieces : 1];
  auto load_x = [&](u32x4_t (&xr)[8], int64_t kc) {
    const uint32_t at = kc < nchunk ? (uint32_t)(kc * kChunk * 2) : kNoLoad;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      xr[i] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, (int)(xo[i] + at), 0, kNt));
  };
  auto load_l = [&](int64_t kc) {
    const uint32_t at = kc < nchunk ? (uint32_t)(kc * kChunk * 2) : kNoLoad;
#pragma unroll
    for (int u = 0; u < kLPieces; ++u)
      lr[u] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(l_rsrc, (int)(lo[u] + at), 0, 0));
  };
  load_l(ks);
  load_x(xa, ks);
  if (kAhead == 2) load_x(xb, ks + kSplit);
  // 1/λ of every channel, its loads issued after the first chunks' so that the two latencies
  // overlap
  if (lambda) {
    // 16 channels per thread at a time; the first batch outside any loop, so that the wait for
    // its loads does not also wait for the X look-ahead issued before it
    const __amdgpu_buffer_rsrc_t lam_rsrc = raw_rsrc(lambda, (uint32_t)(K * 4));
    auto inv_batch = [&](int64_t k0) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t k = k0 + threadIdx.x + kThreads * j;
        v[j] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       lam_rsrc, (int)(k < K ? (uint32_t)(k * 4) : kNoLoad), 0, 0));
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t k = k0 + threadIdx.x + kThreads * j;
        if (k < K) s_inv[k + 4 * (k >> 6)] = 1.0f / v[j];
      }
      // nothing of the batch is left in flight (the X look-ahead, older, has completed too);
      // stated explicitly so that the compiler's wait counting at the main loop starts clean
      wait_vmcnt<0>();
    };
    inv_batch(0);
    for (int64_t k0 = 16 * kThreads; k0 < K; k0 += 16 * kThreads) inv_batch(k0);
  } else {
    for (int64_t k = threadIdx.x; k < K; k += kThreads) s_inv[k + 4 * (k >> 6)] = 1.0f;
  }
  __syncthreads();  // s_inv complete

  auto body = [&](int64_t it, u32x4_t (&xr)[8]) {
    const int64_t kc = it * kSplit + ks;  // this group's chunk
    const bool has = kc < nchunk;
    // registers -> LDS (the previous chunk's readers finished at the loop-end barrier)
    if (has) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4_t*>(&s_x[wave][(2 * i + (lane >> 5)) * kPitch + 8 * (lane & 31)]) = xr[i];
#pragma unroll
      for (int u = 0; u < kLPieces; ++u) {
        const int p = gtid + kGroupThreads * u;
        const int n = p >> 5;
        const u32x4_t v = n < r ? lr[u] : u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(&s_l[ks][n * kPitch + 8 * (p & 31)]) = v;
      }
    }
    __syncthreads();
    load_l(kc + kSplit);
    load_x(xr, kc + kAhead * kSplit);
    if (has) {
      const int64_t kb = kc * kChunk + 64 * q;  // first channel of this lane
      const int64_t kbp = kb + 4 * (kb >> 6);   // its padded index in s_inv
      float x[64];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&s_x[wave][rl * kPitch + 64 * q + 8 * i]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t w = v[c];
          x[8 * i + 2 * c] = bf16_lo(w) * s_inv[kbp + 8 * i + 2 * c];
          x[8 * i + 2 * c + 1] = bf16_hi(w) * s_inv[kbp + 8 * i + 2 * c + 1];
        }
      }

      if (FMT == 0) {
        uint32_t cw[8];
        uint32_t sbytes = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float a = 0.0f;
#pragma unroll
          for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(x[16 * b + j]));
          nsat += (valid && a > amax) ? 1u : 0u;
          float inv;
          const uint32_t sc = nvfp4_block_scale(a, g, d6, &inv);
          float y[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) y[j] = x[16 * b + j] * inv;
          cw[2 * b] = e2m1_pack8(y);
          cw[2 * b + 1] = e2m1_pack8(y + 8);
          sbytes |= sc << (8 * b);
        }
        if (valid) {
          u32x4_t* cp = reinterpret_cast<u32x4_t*>(codes + row * (K / 2) + kb / 2);
          cp[0] = u32x4_t{cw[0], cw[1], cw[2], cw[3]};
          cp[1] = u32x4_t{cw[4], cw[5], cw[6], cw[7]};
          *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(scales) + row * (K / 16) + kb / 16) = sbytes;
        }
      } else if (FMT == 1) {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 64; ++j) a = fmaxf(a, fabsf(x[j]));
        const __half s = __float2half_rn(a / 7.0f);
        const float sf = __half2float(s);
        const float inv = sf != 0.0f ? 1.0f / sf : 0.0f;
        uint32_t cw[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          uint32_t w = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) w |= int4_code(x[8 * d + j] * inv) << (4 * j);
          cw[d] = w;
        }
        if (valid) {
          u32x4_t* cp = reinterpret_cast<u32x4_t*>(codes + row * (K / 2) + kb / 2);
          cp[0] = u32x4_t{cw[0], cw[1], cw[2], cw[3]};
          cp[1] = u32x4_t{cw[4], cw[5], cw[6], cw[7]};
          reinterpret_cast<__half*>(scales)[row * (K / 64) + kb / 64] = s;
        }
      } else if (FMT == 3 || FMT == 4) {
        // MX: the lane's 64 channels are two blocks of 32, each with an E8M0 exponent from its
        // maximum; codes of x · 2^-e (exact scaling), E2M1 (FMT 3) or E4M3 (FMT 4)
        constexpr int kEmax = FMT == 3 ? 2 : 8;
        uint32_t sb = 0;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float a = 0.0f;
#pragma unroll
          for (int j = 0; j < 32; ++j) a = fmaxf(a, fabsf(x[32 * b + j]));
          const int e = mx_exponent(a, kEmax);
          sb |= (uint32_t)(e + 127) << (8 * b);
          // each 16-byte piece of codes is encoded and stored before the next, keeping the
          // E4M3 encodings' temporaries short-lived
          if (FMT == 3) {
            uint32_t cw[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              float y[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) y[j] = __builtin_ldexpf(x[32 * b + 8 * d + j], -e);
              cw[d] = e2m1_pack8(y);
            }
            if (valid)
              reinterpret_cast<u32x4_t*>(codes + row * (K / 2) + kb / 2)[b] =
                  u32x4_t{cw[0], cw[1], cw[2], cw[3]};
          } else {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
              uint32_t cw[4];
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const float* xs = x + 32 * b + 16 * v + 4 * d;
                cw[d] = e4m3_pack4(__builtin_ldexpf(xs[0], -e), __builtin_ldexpf(xs[1], -e),
                                   __builtin_ldexpf(xs[2], -e), __builtin_ldexpf(xs[3], -e));
              }
              if (valid)
                reinterpret_cast<u32x4_t*>(codes + row * K + kb)[2 * b + v] =
                    u32x4_t{cw[0], cw[1], cw[2], cw[3]};
            }
          }
        }
        if (valid) {
          *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(scales) + row * (K / 32) +
                                       kb / 32) = (uint16_t)sb;
        }
      }

      if (NT > 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          u32x4_t av;
          av[0] = pack_bf16x2(x[8 * t + 0], x[8 * t + 1]);
          av[1] = pack_bf16x2(x[8 * t + 2], x[8 * t + 3]);
          av[2] = pack_bf16x2(x[8 * t + 4], x[8 * t + 5]);
          av[3] = pack_bf16x2(x[8 * t + 6], x[8 * t + 7]);
          const bf16x8_t a_op = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const u32x4_t bv =
                *reinterpret_cast<const u32x4_t*>(&s_l[ks][(16 * j + rl) * kPitch + 64 * q + 8 * t]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_op, __builtin_bit_cast(bf16x8_t, bv),
                                                             acc[j], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();  // the LDS chunk buffers are rewritten next iteration
  };
  if (kAhead == 2) {
    // both bodies on every path through the loop (see the look-ahead loads above)
    int64_t it = 0;
    for (; it + 1 < nloop; it += 2) {
      body(it, xa);
      body(it + 1, xb);
    }
    if (it < nloop) body(it, xa);
  } else {
    for (int64_t it = 0; it < nloop; ++it) body(it, xa);
  }

  if (NT > 0) {
    // add the other K groups' partial sums (in group order) through LDS; the X staging buffers
    // are free now
    if (kSplit > 1) {
      f32x4_t* part = reinterpret_cast<f32x4_t*>(&s_x[0][0]);  // [kSplit-1][kWaves][NT][64]
      if (ks > 0) {
#pragma unroll
        for (int j = 0; j < NT; ++j) part[(((ks - 1) * kWaves + rw) * NT + j) * 64 + lane] = acc[j];
      }
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int o = 1; o < kSplit; ++o)
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const f32x4_t v = part[(((o - 1) * kWaves + rw) * NT + j) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] += v[i];
          }
      }
    }
    // 16x16 output: lane holds rank column 16j + rl and rows 4q .. 4q+3 of the wave's 16 rows.
    if (ks == 0) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int n = 16 * j + rl;
        if (n < r) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t m = row0 + 4 * q + i;
            if (m < M) D[m * r + n] = acc[j][i];
          }
        }
      }
    }
  }
  if (FMT == 0 && sat) {
    for (int off = 32; off > 0; off >>= 1) nsat += __shfl_xor(nsat, off);
    if (lane == 0 && nsat) atomicAdd(sat, nsat);
  }
}

// Dynamic tensor amax: max over all elements of |X · 1/λ| (used when no static amax is given).
__global__ __launch_bounds__(256) void k_xhat_amax(const uint16_t* __restrict__ X, int64_t M,
                                                   int64_t K, int64_t ldx,
                                                   const float* __restrict__ lambda,
                                                   float* __restrict__ out) {
  const int64_t col = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  float m = 0.0f;
  if (col < K) {
    float inv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) inv[j] = lambda ? 1.0f / lambda[col + j] : 1.0f;
    for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(X + row * ldx + col);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        m = fmaxf(m, fabsf(bf16_lo(v[c]) * inv[2 * c]));
        m = fmaxf(m, fabsf(bf16_hi(v[c]) * inv[2 * c + 1]));
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0 && m > 0.0f) atomic_max_pos(out, m);
}

__global__ void k_set(float* t, float v) { t[0] = v; }
__global__ void k_amax_to_g(float* t) {
  const float a = t[0];
  t[0] = a == 0.0f ? 1.0f : a / 2688.0f;
}

// Static LDS of an instantiation (the X staging and L1 slices of every K group).
// dynamic LDS of the padded 1/λ table
inline size_t inv_lds_bytes(int64_t K) { return (size_t)(K + 4 * (K / 64)) * sizeof(float); }

constexpr size_t static_lds(int nt, int split) {
  return (size_t)kWaves * split * 16 * kPitch * 2 + (size_t)split * (nt > 0 ? nt : 1) * 16 * kPitch * 2;
}

template <int FMT, int NT, int SPLIT>
hipError_t launch_one(dim3 grid, size_t lds, hipStream_t s, const uint16_t* X, int64_t M, int64_t K,
                      int64_t ldx, const float* lambda, const float* amax_p, const uint16_t* down,
                      int r, uint8_t* codes, void* scales, float* ts, int write_g, float* D,
                      uint32_t* sat) {
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_quant_act<FMT, NT, SPLIT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  k_quant_act<FMT, NT, SPLIT><<<grid, dim3(kGroupThreads * SPLIT), lds, s>>>(
      X, M, K, ldx, lambda, amax_p, down, r, codes, scales, ts, write_g, D, sat);
  return hipGetLastError();
}

template <int FMT>
hipError_t dispatch(int nt, dim3 grid, size_t lds, hipStream_t s, const uint16_t* X, int64_t M,
                    int64_t K, int64_t ldx, const float* lambda, const float* amax_p,
                    const uint16_t* down, int r, uint8_t* codes, void* scales, float* ts,
                    int write_g, float* D, uint32_t* sat) {
  // two K groups when both fit in LDS (160 KB per workgroup), otherwise one
  const bool split = nt <= 2 && static_lds(nt, 2) + lds <= 160 * 1024;
#define SVDQ_QA_CASE(NTV)                                                                  \
  case NTV:                                                                                \
    if constexpr (NTV <= 2) {                                                              \
      if (split)                                                                           \
        return launch_one<FMT, NTV, 2>(grid, lds, s, X, M, K, ldx, lambda, amax_p, down, r, \
                                       codes, scales, ts, write_g, D, sat);                \
    }                                                                                      \
    return launch_one<FMT, NTV, 1>(grid, lds, s, X, M, K, ldx, lambda, amax_p, down, r,    \
                                   codes, scales, ts, write_g, D, sat);
  switch (nt) {
    SVDQ_QA_CASE(0)
    SVDQ_QA_CASE(1)
    SVDQ_QA_CASE(2)
    SVDQ_QA_CASE(3)
    SVDQ_QA_CASE(4)
    SVDQ_QA_CASE(5)
    SVDQ_QA_CASE(6)
    SVDQ_QA_CASE(7)
    SVDQ_QA_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef SVDQ_QA_CASE
}

}  // namespace

size_t quant_act_lds_bytes(int64_t K, int64_t r) {
  const int nt = (int)((r + 15) / 16);
  const size_t dyn = inv_lds_bytes(K);
  const bool split = nt <= 2 && static_lds(nt, 2) + dyn <= 160 * 1024;
  return static_lds(nt, split ? 2 : 1) + dyn;
}

hipError_t launch_quant_act(int fmt, const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                            const float* lambda, const float* act_amax, const uint16_t* down,
                            int64_t r, uint8_t* codes, void* scales, float* tensor_scale,
                            float* D, uint32_t* sat, hipStream_t s) {
  const int nt = (int)((r + 15) / 16);
  const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock));
  const size_t lds = inv_lds_bytes(K);
  if (fmt == 1)
    return dispatch<1>(nt, grid, lds, s, X, M, K, ldx, lambda, nullptr, down, (int)r, codes,
                       scales, nullptr, 0, D, nullptr);
  if (fmt == 2)  // MXFP4
    return dispatch<3>(nt, grid, lds, s, X, M, K, ldx, lambda, nullptr, down, (int)r, codes,
                       scales, nullptr, 0, D, nullptr);
  if (fmt == 3)  // MXFP8
    return dispatch<4>(nt, grid, lds, s, X, M, K, ldx, lambda, nullptr, down, (int)r, codes,
                       scales, nullptr, 0, D, nullptr);
  const float* amax_p = act_amax;
  int write_g = 1;
  if (!act_amax) {
    // Dynamic pre-pass: tensor_scale holds max|X̂| until the final conversion to g.
    k_set<<<1, 1, 0, s>>>(tensor_scale, 0.0f);
    const dim3 g2((unsigned)((K / 8 + 255) / 256), (unsigned)(M < 1024 ? M : 1024));
    k_xhat_amax<<<g2, dim3(256), 0, s>>>(X, M, K, ldx, lambda, tensor_scale);
    amax_p = tensor_scale;
    write_g = 0;
  }
  hipError_t e = dispatch<0>(nt, grid, lds, s, X, M, K, ldx, lambda, amax_p, down, (int)r, codes,
                             scales, tensor_scale, write_g, D, sat);
  if (e != hipSuccess) return e;
  if (!act_amax) {
    k_amax_to_g<<<1, 1, 0, s>>>(tensor_scale);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace svdq
