// DeltaQuant variant ("DeltaQuant on MiniMax-H3": a cube of tokens is represented by one core
// plus per-token deltas; the delta's NVFP4 tensor scale comes from the bound
// |x − core| ≤ 2·max|x| ("The activation scale bound held"); the core branch stays on a 16-bit
// path ("Deviations from the paper")).
//
// k_delta_act: one workgroup per cube (at most 16 member rows), walking K in chunks of 256
// channels.  Per chunk the members' smoothed rows X̂ = X · 1/λ are staged in LDS (fp32, read from
// HBM once, coalesced, the next chunk's loads in flight while this one is processed); a thread
// per channel sums the members in ascending row order in fp32 and divides by the member count
// (the core row stays in LDS); a thread per member row and 16-channel block quantises the delta
// X̂ − core (unquantised core) to NVFP4 with tensor amax 2·act_amax.  After the last chunk the
// core row's amax gives its E4M3 scale amax/448 and the core codes are written from LDS.  The
// workgroup needs about 4·K + 18 KB of LDS, so several cubes are resident per CU.
// The members' low-rank activations D = bf16(X̂)·L1 come from the activation kernel's D-only
// mode, whose 64-row tiles share each slice of L1 across many rows.
// k_gemm_core: core_out[c, n] = s_c · g_w · Σ_k e4m3(core[c, k]) · (c_w·s_w)[n, k] on fp16 MFMA:
// E4M3 values and the NVFP4 weight products are exact in fp16.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 256;       // k_gemm_core and k_delta_act: 4 waves
constexpr int kMaxCube = 16;        // rows per cube (svdq_cube_geometry guarantees it)
constexpr int kChunk = 256;         // channels per chunk
constexpr int kStashPitch = kChunk + 4;  // floats per staged row (padded)

__global__ __launch_bounds__(kThreads) void k_delta_act(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ lambda, const float* __restrict__ act_amax,
    const int32_t* __restrict__ cube_ptr, const int32_t* __restrict__ cube_rows,
    uint8_t* __restrict__ core_codes, float* __restrict__ core_scale,
    uint8_t* __restrict__ dcodes, uint8_t* __restrict__ dscales, float* __restrict__ g_delta,
    uint32_t* __restrict__ sat) {
  extern __shared__ __attribute__((aligned(16))) float s_dyn[];
  float* s_core = s_dyn;                          // [K] fp32 core row
  float* s_x = s_dyn + K;                         // [kMaxCube][kStashPitch] staged X̂ chunk
  float* s_inv = s_x + kMaxCube * kStashPitch;    // [2][kChunk] 1/λ of this and the next chunk
  __shared__ int s_rows[kMaxCube];
  __shared__ float s_red[kThreads / 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t c = blockIdx.x;
  const int p0 = cube_ptr[c];
  int n = cube_ptr[c + 1] - p0;
  n = n < 0 ? 0 : (n > kMaxCube ? kMaxCube : n);
  if (n == 0) return;  // uniform: nothing to do for an empty cube
  if (tid < n) {
    const int m = cube_rows[p0 + tid];
    s_rows[tid] = m < 0 ? 0 : (m < M ? m : (int)M - 1);
  }
  s_inv[tid] = lambda ? 1.0f / lambda[tid] : 1.0f;
  const float amax_t = 2.0f * act_amax[0];
  const float g = amax_t == 0.0f ? 1.0f : amax_t / 2688.0f;
  const float d6 = 6.0f * g;
  if (c == 0 && tid == 0) g_delta[0] = g;
  __syncthreads();

  // staging: rows tid/32 and tid/32 + 8, channels 8·(tid%32) .. +8 (rows past n repeat row n-1
  // and are not stored)
  const int g8 = tid & 31;
  const uint16_t* xg[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = (tid >> 5) + 8 * t;
    xg[t] = X + (int64_t)s_rows[row < n ? row : n - 1] * ldx + 8 * g8;
  }
  u32x4_t xr[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) xr[t] = *reinterpret_cast<const u32x4_t*>(xg[t]);
  const int dl_row = tid >> 4, dl_blk = tid & 15;  // delta: one 16-channel block of one row
  float core_amax = 0.0f;
  uint32_t nsat = 0;

  for (int64_t k0 = 0; k0 < K; k0 += kChunk) {
    const int buf = (int)((k0 / kChunk) & 1);
    const float* inv = s_inv + buf * kChunk;
    // 1. stage X̂ (fp32) and issue the next chunk's loads
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = (tid >> 5) + 8 * t;
      if (row < n) {
        const f32x4_t i0 = *reinterpret_cast<const f32x4_t*>(inv + 8 * g8);
        const f32x4_t i1 = *reinterpret_cast<const f32x4_t*>(inv + 8 * g8 + 4);
        const u32x4_t v = xr[t];
        f32x4_t x0, x1;
        x0[0] = bf16_lo(v[0]) * i0[0]; x0[1] = bf16_hi(v[0]) * i0[1];
        x0[2] = bf16_lo(v[1]) * i0[2]; x0[3] = bf16_hi(v[1]) * i0[3];
        x1[0] = bf16_lo(v[2]) * i1[0]; x1[1] = bf16_hi(v[2]) * i1[1];
        x1[2] = bf16_lo(v[3]) * i1[2]; x1[3] = bf16_hi(v[3]) * i1[3];
        float* dst = s_x + row * kStashPitch + 8 * g8;
        *reinterpret_cast<f32x4_t*>(dst) = x0;
        *reinterpret_cast<f32x4_t*>(dst + 4) = x1;
      }
    }
    if (k0 + kChunk < K) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        xr[t] = *reinterpret_cast<const u32x4_t*>(xg[t] + k0 + kChunk);
      s_inv[(buf ^ 1) * kChunk + tid] = lambda ? 1.0f / lambda[k0 + kChunk + tid] : 1.0f;
    }
    __syncthreads();

    // 2. core channel: ascending fp32 sum over the members, divided by the count
    {
      float acc = 0.0f;
      for (int j = 0; j < n; ++j) acc += s_x[j * kStashPitch + tid];
      const float cv = acc / (float)n;
      s_core[k0 + tid] = cv;
      core_amax = fmaxf(core_amax, fabsf(cv));
    }
    __syncthreads();

    // 3. delta block: X̂ − core, NVFP4 with the static tensor amax
    if (dl_row < n) {
      const float* xrow = s_x + dl_row * kStashPitch + 16 * dl_blk;
      const float* crow = s_core + k0 + 16 * dl_blk;
      float d[16];
      float a = 0.0f;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4_t xq = *reinterpret_cast<const f32x4_t*>(xrow + 4 * e4);
        const f32x4_t cq = *reinterpret_cast<const f32x4_t*>(crow + 4 * e4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          d[4 * e4 + e] = xq[e] - cq[e];
          a = fmaxf(a, fabsf(d[4 * e4 + e]));
        }
      }
      nsat += a > amax_t ? 1u : 0u;
      float sinv;
      const uint32_t scode = nvfp4_block_scale(a, g, d6, &sinv);
      float y[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) y[e] = d[e] * sinv;
      const int64_t m = s_rows[dl_row];
      const int64_t kq = k0 + 16 * dl_blk;
      *reinterpret_cast<uint2*>(dcodes + m * (K / 2) + kq / 2) =
          uint2{e2m1_pack8(y), e2m1_pack8(y + 8)};
      dscales[m * (K / 16) + kq / 16] = (uint8_t)scode;
    }
    __syncthreads();  // the staged rows are rewritten by the next chunk
  }

  // core scale and FP8 codes: sign | E4M3(|core| · 1/s_c), 8 channels per thread per step
  for (int off = 32; off > 0; off >>= 1) core_amax = fmaxf(core_amax, __shfl_xor(core_amax, off));
  if (lane == 0) s_red[wave] = core_amax;
  __syncthreads();
  const float am = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float sc = am / 448.0f;
  const float inv_c = sc != 0.0f ? 1.0f / sc : 0.0f;
  if (tid == 0) core_scale[c] = sc;
  for (int64_t k = 8 * tid; k < K; k += 8 * kThreads) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = s_core[k + e];
      float val;
      const uint32_t code =
          e4m3_encode_pos(fabsf(v) * inv_c, &val) | (__builtin_signbit(v) ? 0x80u : 0u);
      if (e < 4)
        lo |= code << (8 * e);
      else
        hi |= code << (8 * (e - 4));
    }
    *reinterpret_cast<uint2*>(core_codes + c * K + k) = uint2{lo, hi};
  }
  if (sat) {
    for (int off = 32; off > 0; off >>= 1) nsat += __shfl_xor(nsat, off);
    if (lane == 0 && nsat) atomicAdd(sat, nsat);
  }
}

// core_out GEMM: workgroup tile 128 cubes x 128 columns, 4 waves of 64 x 64 (2 x 2 tiles of
// 32x32).  K mapping: in a 64-element chunk, lane (row = lane % 32, h = lane / 32) holds elements
// [32h, 32h + 32); MFMA step t takes [8t, 8t + 8), for the core and the weight alike.
// Each chunk's operands are converted to fp16 once per workgroup (thread t: row t / 2, elements
// [32 (t % 2), +32) of the core tile and of the weight tile) into a double-buffered LDS tile,
// and the waves read ready fragments; the raw bytes of chunk c + 2 are loaded while chunk c is
// multiplied.  Rows are 72 halves apart (144 B), which keeps both the 16-byte conversion stores
// and the 16-byte fragment reads free of bank conflicts.
constexpr int kCorePitch = 72;  // halves per LDS row

__global__ __launch_bounds__(kThreads) void k_gemm_core(
    int64_t n_cubes, int64_t N, int64_t K, const uint8_t* __restrict__ cc,
    const float* __restrict__ cs, const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs,
    const float* __restrict__ g_w, float* __restrict__ out) {
  constexpr int FM = 2, FN = 2;
  __shared__ __attribute__((aligned(16))) _Float16 s_a[2][128 * kCorePitch];
  __shared__ __attribute__((aligned(16))) _Float16 s_b[2][128 * kCorePitch];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t c_base = (int64_t)blockIdx.y * 128 + wm * 64;
  const int64_t n_base = (int64_t)blockIdx.x * 128 + wn * 64;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2, ks = K / 16;
  const int64_t nchunk = K / 64;

  // conversion role of this thread
  const int crow = tid >> 1, chh = tid & 1;
  int64_t ac = (int64_t)blockIdx.y * 128 + crow;
  ac = ac < n_cubes ? ac : n_cubes - 1;
  const uint8_t* pa = cc + ac * K + 32 * chh;
  const int64_t bcol = (int64_t)blockIdx.x * 128 + crow;
  const uint8_t* pb = B + bcol * kb + 16 * chh;
  const uint8_t* psb = Bs + bcol * ks;

  u32x4_t ra[2], rb;
  uint32_t rs;
  auto load_raw = [&](int64_t c0) {
    ra[0] = reinterpret_cast<const u32x4_t*>(pa + c0 * 64)[0];
    ra[1] = reinterpret_cast<const u32x4_t*>(pa + c0 * 64)[1];
    rb = *reinterpret_cast<const u32x4_t*>(pb + c0 * 32);
    rs = *reinterpret_cast<const uint32_t*>(psb + c0 * 4);
  };
  auto convert = [&](int buf) {
    _Float16* da = &s_a[buf][crow * kCorePitch + 32 * chh];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w0 = ra[q >> 1][2 * (q & 1)], w1 = ra[q >> 1][2 * (q & 1) + 1];
      const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
      const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
      const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
      const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
      *reinterpret_cast<f16x8_t*>(da + 8 * q) =
          f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
    const f16x2_t p = e4m3x2_to_f16x2((rs >> (16 * chh)) & 0xFFFFu);  // blocks 2hh, 2hh+1
    _Float16* db = &s_b[buf][crow * kCorePitch + 32 * chh];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f16x8_t*>(db + 8 * q) =
          dequant8(rb[q], (q >> 1) ? f16x2_t{p[1], p[1]} : f16x2_t{p[0], p[0]});
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  load_raw(0);
  convert(0);
  if (nchunk > 1) load_raw(1);
  __syncthreads();
  for (int64_t c0 = 0; c0 < nchunk; ++c0) {
    const int buf = (int)(c0 & 1);
    const _Float16* fa = &s_a[buf][(wm * 64 + r32) * kCorePitch + 32 * h];
    const _Float16* fb = &s_b[buf][(wn * 64 + r32) * kCorePitch + 32 * h];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8_t a_op[FM], b_op[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a_op[i] = *reinterpret_cast<const f16x8_t*>(fa + 32 * i * kCorePitch + 8 * t);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        b_op[j] = *reinterpret_cast<const f16x8_t*>(fb + 32 * j * kCorePitch + 8 * t);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_op[i], b_op[j], acc[i][j], 0, 0, 0);
    }
    // chunk c0 + 1 into the other buffer (last read before the previous barrier), then the
    // raw bytes of chunk c0 + 2
    if (c0 + 1 < nchunk) {
      convert(buf ^ 1);
      if (c0 + 2 < nchunk) load_raw(c0 + 2);
    }
    __syncthreads();
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

size_t delta_act_lds_bytes(int64_t K) {
  return ((size_t)K + kMaxCube * kStashPitch + 2 * kChunk) * sizeof(float);
}

hipError_t launch_delta_quant_act(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                  const float* lambda, const float* act_amax,
                                  const int32_t* cube_ptr, const int32_t* cube_rows,
                                  int64_t n_cubes, const uint16_t* down, int64_t r,
                                  uint8_t* core_codes, float* core_scale, uint8_t* delta_codes,
                                  uint8_t* delta_scales, float* g_delta, float* D, uint32_t* sat,
                                  hipStream_t s) {
  const size_t lds = delta_act_lds_bytes(K);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_delta_act),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  k_delta_act<<<dim3((unsigned)n_cubes), dim3(kThreads), lds, s>>>(
      X, M, K, ldx, lambda, act_amax, cube_ptr, cube_rows, core_codes, core_scale, delta_codes,
      delta_scales, g_delta, sat);
  e = hipGetLastError();
  if (e != hipSuccess || r == 0) return e;
  return launch_lowrank_down(X, M, K, ldx, lambda, down, r, D, s);
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
