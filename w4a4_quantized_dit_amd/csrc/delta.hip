// DeltaQuant variant ("DeltaQuant on MiniMax-H3": a cube of tokens is represented by one core
// plus per-token deltas; the delta's NVFP4 tensor scale comes from the bound
// |x − core| ≤ 2·max|x| ("The activation scale bound held"); the core branch stays on a 16-bit
// path ("Deviations from the paper, and one replication")).
//
// k_delta_act: one pass over X.  A workgroup (4 waves) owns a group of consecutive cubes of at
// most 64 member rows and 16 cubes (packed on the host), gathers the members' rows through the
// CSR and walks K in chunks of 128 channels:
//   1. the rows' chunk (bf16) and the matching slice of L1 go from registers (loaded two chunks
//      ahead) into LDS;
//   2. a thread per (cube, channel pair) sums the cube's smoothed members X̂ = X · 1/λ in
//      ascending row order in fp32 and divides by the member count; the core chunk stays in
//      LDS for step 3 and goes to the caller's fp32 workspace for step 4, and the thread keeps
//      the running |core| maximum of its channels;
//   3. lane (row = lane % 16 of its wave, q = lane / 16) takes its row's 32 channels
//      [32q, 32q + 32): the delta X̂ − core (unquantised core) is quantised to NVFP4 with the
//      static tensor amax 2·act_amax (two whole blocks per lane, lane-local block maxima), and
//      bf16(X̂) feeds v_mfma_f32_16x16x32_bf16 against the L1 slice for D = bf16(X̂)·L1 at rank r;
//   4. after the last chunk every cube's amax gives its E4M3 scale amax/448, and each lane
//      re-reads the fp32 core values it wrote in step 2 and encodes them.
// The core's scale needs the whole row's maximum before any code can be written, which is why
// the fp32 core makes one round trip through the workspace; X itself is read exactly once.
// k_gemm_core: core_out[c, n] = s_c · g_w · Σ_k e4m3(core[c, k]) · (c_w·s_w)[n, k] on fp16 MFMA:
// E4M3 values and the NVFP4 weight products are exact in fp16.
#include <mutex>

#include "device.h"
#include "launch.h"

namespace svdq {

// Scratch of the allocation-free DeltaQuant entry point: the fp32 cores of one call.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code never uses this
// name as an address: the per-device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[kDeltaScratchBytes];

namespace {

constexpr int kThreads = 256;              // k_gemm_core and k_delta_act: 4 waves
constexpr int kDRows = 64;                 // rows of a cube group (4 waves x 16)
constexpr int kDCubes = 16;                // cubes of a cube group
constexpr int kDChunk = 128;               // channels per chunk
constexpr int kDPitch = kDChunk + 8;       // bf16 per staged row: 272 B, conflict-free 16-B reads
constexpr int kDCorePitch = kDChunk + 4;   // fp32 per core row in LDS

template <int NT>
__global__ __launch_bounds__(kThreads, 2) void k_delta_act(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ lambda, const float* __restrict__ act_amax,
    const int32_t* __restrict__ cube_ptr, const int32_t* __restrict__ cube_rows,
    const int32_t* __restrict__ group_ptr, const uint16_t* __restrict__ down, int r,
    uint8_t* __restrict__ core_codes, float* __restrict__ core_scale,
    uint8_t* __restrict__ dcodes, uint8_t* __restrict__ dscales, float* __restrict__ g_delta,
    float* __restrict__ D, uint32_t* __restrict__ sat, float* __restrict__ core32) {
  constexpr int NTc = NT > 0 ? NT : 1;
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kDRows * kDPitch];
  __shared__ __attribute__((aligned(16))) uint16_t s_l[NTc * 16 * kDPitch];
  __shared__ __attribute__((aligned(16))) float s_core[kDCubes * kDCorePitch];
  __shared__ __attribute__((aligned(16))) float s_inv[2][kDChunk];
  __shared__ int s_row[kDRows], s_slot[kDRows], s_first[kDCubes], s_cnt[kDCubes];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c0 = group_ptr[blockIdx.x], ncub = group_ptr[blockIdx.x + 1] - c0;
  const int p0 = cube_ptr[c0];
  const int nrows = ncub > 0 ? cube_ptr[c0 + ncub] - p0 : 0;
  if (ncub < 1 || ncub > kDCubes || nrows < 1 || nrows > kDRows) {
    // not a group the host packer makes: its cubes get a NaN scale (uniform exit)
    if (tid < ncub && tid < kDCubes) core_scale[c0 + tid] = __builtin_nanf("");
    return;
  }
  if (tid < ncub) {
    s_first[tid] = cube_ptr[c0 + tid] - p0;
    s_cnt[tid] = cube_ptr[c0 + tid + 1] - cube_ptr[c0 + tid];
  }
  if (tid < kDRows) {
    int m = cube_rows[p0 + (tid < nrows ? tid : nrows - 1)];
    s_row[tid] = m < 0 ? 0 : (m < M ? m : (int)M - 1);  // rows past the group repeat its last
  }
  const float amax_t = 2.0f * act_amax[0];
  const float g = amax_t == 0.0f ? 1.0f : amax_t / 2688.0f;
  const float d6 = 6.0f * g;
  if (blockIdx.x == 0 && tid == 0) g_delta[0] = g;
  __syncthreads();
  if (tid < kDRows) {
    int sl = -1;
    if (tid < nrows)
      for (int s = 0; s < ncub; ++s)
        if (tid >= s_first[s]) sl = s;
    s_slot[tid] = sl;
  }

  // staging roles: X piece i of this thread is row (tid / 16) + 16 i, 16 bytes at 8·(tid % 16);
  // L1 piece u is rank (tid + 256 u) / 16 at the same channels (ranks past r are zeroed)
  const int seg = tid & 15;
  const uint16_t* xp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xp[i] = X + (int64_t)s_row[(tid >> 4) + 16 * i] * ldx + 8 * seg;
  const uint16_t* lp[NTc];
#pragma unroll
  for (int u = 0; u < NTc; ++u) {
    const int n = (tid >> 4) + 16 * u;
    lp[u] = down + (int64_t)(n < r ? n : (r > 0 ? r - 1 : 0)) * K + 8 * seg;
  }
  const int64_t nchunk = K / kDChunk;
  auto load_x = [&](u32x4_t (&v)[4], int64_t c) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(xp[i] + c * kDChunk));
  };
  auto load_l = [&](u32x4_t (&v)[NTc], int64_t c) {
#pragma unroll
    for (int u = 0; u < NT; ++u) v[u] = *reinterpret_cast<const u32x4_t*>(lp[u] + c * kDChunk);
  };
  // 1/λ of chunk c into s_inv[c & 1]: threads 0..127, one channel each
  auto stage_inv = [&](float lam_v, int64_t c) {
    if (tid < kDChunk) s_inv[c & 1][tid] = lambda ? 1.0f / lam_v : 1.0f;
  };
  auto load_lam = [&](int64_t c) {
    return (lambda && tid < kDChunk && c < nchunk) ? lambda[c * kDChunk + tid] : 1.0f;
  };

  // lane roles in steps 3 and 4
  const int rl = lane & 15, q = lane >> 4;
  const int srow = 16 * wave + rl;
  const bool valid = srow < nrows;
  const int64_t grow = s_row[srow];
  f32x4_t acc[NTc];
#pragma unroll
  for (int j = 0; j < NTc; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float camax[4] = {0.f, 0.f, 0.f, 0.f};
  uint32_t nsat = 0;

  auto chunk = [&](int64_t c, u32x4_t (&xcur)[4], u32x4_t (&lr)[NTc], float& lam_next) {
    const int64_t k0 = c * kDChunk;
    // 1. registers -> LDS
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(&s_x[((tid >> 4) + 16 * i) * kDPitch + 8 * seg]) = xcur[i];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int n = (tid >> 4) + 16 * u;
      *reinterpret_cast<u32x4_t*>(&s_l[n * kDPitch + 8 * seg]) =
          n < r ? lr[u] : u32x4_t{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // the next chunks' loads: λ two chunks ahead, L1 one, X two (into the registers just
    // stored).  Loads complete in issue order for the wait counter, so X goes last: waiting for
    // the L1 slice at the next chunk then leaves the X prefetch in flight.
    const float lam_c1 = lam_next;
    lam_next = load_lam(c + 2);
    if (c + 1 < nchunk) load_l(lr, c + 1);
    if (c + 2 < nchunk) load_x(xcur, c + 2);
    // 2. core chunk: (cube slot, channel pair) items, ascending fp32 sum over the members
    const float* inv = s_inv[c & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int item = tid + kThreads * i;
      const int sl = item >> 6, pr = item & 63;
      if (sl < ncub) {
        const int f = s_first[sl], n = s_cnt[sl];
        const float i0 = inv[2 * pr], i1 = inv[2 * pr + 1];
        float a0 = 0.0f, a1 = 0.0f;
        const uint16_t* xc = &s_x[f * kDPitch + 2 * pr];
        int j = 0;
        // four members' reads issued together, then added in ascending order
        for (; j + 4 <= n; j += 4) {
          uint32_t w[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            w[u] = *reinterpret_cast<const uint32_t*>(xc + (j + u) * kDPitch);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            a0 += bf16_lo(w[u]) * i0;
            a1 += bf16_hi(w[u]) * i1;
          }
        }
        for (; j < n; ++j) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(xc + j * kDPitch);
          a0 += bf16_lo(w) * i0;
          a1 += bf16_hi(w) * i1;
        }
        const float v0 = a0 / (float)n, v1 = a1 / (float)n;
        *reinterpret_cast<float2*>(&s_core[sl * kDCorePitch + 2 * pr]) = float2{v0, v1};
        *reinterpret_cast<float2*>(core32 + (int64_t)(c0 + sl) * K + k0 + 2 * pr) =
            float2{v0, v1};
        camax[i] = fmaxf(camax[i], fmaxf(fabsf(v0), fabsf(v1)));
      }
    }
    stage_inv(lam_c1, c + 1);   // s_inv[(c + 1) & 1] was last read before the previous barrier
    __syncthreads();
    // 3. delta NVFP4 blocks and the low-rank MFMA of the lane's row and 32 channels
    {
      const int sl = s_slot[srow] < 0 ? 0 : s_slot[srow];
      float x[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&s_x[srow * kDPitch + 32 * q + 8 * i]);
        const f32x4_t ia = *reinterpret_cast<const f32x4_t*>(inv + 32 * q + 8 * i);
        const f32x4_t ib = *reinterpret_cast<const f32x4_t*>(inv + 32 * q + 8 * i + 4);
        x[8 * i + 0] = bf16_lo(v[0]) * ia[0]; x[8 * i + 1] = bf16_hi(v[0]) * ia[1];
        x[8 * i + 2] = bf16_lo(v[1]) * ia[2]; x[8 * i + 3] = bf16_hi(v[1]) * ia[3];
        x[8 * i + 4] = bf16_lo(v[2]) * ib[0]; x[8 * i + 5] = bf16_hi(v[2]) * ib[1];
        x[8 * i + 6] = bf16_lo(v[3]) * ib[2]; x[8 * i + 7] = bf16_hi(v[3]) * ib[3];
      }
      const float* cr = s_core + sl * kDCorePitch + 32 * q;
      uint32_t cw[4];
      uint32_t sb = 0;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float d[16];
        float a = 0.0f;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const f32x4_t cq = *reinterpret_cast<const f32x4_t*>(cr + 16 * b + 4 * e4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d[4 * e4 + e] = x[16 * b + 4 * e4 + e] - cq[e];
            a = fmaxf(a, fabsf(d[4 * e4 + e]));
          }
        }
        nsat += (valid && a > amax_t) ? 1u : 0u;
        float sinv;
        sb |= nvfp4_block_scale(a, g, d6, &sinv) << (8 * b);
        float y[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) y[e] = d[e] * sinv;
        cw[2 * b] = e2m1_pack8(y);
        cw[2 * b + 1] = e2m1_pack8(y + 8);
      }
      if (valid) {
        const int64_t kq = k0 + 32 * q;
        *reinterpret_cast<u32x4_t*>(dcodes + grow * (K / 2) + kq / 2) =
            u32x4_t{cw[0], cw[1], cw[2], cw[3]};
        *reinterpret_cast<uint16_t*>(dscales + grow * (K / 16) + kq / 16) = (uint16_t)sb;
      }
      if (NT > 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          u32x4_t av;
          av[0] = pack_bf16x2(x[8 * t + 0], x[8 * t + 1]);
          av[1] = pack_bf16x2(x[8 * t + 2], x[8 * t + 3]);
          av[2] = pack_bf16x2(x[8 * t + 4], x[8 * t + 5]);
          av[3] = pack_bf16x2(x[8 * t + 6], x[8 * t + 7]);
          const bf16x8_t a_op = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(
                &s_l[(16 * j + rl) * kDPitch + 32 * q + 8 * t]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a_op, __builtin_bit_cast(bf16x8_t, bv), acc[j], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();  // the staging buffers are rewritten by the next chunk
  };

  // prologue: chunks 0 and 1 of X, chunk 0 of L1, 1/λ of chunk 0; λ of chunk 1 in flight
  u32x4_t xa[4], xb[4], lr[NTc];
  const float lam0 = load_lam(0);
  float lam_next = load_lam(1);
  load_l(lr, 0);
  load_x(xa, 0);
  if (nchunk > 1) load_x(xb, 1);
  stage_inv(lam0, 0);
  __syncthreads();
  for (int64_t c = 0; c < nchunk; c += 2) {
    chunk(c, xa, lr, lam_next);
    if (c + 1 < nchunk) chunk(c + 1, xb, lr, lam_next);
  }

  // D rows (16x16 output: lane holds rank column 16j + rl and staged rows 4q .. 4q + 3)
  if (NT > 0) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = 16 * j + rl;
      if (n < r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sr = 16 * wave + 4 * q + i;
          if (sr < nrows) D[(int64_t)s_row[sr] * r + n] = acc[j][i];
        }
      }
    }
  }
  // 4. core scales and FP8 codes: wave w owns cube slots w, w + 4, ...; lane l re-reads the
  // channel pair 2l, 2l + 1 of every chunk that it wrote in step 2 (its own stores, visible
  // to it after the barrier's fence).  The values of all the wave's slots are requested
  // together, 32 per lane, so a wave waits for memory a few times per group rather than once
  // per slot and batch.
  float inv_c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sl = wave + 4 * i;
    float am = camax[i];
    for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    const float sc = am / 448.0f;
    inv_c[i] = sc != 0.0f ? 1.0f / sc : 0.0f;
    if (lane == 0 && sl < ncub) core_scale[c0 + sl] = sc;
  }
  {
    // a batch covers 2^LCB chunks of each of the wave's (up to four) slots: 32 values per lane
    const int own = ncub > wave ? (ncub - wave + 3) / 4 : 0;  // slots of this wave
    auto encode = [&](auto lcb_c) {
      constexpr int LCB = decltype(lcb_c)::value, CB = 1 << LCB, NS = 32 >> LCB;
      const float* src[NS];
      uint8_t* dst[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int64_t c = c0 + wave + 4 * (i < own ? i : 0);
        src[i] = core32 + c * K + 2 * lane;
        dst[i] = core_codes + c * K + 2 * lane;
      }
      for (int64_t cc0 = 0; cc0 < nchunk; cc0 += CB) {
        float2 v[NS][CB];
#pragma unroll
        for (int i = 0; i < NS; ++i)
#pragma unroll
          for (int b = 0; b < CB; ++b)
            v[i][b] = (i < own && cc0 + b < nchunk)
                          ? *reinterpret_cast<const float2*>(src[i] + (cc0 + b) * kDChunk)
                          : float2{0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NS; ++i)
#pragma unroll
          for (int b = 0; b < CB; ++b)
            if (i < own && cc0 + b < nchunk) {
              *reinterpret_cast<uint16_t*>(dst[i] + (cc0 + b) * kDChunk) =
                  (uint16_t)e4m3_pack2(v[i][b].x * inv_c[i], v[i][b].y * inv_c[i]);
            }
      }
    };
    if (own > 2) encode(std::integral_constant<int, 3>{});
    else if (own == 2) encode(std::integral_constant<int, 4>{});
    else if (own == 1) encode(std::integral_constant<int, 5>{});
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

int64_t delta_workspace_bytes(int64_t n_cubes, int64_t K) { return n_cubes * K * 4; }

hipError_t launch_delta_quant_act(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                                  const float* lambda, const float* act_amax,
                                  const int32_t* cube_ptr, const int32_t* cube_rows,
                                  const int32_t* group_ptr, int64_t n_groups,
                                  const uint16_t* down, int64_t r, uint8_t* core_codes,
                                  float* core_scale, uint8_t* delta_codes, uint8_t* delta_scales,
                                  float* g_delta, float* D, uint32_t* sat, void* workspace,
                                  hipStream_t s) {
  const int nt = (int)((r + 15) / 16);
  float* core32 = reinterpret_cast<float*>(workspace);
#define SVDQ_DELTA_CASE(NTV)                                                                 \
  case NTV:                                                                                  \
    k_delta_act<NTV><<<dim3((unsigned)n_groups), dim3(kThreads), 0, s>>>(                    \
        X, M, K, ldx, lambda, act_amax, cube_ptr, cube_rows, group_ptr, down, (int)r,        \
        core_codes, core_scale, delta_codes, delta_scales, g_delta, D, sat, core32);         \
    break;
  switch (nt) {
    SVDQ_DELTA_CASE(0)
    SVDQ_DELTA_CASE(1)
    SVDQ_DELTA_CASE(2)
    SVDQ_DELTA_CASE(3)
    SVDQ_DELTA_CASE(4)
    SVDQ_DELTA_CASE(5)
    SVDQ_DELTA_CASE(6)
    SVDQ_DELTA_CASE(7)
    SVDQ_DELTA_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef SVDQ_DELTA_CASE
  return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t delta_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // once per device, with that device current
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
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
