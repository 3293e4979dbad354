// W4A4 GEMM on gfx950 MFMA with the low-rank up-projection folded into the accumulators before
// the bf16 store:  Y = bf16( g_a·g_w · Σ_k A_deq·W_deq + D·L2 [+ core_out[cube(m)]] )
// ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph; DeltaQuant core term:
// "DeltaQuant on MiniMax-H3").
//
// NVFP4 operands (E2M1 code × E4M3 block scale) need at most 6 significant bits and lie in
// [2^-10, 2688], so they are EXACT in fp16.  The kernel dequantises both operands to fp16
// (v_cvt_scalef32_pk_f16_fp4 with unit scale, then a packed fp16 multiply by the block scale)
// and runs v_mfma_f32_32x32x16_f16; every product is exact in the fp32 accumulator, and the two
// tensor scales are applied once at the store.  The hardware block-scaled FP4 MFMA takes
// power-of-two (E8M0) scales per 32 elements, which cannot carry an E4M3 scale per 16 exactly,
// so it is not used for this format.
//
// K mapping: MFMA step t of a 64-element stage covers elements [16t, 16t + 16); lane (row =
// lane % 32, h = lane / 32) supplies elements [16t + 8h, 16t + 8h + 8) of its row, for A and W
// alike, so every product pairs equal K indices.
#include <atomic>

#include "device.h"
#include "gemm_common.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kThreads = 512;  // 8 waves, 2 x 4 over the workgroup tile (two per SIMD)

// Workgroup tile 256 x 256, 8 waves in 2 x 4 (two per SIMD), each wave 128 x 64 (4 x 2 MFMA
// tiles of 32x32), tiles assigned in XCD-grouped order.
//
// Dequantisation is shared by the workgroup: K advances 64 elements per stage, and every
// thread converts one row of one operand (thread t: operand t % 2, row t / 2) of the stage to
// fp16 and stores it in LDS; the waves then read ready fp16 fragments.  Each code is converted
// once per workgroup instead of once per wave that uses it (four waves share an A row, two a W
// row).  The conversion of stage s+1 is spread over the four MFMA steps of stage s, and two fp16
// LDS buffers alternate with one barrier per stage.
//
// Global traffic is shaped for the vector L1, which cannot hold a stage's 512 rows from one
// stage to the next: a row is fetched as 64 code bytes (two stages, four 16-byte loads into
// registers, two rounds in flight) and its E4M3 scales as 16 bytes covering four stages
// (straight into LDS with global_load_lds, up to two chunks ahead), so a line is requested
// about once per two stages instead of twice per stage.
//
// LDS: [A fp16 buf 0][A buf 1][W buf 0][W buf 1] (256 rows x 64 fp16 = 128 bytes each), then
// two scale chunks [row][operand][16 bytes].  The 16-byte chunk c (elements [8c, 8c + 8)) of
// row R sits at chunk c ^ swz(R), and at c ^ swz(R) ^ 4 in W, which keeps the fragment reads
// (32 consecutive rows, one chunk) and the conversion stores (A and W rows interleaved in a
// wave, one chunk each) free of bank conflicts.
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kRowBytes = kBK * 2;          // fp16 row of one stage
constexpr int kOpBytes = kBM * kRowBytes;   // one operand, one buffer: 32 KB
constexpr int kWOffset = 2 * kOpBytes;      // W buffers follow the two A buffers
constexpr int kScaleOffset = 4 * kOpBytes;  // scale chunks follow the fp16 buffers
constexpr int kScaleChunk = 2 * kBM * 16;   // both operands, four stages: 8 KB
constexpr int kLdsBytes = kScaleOffset + 2 * kScaleChunk;

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// Workgroup barrier ordering LDS accesses only.  Loads in flight are waited for explicitly (scale
// chunks) or where their registers are used (codes), so the barrier must not wait for them,
// which a full __syncthreads() fence would do.  (The memory clobber keeps the compiler from
// moving memory accesses across it.)
// Chunk swizzle of fp16 row R (W rows additionally flip bit 2).  Fragment reads are served 16
// lanes (256 bytes) per pass and the conversion stores 8 lanes (128 bytes) per pass; this
// function gives distinct chunks to the 8 even and the 8 odd rows of 16 consecutive rows (reads)
// and to the rows of any aligned group of 4 (stores, A and W rows interleaved).
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


__global__ __launch_bounds__(kThreads) void k_gemm_nvfp4(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
    const uint8_t* __restrict__ As, const float* __restrict__ g_a,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs,
    const float* __restrict__ g_w, const float* __restrict__ D,
    const uint16_t* __restrict__ up, int r, const float* __restrict__ core_out,
    const int32_t* __restrict__ row_to_cube, uint16_t* __restrict__ Y, int64_t ldy) {
  constexpr int FM = 4, FN = 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  // Tile walk: workgroup `slot` of an XCD takes positions slot, slot + P, slot + 2P, ... of that
  // XCD's run of the tile sequence (P workgroups per XCD; P = the run's length gives one tile per
  // workgroup).  After a tile's store the next tile's first loads are issued at once, ahead of
  // its low-rank prologue, so their latency overlaps the prologue's own loads.
  // (Tile counts fit 32 bits: M < 2^31 rows and N < 2^31 columns in tiles of 256.)
  const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)(N / kBN);
  const int total = tiles_m * tiles_n, per_xcd = (total + 7) / 8;
  const int P = (int)gridDim.x / 8, xcd = (int)blockIdx.x % 8, slot = (int)blockIdx.x / 8;
  auto seq_of = [&](int k) -> int {
    const int w = slot + P * k, sq = xcd * per_xcd + w;
    return (w < per_xcd && sq < total) ? sq : -1;
  };
  const int seq0 = seq_of(0);
  if (seq0 < 0) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2, ks = K / 16;
  const int64_t nstage = K / kBK;    // a multiple of 4 (K % 256 == 0)
  const int64_t nround = nstage / 2;  // code rounds of two stages
  const int64_t nchunk = nstage / 4;  // scale chunks of four stages

  // Conversion share: operand co (0 A, 1 W), row crow of the tile.  Rows of A past M read row
  // M-1 (never stored).
  const int co = tid & 1, crow = tid >> 1;
  const int w_base = co * kWOffset + crow * kRowBytes;
  const int w_swz = swz(crow) ^ (co << 2);
  const uint8_t* pcode;
  const uint8_t* pscale;
  int64_t m_base, n_base;
  // the conversion rows of tile `sq` (and its wave-tile origin: m0 + 128 wm, n0 + 64 wn)
  auto tile_rows = [&](int sq, int64_t& mb, int64_t& nb) {
    int tm, tn;
    tile_of_seq32(sq, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
    int64_t ar = m0 + crow;
    ar = ar < M ? ar : M - 1;
    pcode = co ? B + (n0 + crow) * kb : A + ar * kb;
    pscale = co ? Bs + (n0 + crow) * ks : As + ar * ks;
    mb = m0 + wm * 128;
    nb = n0 + wn * 64;
  };
  tile_rows(seq0, m_base, n_base);

  // Scale chunks: the thread fetches the 16 scale bytes (four stages) of its own row and operand
  // into LDS slot tid (global_load_lds puts lane l of wave w at w * 1024 + 16 l) and reads them
  // back from there.
  auto load_scales = [&](int buf, int64_t c) {
    __builtin_amdgcn_global_load_lds((gvoid_t*)(pscale + c * 16),
                                     (lvoid_t*)(lds + kScaleOffset + buf * kScaleChunk +
                                                wave * 1024),
                                     16, 0, 0);
  };

  // Fragment reads: step t (elements [16t, 16t + 16) of a stage) of the lane's row is chunk
  // 2t + h; fragments i (j) of the wave are 32 rows apart (same low row bits, same swizzle).
  const int x = swz(r32);
  int ra[4], rb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    ra[t] = (wm * 128 + r32) * kRowBytes + 16 * ((2 * t + h) ^ x);
    rb[t] = kWOffset + (wn * 64 + r32) * kRowBytes + 16 * ((2 * t + h) ^ x ^ 4);
  }

  // a round: the row's 64 code bytes of stages 2q, 2q + 1
  auto load_round = [&](u32x4_t (&g)[4], int64_t q) {
#pragma unroll
    for (int v = 0; v < 4; ++v) g[v] = *reinterpret_cast<const u32x4_t*>(pcode + q * 64 + v * 16);
  };
  // code dword d (elements [8d, 8d + 8), block d / 2) of the stage held in words w[0..7] -> LDS
  auto convert = [&](const uint32_t* w, f16x2_t s01, f16x2_t s23, int buf, int d) {
    const _Float16 sc = d < 2 ? s01[0] : d < 4 ? s01[1] : d < 6 ? s23[0] : s23[1];
    *reinterpret_cast<f16x8_t*>(lds + buf * kOpBytes + w_base + 16 * (d ^ w_swz)) =
        dequant8(w[d], f16x2_t{sc, sc});
  };
  // the thread's scale chunk of four stages, read back from LDS once per chunk
  auto read_chunk = [&](int64_t c) {
    return *reinterpret_cast<const u32x4_t*>(lds + kScaleOffset + (int)(c & 1) * kScaleChunk +
                                             tid * 16);
  };
  auto stage_scales = [&](uint32_t v, f16x2_t& s01, f16x2_t& s23) {
    s01 = e4m3x2_to_f16x2(v & 0xFFFFu);
    s23 = e4m3x2_to_f16x2(v >> 16);
  };
  auto read_frags = [&](int buf, int t, f16x8_t (&fa)[FM], f16x8_t (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = *reinterpret_cast<const f16x8_t*>(lds + buf * kOpBytes + ra[t] + i * 32 * kRowBytes);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[j] = *reinterpret_cast<const f16x8_t*>(lds + buf * kOpBytes + rb[t] + j * 32 * kRowBytes);
  };

  // a tile's first loads: scale chunks 0, 1 and code rounds 0, 1
  u32x4_t g0[4], g1[4];
  auto first_loads = [&]() {
    load_scales(0, 0);
    load_scales(1, nchunk > 1 ? 1 : 0);
    load_round(g0, 0);
    load_round(g1, nround > 1 ? 1 : 0);
  };
  const float gsc = g_a[0] * g_w[0];
  first_loads();
  f32x16_t acc[FM][FN];
  u32x4_t sq;  // scales of stages 4c .. 4c + 3 (chunk c of the stage converted)
  f16x8_t a_op[FM], b_op[FN];
  // prologue of a tile (its first loads in flight): low-rank term into the accumulators, stage 0
  // converted into buffer 0
  auto prologue = [&]() {
    // (lane behind an opaque copy per tile: the compiler would otherwise compute the store's and
    // the low-rank term's lane-dependent addresses once, before the tile loop, and keep them
    // live through the main loop)
    int lo = lane;
    asm volatile("" : "+v"(lo));
    gemm_lowrank_init<FM, FN>(acc, 1.0f / gsc, M, m_base, n_base, lo & 31, lo >> 5, D, up, r);
    wait_vmcnt<0>();
    barrier_lds();
    sq = read_chunk(0);
    {
      f16x2_t s01, s23;
      stage_scales(sq[0], s01, s23);
      const uint32_t* w = reinterpret_cast<const uint32_t*>(g0);
#pragma unroll
      for (int d = 0; d < 8; ++d) convert(w, s01, s23, 0, d);
    }
    barrier_lds();
    read_frags(0, 0, a_op, b_op);
  };

  // Iteration s computes stage s from buffer s % 2 while converting stage s+1 (words w of a
  // register round) into the other buffer.  Extra work of the four-stage pattern, by s % 4:
  //   0: round s/2 + 2 loaded into g0 at the end (g0 consumed)
  //   2: round s/2 + 2 loaded into g1 at the end; scale chunk s/4 + 1 waited for before the
  //      barrier (read from iteration s + 1 on)
  //   3: scale chunk s/4 + 2 requested at the end.  (Issued here, the chunk is older than the
  //      code round that iteration s + 2 waits for, so the compiler's wait there stays partial.)
  // Past the end, loads repeat the last round / chunk into idle registers and buffers.
  auto iteration = [&](auto phase, int64_t s, const uint32_t* w, u32x4_t (&refill)[4]) {
    constexpr int ph = decltype(phase)::value;  // s % 4
    constexpr int p = ph & 1;
    // stage s+1 opens chunk s/4 + 1 at phase 3; that chunk landed before the previous barrier
    if (ph == 3) sq = read_chunk(s / 4 + 1);
    f16x2_t s01, s23;
    stage_scales(sq[(ph + 1) & 3], s01, s23);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // next step's fragments are requested before this step's MFMAs (the scheduling barriers
      // keep the compiler from sinking the reads to their use)
      f16x8_t na[FM], nb[FN];
      if (t < 3) read_frags(p, t + 1, na, nb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_op[i], b_op[j], acc[i][j], 0, 0, 0);
      convert(w, s01, s23, p ^ 1, 2 * t);
      convert(w, s01, s23, p ^ 1, 2 * t + 1);
      __builtin_amdgcn_sched_barrier(0);
      if (t < 3) {
#pragma unroll
        for (int i = 0; i < FM; ++i) a_op[i] = na[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) b_op[j] = nb[j];
      }
    }
    if (ph == 0 || ph == 2) {
      const int64_t q = s / 2 + 2;
      load_round(refill, q < nround ? q : nround - 1);
    }
    // all but the round just issued: at phase 2 the scale chunk read from the next iteration
    // on has landed; at phase 0 the round of g1 (used next) has, which spares the next iteration
    // a full wait (the compiler, unable to place the older scale chunk in the count, would
    // wait for everything)
    if (ph == 0 || ph == 2) wait_vmcnt<4>();
    if (ph == 3) {
      // chunk s/4 + 2 into the buffer of chunk s/4, whose last stage was converted in the
      // previous iteration
      const int64_t c = s / 4 + 2;
      load_scales((int)(c & 1), c < nchunk ? c : nchunk - 1);
    }
    barrier_lds();
    read_frags(p ^ 1, 0, a_op, b_op);
  };
  for (int k = 0;; ++k) {
    prologue();
    for (int64_t s = 0; s < nstage; s += 4) {
      // stage s+1: second half of round s/2 (g0); s+2, s+3: round s/2 + 1 (g1); s+4: g0 again
      iteration(std::integral_constant<int, 0>{}, s, reinterpret_cast<const uint32_t*>(g0) + 8, g0);
      iteration(std::integral_constant<int, 1>{}, s + 1, reinterpret_cast<const uint32_t*>(g1), g1);
      iteration(std::integral_constant<int, 2>{}, s + 2, reinterpret_cast<const uint32_t*>(g1) + 8, g1);
      iteration(std::integral_constant<int, 3>{}, s + 3, reinterpret_cast<const uint32_t*>(g0), g0);
    }
    // Every wave passed the last barrier after its final fragment reads: the fp16 buffers are
    // free for the output staging (each wave its own 16 KB; the scale chunks lie above them).
    static_assert(8 * gemm_store_bytes<FM, FN>() <= kScaleOffset, "output staging fits the LDS");
    int lo = lane;
    asm volatile("" : "+v"(lo));
    gemm_store<FM, FN>(acc, gsc, lds + wave * gemm_store_bytes<FM, FN>(), lo, M, N, m_base,
                       n_base, core_out, row_to_cube, Y, ldy);
    const int seq_n = seq_of(k + 1);
    if (seq_n < 0) break;
    // the next tile: the loads the last iterations repeated past the end have landed before its
    // first loads rewrite the same scale buffers and registers.  (The wait also covers the
    // store's writes; leaving it out, with the prologue's full wait covering both, measured the
    // same.)
    wait_vmcnt<0>();
    tile_rows(seq_n, m_base, n_base);
    first_loads();
    // every wave's staging reads are done before stage 0 is converted into buffer 0
    barrier_lds();
  }
}

}  // namespace

hipError_t launch_gemm_int4(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const void* a_scales, const uint8_t* w_codes, const void* w_scales,
                            const float* D, const uint16_t* up, int64_t r, uint16_t* Y,
                            int64_t ldy, hipStream_t s);

hipError_t launch_gemm_mx(int fp8, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                          const uint8_t* a_scales, const uint8_t* w_codes,
                          const uint8_t* w_scales, const float* D, const uint16_t* up, int64_t r,
                          uint16_t* Y, int64_t ldy, hipStream_t s);

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const void* a_scales, const float* g_a, const uint8_t* w_codes,
                       const void* w_scales, const float* g_w, const float* D,
                       const uint16_t* up, int64_t r, const float* core_out,
                       const int32_t* row_to_cube, uint16_t* Y, int64_t ldy, hipStream_t s) {
  if (fmt == 1)
    return launch_gemm_int4(M, N, K, a_codes, a_scales, w_codes, w_scales, D, up, r, Y, ldy, s);
  if (fmt == 2 || fmt == 3)
    return launch_gemm_mx(fmt == 3, M, N, K, a_codes, reinterpret_cast<const uint8_t*>(a_scales),
                          w_codes, reinterpret_cast<const uint8_t*>(w_scales), D, up, r, Y, ldy,
                          s);
  // one workgroup per CU walking its XCD's share of the tile sequence
  const int64_t total = ((M + kBM - 1) / kBM) * (N / kBN), per_xcd = (total + 7) / 8;
  int64_t per = device_cus() / 8;
  if (per < 1 || per > per_xcd) per = per_xcd;
  const dim3 grid((unsigned)(8 * per));
  k_gemm_nvfp4<<<grid, dim3(kThreads), 0, s>>>(
      M, N, K, a_codes, reinterpret_cast<const uint8_t*>(a_scales), g_a, w_codes,
      reinterpret_cast<const uint8_t*>(w_scales), g_w, D, up, (int)r, core_out, row_to_cube, Y,
      ldy);
  return hipGetLastError();
}

}  // namespace svdq
