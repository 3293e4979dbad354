// MX variant of the layer's GEMM on gfx950's hardware block-scaled MFMA:
//   Y = bf16( Σ_blocks 2^(e_a + e_w) · Σ_{k in block} c_a·c_w  +  D·L2 )
// with E2M1 (MXFP4, W4A4) or E4M3 (MXFP8, W8A8) codes and one E8M0 exponent per 32 along K
// ("MiniMax-H3 — MXFP8 (weight-quantized, vLLM-Omni native layout)", section "Quant format";
// the layer: "MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph).
//
// This is the scale layout v_mfma_scale_f32_32x32x64_f8f6f4 takes natively: one MFMA covers 64
// elements of K, i.e. two scale blocks per row, and each lane supplies the E8M0 byte of its
// (row, block).  The codes go from global memory through LDS into the MFMA with no conversion at
// all.  Operand layout (measured): lane (row = lane % 32,
// h = lane / 32) holds, for FP4, elements [32h, 32h + 32) of the 64 in dwords 0..3 (element 8d
// + j in nibble j of dword d); for FP8, dwords 0..3 hold elements [16h, 16h + 16) of block 0 and
// dwords 4..7 the same positions of block 1, with lane h supplying block h's scale.  Inside a
// block the element order only has to agree between A and W.
//
// MXFP4 kernel.  Tiling: workgroup 256 x 256, 8 waves (two per SIMD) of 128 x 64 (4 x 2 tiles of
// 32x32), XCD-grouped tile order.  K advances 256 elements per stage (four MFMA steps of 64).  A
// stage goes global -> registers (one stage ahead) -> LDS (two buffers); the fragments are
// double-buffered per MFMA step, so the LDS reads of the next step run under the MFMAs of the
// current one, with one LDS-only barrier per stage.
//
// What bounds the loads is the rate at which a CU issues requests to L2 (measured: about one per
// four clocks whatever their size, i.e. about 64 GB/s per CU with full 128-byte lines), not
// their bytes: a row's contiguous code bytes of a stage go out as one request, and so do its
// scale bytes.  The deep stage makes these 128 code bytes per row and stage, eight consecutive
// lanes reading one row's 128 bytes in order, and the scale bytes are fetched 16 per row for
// two stages at a time (8 per stage would make them half of all requests).
//
// LDS layout of one operand's stage: region g (g = 0..3, one per MFMA step) holds bytes
// [32g, 32g + 32) of every row's 128, as two 16-byte halves swapped on rows with bit 3 set;
// regions are 64 bytes longer than their 8 KB of data.  A fragment read (32 consecutive rows,
// one half each) then touches every bank once per 16 lanes, the eight lanes of one row write
// four regions on disjoint banks, and every fragment address is one per-lane base plus a
// constant.  A row's eight E8M0 bytes of the stage are one 8-byte word.  The low-rank term and
// the LDS-staged bf16 store are the ones of the NVFP4 GEMM.
#include "device.h"
#include "gemm_common.h"
#include "launch.h"

#include <type_traits>

namespace svdq {

namespace {

constexpr int kThreads = 512;
constexpr int kBM = 256, kBN = 256;
constexpr int FM = 4, FN = 2;

struct Fp4Cfg {
  static constexpr int kBK = 256;                         // K per stage
  static constexpr int kSteps = kBK / 64;                 // MFMA steps per stage
  static constexpr int kRowBytes = kBK / 2;               // codes of a row per stage
  static constexpr int kRegionBytes = kBM * 32 + 64;      // one step's 32 bytes of every row
  static constexpr int kCodeBuf = kSteps * kRegionBytes;  // one operand, one stage
  static constexpr int kScaleRow = kBK / 32;              // E8M0 bytes of a row per stage
  static constexpr int kScaleBuf = kBM * kScaleRow;
  static constexpr int kStageBytes = 2 * kCodeBuf + 2 * kScaleBuf;
  static constexpr int kPerThread = kBM * kRowBytes / 16 / kThreads;  // 16-byte loads per operand
  static constexpr int kStoreBytes = 8 * gemm_store_bytes<FM, FN>();
  static constexpr int kLdsBytes = 2 * kStageBytes > kStoreBytes ? 2 * kStageBytes : kStoreBytes;
};

// stored half of a row's region: the logical half XOR this
__device__ __forceinline__ int half_swz(int row) { return (row >> 3) & 1; }

// Workgroup barrier ordering LDS accesses only (the next stage's global loads stay in flight,
// which a full __syncthreads() fence would drain).  The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One stage in registers.  Load q of thread tid is 16-byte chunk c = 512q + tid of the operand
// tile: row c / 8, bytes 16 (c % 8) onward of the row's stage slab.  Thread tid also owns the
// scale row tid (A) or tid - 256 (W), whose E8M0 words it fetches two stages at a time: a row's
// scale bytes are a request of their own, as many as its code bytes, so one 16-byte request per
// two stages instead of an 8-byte one per stage takes a quarter off the kernel's requests.
// A's loads go through range-checked buffer resources whose base and record count carry the
// row slice and the stage, with only the lane's own offset in the VGPR (the scalar offset is not
// part of the range check), so rows past M read as zero without touching memory; their results
// are never stored.
struct StageRegs {
  u32x4_t a[Fp4Cfg::kPerThread], b[Fp4Cfg::kPerThread];
  uint32_t sc[4];  // scale words of two consecutive stages: sc[0..1] the first, sc[2..3] the second
};

struct StageSrc {
  const uint8_t* a;   // A codes of the tile's first row
  const uint8_t* b;   // W codes of the tile's first row
  const uint8_t* s;   // scale row 0 of this wave's operand (A: waves 0..3, W: 4..7)
  int64_t a_rows;     // valid rows of the A tile
  int64_t s_rows;     // valid rows of this wave's scale operand
  uint32_t kb, ks, voff, s_voff;
};

constexpr int kRaw = 0x00020000;  // raw buffer resource, word 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint8_t* base, int64_t rows,
                                                            uint32_t pitch, uint32_t skip) {
  const int64_t n = rows > 0 ? rows * (int64_t)pitch - skip : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(base + skip), (short)0, (int)n, kRaw);
}

__device__ __forceinline__ void codes_load(StageRegs& R, const StageSrc& src, uint32_t stage) {
  using C = Fp4Cfg;
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)src.b, (short)0, (int)(kBN * src.kb), kRaw);
#pragma unroll
  for (int q = 0; q < C::kPerThread; ++q) {
    const uint32_t skip = stage * C::kRowBytes;
    const __amdgpu_buffer_rsrc_t ra =
        rows_rsrc(src.a + (int64_t)q * 64 * src.kb, src.a_rows - 64 * q, src.kb, skip);
    R.a[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, src.voff, 0, 0));
    R.b[q] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, src.voff, (int)(q * 64 * src.kb + skip), 0));
  }
}

// Scale words of stages u and u + 1 of the thread's scale row (16 bytes).  Near the end of K
// (u >= last) the pair of stages last - 1 and last is read instead, so that the load stays
// inside the row; stage last is then the upper half.  With a single stage (last == 0) the load
// is out of the resource's range: zeros, no memory access.
__device__ __forceinline__ void scale_pair_load(StageRegs& R, const StageSrc& src, uint32_t u,
                                                uint32_t last) {
  using C = Fp4Cfg;
  const uint32_t o = last == 0 ? 0 : (u < last ? u : last - 1);
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(src.s, src.s_rows, src.ks, o * C::kScaleRow);
  const u32x4_t v = __builtin_bit_cast(
      u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, last == 0 ? kNoLoad : src.s_voff, 0, 0));
#pragma unroll
  for (int e = 0; e < 4; ++e) R.sc[e] = v[e];
}

// The stage's codes, and its scale words from the lower (hi = false) or upper half of the pair.
__device__ __forceinline__ void stage_store(const StageRegs& R, uint8_t* buf, int st_off,
                                            int tid, bool hi) {
  using C = Fp4Cfg;
#pragma unroll
  for (int q = 0; q < C::kPerThread; ++q) {
    *reinterpret_cast<u32x4_t*>(buf + st_off + q * 64 * 32) = R.a[q];
    *reinterpret_cast<u32x4_t*>(buf + C::kCodeBuf + st_off + q * 64 * 32) = R.b[q];
  }
  const uint2 w = hi ? uint2{R.sc[2], R.sc[3]} : uint2{R.sc[0], R.sc[1]};
  *reinterpret_cast<uint2*>(buf + 2 * C::kCodeBuf + tid * C::kScaleRow) = w;
}

// Fragments of one MFMA step: the lane's 16 bytes of each of the wave's 4 + 2 tiles.
struct Frags {
  u32x4_t a[FM], b[FN];
};

__device__ __forceinline__ void frags_read(Frags& F, const uint8_t* a_lds, const uint8_t* b_lds,
                                           int t) {
  using C = Fp4Cfg;
#pragma unroll
  for (int i = 0; i < FM; ++i)
    F.a[i] = *reinterpret_cast<const u32x4_t*>(a_lds + t * C::kRegionBytes + i * 32 * 32);
#pragma unroll
  for (int j = 0; j < FN; ++j)
    F.b[j] = *reinterpret_cast<const u32x4_t*>(b_lds + t * C::kRegionBytes + j * 32 * 32);
}

// The fragments' rows' scale bytes of a stage, one word per row: byte t is the E8M0 byte of
// block 2t + h, the one lane h uses in MFMA step t (a row's eight bytes come from LDS as one
// 8-byte word; a byte permute gathers the lane's four).
struct Scales {
  uint32_t a[FM], b[FN];
};

__device__ __forceinline__ void scales_read(Scales& S, const uint8_t* buf, int a_row0, int b_row0,
                                            uint32_t sel) {
  using C = Fp4Cfg;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const uint2 v = *reinterpret_cast<const uint2*>(buf + 2 * C::kCodeBuf +
                                                    (a_row0 + 32 * i) * C::kScaleRow);
    S.a[i] = __builtin_amdgcn_perm(v.y, v.x, sel);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const uint2 v = *reinterpret_cast<const uint2*>(buf + 2 * C::kCodeBuf + C::kScaleBuf +
                                                    (b_row0 + 32 * j) * C::kScaleRow);
    S.b[j] = __builtin_amdgcn_perm(v.y, v.x, sel);
  }
}

__device__ __forceinline__ i32x8_t fp4_op(u32x4_t v) {
  return i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
}

__device__ __forceinline__ void mfma_step(f32x16_t (&acc)[FM][FN], const Frags& F, const Scales& S,
                                          int t) {
  constexpr int kFp4 = 4;  // MFMA operand format E2M1
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          fp4_op(F.a[i]), fp4_op(F.b[j]), acc[i][j], kFp4, kFp4, 0,
          (int)((S.a[i] >> (8 * t)) & 0xFFu), 0, (int)((S.b[j] >> (8 * t)) & 0xFFu));
}

__global__ __launch_bounds__(kThreads) void k_gemm_mxfp4(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
    const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const float* __restrict__ D,
    const uint16_t* __restrict__ up, int r, uint16_t* __restrict__ Y, int64_t ldy) {
  using C = Fp4Cfg;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLdsBytes];
  int64_t tm, tn;
  if (!tile_of_block((M + kBM - 1) / kBM, N / kBN, tm, tn)) return;
  const int64_t m0 = tm * kBM, n0 = tn * kBN;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t m_base = m0 + wm * 128, n_base = n0 + wn * 64;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t kb = K / 2, ks = K / 32;
  const int64_t nstage = K / C::kBK;

  // stage sources: this thread's 16-byte part of its row (row q·64 + tid / 8 of load q) and its
  // scale row; and the LDS offset of its stores (region part / 2, row, swizzled half part % 2)
  const int part = tid & 7;
  const int lrow = tid >> 3;  // row within each load's 64-row slice (same swizzle for every q)
  const int64_t a_rows = M - m0 < kBM ? M - m0 : kBM;
  const bool a_side = __builtin_amdgcn_readfirstlane(wave) < 4;
  StageSrc src;
  src.a = A + m0 * kb;
  src.b = B + n0 * kb;
  src.s = a_side ? As + m0 * ks : Bs + n0 * ks;
  src.a_rows = a_rows;
  src.s_rows = a_side ? a_rows : kBN;
  src.kb = (uint32_t)kb;
  src.ks = (uint32_t)ks;
  src.voff = (uint32_t)(lrow * kb + 16 * part);
  src.s_voff = (uint32_t)((tid & 255) * ks);
  const int st_off = (part >> 1) * C::kRegionBytes + lrow * 32 + 16 * ((part & 1) ^ half_swz(lrow));
  // LDS bases of this lane's fragments (the fragment rows share their low 5 bits with r32)
  const int frag_off = r32 * 32 + 16 * (h ^ half_swz(r32));
  const int a_lds = wm * 128 * 32 + frag_off;
  const int b_lds = C::kCodeBuf + wn * 64 * 32 + frag_off;
  const int a_row0 = wm * 128 + r32, b_row0 = wn * 64 + r32;
  // byte permute of a row's two scale words (high word first) taking blocks h, 2 + h, 4 + h, 6 + h
  const uint32_t sel = h ? 0x07050301u : 0x06040200u;

  f32x16_t acc[FM][FN];
  gemm_lowrank_init<FM, FN>(acc, 1.0f, M, m_base, n_base, r32, h, D, up, r);

  // prologue: stage 0 in LDS buffer 0, stage 1 in registers (its scale words are the upper half
  // of the pair loaded with stage 0's), step (0, 0) in F0
  const uint32_t last = (uint32_t)(nstage - 1);
  StageRegs R;
  codes_load(R, src, 0);
  if (last > 0) {
    scale_pair_load(R, src, 0, last);
  } else {  // a single stage: its 8 bytes are the whole scale row
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(src.s, src.s_rows, src.ks, 0);
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, src.s_voff, 0, 0);
    R.sc[0] = v[0];
    R.sc[1] = v[1];
  }
  stage_store(R, lds, st_off, tid, false);
  codes_load(R, src, last < 1 ? last : 1);
  barrier_lds();
  Frags F0, F1;
  Scales Sc;
  scales_read(Sc, lds, a_row0, b_row0, sel);
  frags_read(F0, lds + a_lds, lds + b_lds, 0);

  // Iteration s computes stage s and stores stage s + 1 from registers.  Iterations come in
  // pairs: an even s stores the odd stage s + 1 from the upper half of the pair loaded two
  // iterations earlier and then loads the pair of stages s + 2 and s + 3; an odd s stores the
  // even stage s + 1 from the lower half of that pair (the upper half for the last stage of an
  // odd count, whose pair was moved back one stage) and loads no scales.  The body has no
  // branches, so the MFMAs stay where they are placed: past the last stage the loads repeat the
  // last stage (in bounds) and the stores and reads of the next buffer touch a buffer nobody
  // reads any more.
  auto body = [&](uint32_t s, auto even_tag) {
    constexpr bool kEven = decltype(even_tag)::value;
    uint8_t* cur = lds + (s & 1) * C::kStageBytes;
    uint8_t* nxt = lds + ((s + 1) & 1) * C::kStageBytes;
    frags_read(F1, cur + a_lds, cur + b_lds, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(acc, F0, Sc, 0);
    __builtin_amdgcn_sched_barrier(0);
    frags_read(F0, cur + a_lds, cur + b_lds, 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(acc, F1, Sc, 1);
    __builtin_amdgcn_sched_barrier(0);
    frags_read(F1, cur + a_lds, cur + b_lds, 3);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(acc, F0, Sc, 2);
    __builtin_amdgcn_sched_barrier(0);
    // the next buffer held stage s-1, which every wave finished reading before the previous
    // barrier; stage s+1 is in registers
    stage_store(R, nxt, st_off, tid, kEven ? true : s + 1 >= last);
    const uint32_t u = s + 2 < last ? s + 2 : last;
    codes_load(R, src, u);
    if (kEven) scale_pair_load(R, src, u, last);
    barrier_lds();
    frags_read(F0, nxt + a_lds, nxt + b_lds, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(acc, F1, Sc, 3);
    __builtin_amdgcn_sched_barrier(0);
    // the scale words of stage s+1 (their LDS latency runs under the next fragment reads)
    scales_read(Sc, nxt, a_row0, b_row0, sel);
  };
  uint32_t s = 0;
  for (; s + 1 < (uint32_t)nstage; s += 2) {
    body(s, std::true_type{});
    body(s + 1, std::false_type{});
  }
  if (s < (uint32_t)nstage) body(s, std::true_type{});

  // every wave's fragment reads completed before its last MFMAs; after this barrier the LDS is
  // free for the output staging (each wave its own 16 KB)
  barrier_lds();
  static_assert(C::kStoreBytes <= C::kLdsBytes, "output staging fits the LDS");
  gemm_store<FM, FN>(acc, 1.0f, lds + wave * gemm_store_bytes<FM, FN>(), lane, M, N, m_base,
                     n_base, nullptr, nullptr, Y, ldy);
}

// MXFP8 kernel: the codes go from global memory straight into LDS (global_load_lds), 128 elements
// of K per stage in a ring of two stages, 16-byte chunk c of a row stored at chunk c ^ ((row >> 1)
// & 7).  (The register-staged pipeline of the FP4 kernel needs twice the fragment registers with
// 8-bit codes and does not fit the register file at this tile shape.)
constexpr int kBK = 128;  // K per stage of this variant

template <int FP8>
struct DmaCfg {
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
__device__ __forceinline__ int dma_chunk_swz(int row) {
  return FP8 ? (row >> 1) & 7 : (row >> 2) & 3;
}


// This wave's share of one stage: code chunks (chunk id c of an operand: row c / kChunks, stored
// part c % kChunks holding logical part (c % kChunks) ^ f(row)); then, without CHUNK, the scale
// dwords of 64 rows (waves 0..3: A, 4..7: W).  Rows of A past M read row M-1 (never stored).
template <int FP8, bool CHUNK>
__device__ __forceinline__ void dma_stage_issue(uint8_t* buf, const uint8_t* __restrict__ A,
                                            const uint8_t* __restrict__ As,
                                            const uint8_t* __restrict__ B,
                                            const uint8_t* __restrict__ Bs, int64_t M, int64_t m0,
                                            int64_t n0, int64_t kb, int64_t ks, int64_t stage,
                                            int wave, int lane) {
  using C = DmaCfg<FP8>;
#pragma unroll
  for (int q = 0; q < C::kPerWave; ++q) {
    const int c = (wave * C::kPerWave + q) * 64 + lane;
    const int row = c / C::kChunks, part = (c % C::kChunks) ^ dma_chunk_swz<FP8>(row);
    int64_t ar = m0 + row;
    ar = ar < M ? ar : M - 1;
    __builtin_amdgcn_global_load_lds(
        (gvoid_t*)(A + ar * kb + stage * C::kRowBytes + part * 16),
        (lvoid_t*)(buf + (wave * C::kPerWave + q) * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(
        (gvoid_t*)(B + (n0 + row) * kb + stage * C::kRowBytes + part * 16),
        (lvoid_t*)(buf + C::kCodeBuf + (wave * C::kPerWave + q) * 1024), 16, 0, 0);
  }
  if (CHUNK) return;  // the scale words come four stages at a time (the kernel's chunk loads)
  const int srow = (wave & 3) * 64 + lane;
  int64_t sr = (wave < 4 ? m0 : n0) + srow;
  if (wave < 4) sr = sr < M ? sr : M - 1;
  __builtin_amdgcn_global_load_lds(
      (gvoid_t*)((wave < 4 ? As : Bs) + sr * ks + stage * (kBK / 32)),
      (lvoid_t*)(buf + 2 * C::kCodeBuf + (wave < 4 ? 0 : C::kScaleBuf) + (wave & 3) * 256), 4, 0,
      0);
}

template <int FP8, bool CHUNK>
__global__ __launch_bounds__(kThreads) void k_gemm_mx_dma(
    int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
    const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, const float* __restrict__ D,
    const uint16_t* __restrict__ up, int r, uint16_t* __restrict__ Y, int64_t ldy) {
  using C = DmaCfg<FP8>;
  constexpr int kFmt = FP8 ? 0 : 4;  // MFMA operand format: 0 E4M3, 4 E2M1
  // CHUNK: two chunk slots after the stages, each [A rows | W rows] x 16 bytes, and a third slot
  // that takes the chunk stores of the iterations that have nothing to store
  constexpr int kSlot = 2 * kBM * 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kStages * C::kStageBytes + (CHUNK ? 3 * kSlot : 0)];
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
  const int sw = dma_chunk_swz<FP8>(r32);
  int a_row[FM], b_row[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_row[i] = (wm * 128 + 32 * i + r32);
#pragma unroll
  for (int j = 0; j < FN; ++j) b_row[j] = (wn * 64 + 32 * j + r32);

  // CHUNK (at least four stages): thread tid fetches the scale words of its row (A row tid, or
  // W row tid - 256) for four stages at a time, one 16-byte request instead of four of 4 bytes
  // (a row's scale bytes are a request of their own, as many as its code bytes).  Chunk c covers
  // stages base(c) .. base(c) + 3 with base(c) = min(4c, nstage - 4), so that the load stays in
  // the row; it is loaded into registers in iteration 4c - 2 (the iteration's full wait lands
  // it), written to ring slot c % 2 at the top of iteration 4c - 1 (before that iteration's
  // barrier) and read in iterations 4c .. 4c + 3.  The slot held chunk c - 2, last read in
  // iteration 4c - 5.  Every iteration issues the store and the load, without a branch: the
  // other iterations store to the spare slot and load out of the resource's range (zeros, no
  // memory access).  A's rows past M read as zero through the range-checked resource (never
  // stored).
  uint8_t* ring = lds + C::kStages * C::kStageBytes;
  const bool s_a = __builtin_amdgcn_readfirstlane(wave) < 4;
  const int srow = tid & 255;
  const __amdgpu_buffer_rsrc_t s_rsrc =
      s_a ? rows_rsrc(As + m0 * ks, M - m0 < kBM ? M - m0 : kBM, (uint32_t)ks, 0)
          : rows_rsrc(Bs + n0 * ks, kBN, (uint32_t)ks, 0);
  const uint32_t ns = (uint32_t)nstage;
  auto chunk_base = [&](uint32_t c) { return 4 * c < ns - 4 ? 4 * c : ns - 4; };
  const uint32_t s_voff = (uint32_t)srow * (uint32_t)ks;
  // chunk c, or nothing (no memory access) when `go` is false
  auto chunk_load = [&](uint32_t c, bool go) {
    return __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(s_rsrc, go ? s_voff : kNoLoad,
                                                       (int)(go ? 4 * chunk_base(c) : 0), 0));
  };
  // A slot is stage-major: word (stage e of the chunk, row) at (e * 512 + row') * 4 with row' =
  // row (A) or 256 + row (W), so the per-stage reads of 32 consecutive rows hit distinct banks.
  const int ring_off = ((s_a ? 0 : kBM) + srow) * 4;
  // into the slot of chunk c, or the spare slot when `go` is false
  auto chunk_store = [&](const u32x4_t& v, uint32_t c, bool go) {
    uint8_t* dst = ring + (go ? (c & 1) : 2) * kSlot + ring_off;
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(dst + e * 2 * kBM * 4) = v[e];
  };

  // chunk 0 requested before the low-rank term, whose loads it overlaps; stored after the
  // prologue's wait
  u32x4_t chunk_regs = u32x4_t{0u, 0u, 0u, 0u};
  if (CHUNK) chunk_regs = chunk_load(0, true);

  f32x16_t acc[FM][FN];
  gemm_lowrank_init<FM, FN>(acc, 1.0f, M, m_base, n_base, r32, h, D, up, r);

  // prologue: stages 0 .. S-2 in flight, stage 0 landed
#pragma unroll
  for (int p = 0; p < C::kStages - 1; ++p)
    if (p < nstage)
      dma_stage_issue<FP8, CHUNK>(lds + p * C::kStageBytes, A, As, B, Bs, M, m0, n0, kb, ks, p, wave, lane);
  if (nstage >= C::kStages - 1)
    wait_vmcnt<(C::kStages - 2) * C::kLoads>();
  else
    wait_vmcnt<0>();
  if (CHUNK) chunk_store(chunk_regs, 0, true);
  barrier_lds();

  for (int64_t s = 0; s < nstage; ++s) {
    // stage s+S-1 into the buffer computed in the previous iteration (all waves passed the
    // barrier after it)
    if (s + C::kStages - 1 < nstage)
      dma_stage_issue<FP8, CHUNK>(lds + ((s + C::kStages - 1) % C::kStages) * C::kStageBytes, A, As, B, Bs,
                       M, m0, n0, kb, ks, s + C::kStages - 1, wave, lane);
    if (CHUNK) {
      chunk_store(chunk_regs, (uint32_t)(s + 1) >> 2, (s & 3) == 3 && s + 1 < nstage);
      chunk_regs = chunk_load((uint32_t)(s + 2) >> 2, (s & 3) == 2 && s + 2 < nstage);
    }
    const uint8_t* buf = lds + (s % C::kStages) * C::kStageBytes;
    // E8M0 bytes of the fragments' rows for the stage's four blocks; step t, lane h uses block
    // 2t + h
    uint32_t sa[FM], sb[FN];
    if (CHUNK) {
      const uint32_t su = (uint32_t)s;
      const uint8_t* slot =
          ring + ((su >> 2) & 1) * kSlot + (su - chunk_base(su >> 2)) * 2 * kBM * 4;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        sa[i] = *reinterpret_cast<const uint32_t*>(slot + a_row[i] * 4) >> (8 * h);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        sb[j] = *reinterpret_cast<const uint32_t*>(slot + (kBM + b_row[j]) * 4) >> (8 * h);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        sa[i] = *reinterpret_cast<const uint32_t*>(buf + 2 * C::kCodeBuf + a_row[i] * 4) >> (8 * h);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        sb[j] = *reinterpret_cast<const uint32_t*>(buf + 2 * C::kCodeBuf + C::kScaleBuf +
                                                   b_row[j] * 4) >> (8 * h);
    }
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
  if (fp8 && K >= 4 * kBK)  // at least four stages: scale words four stages at a time
    k_gemm_mx_dma<1, true><<<grid, dim3(kThreads), 0, s>>>(M, N, K, a_codes, a_scales, w_codes,
                                                           w_scales, D, up, (int)r, Y, ldy);
  else if (fp8)
    k_gemm_mx_dma<1, false><<<grid, dim3(kThreads), 0, s>>>(M, N, K, a_codes, a_scales, w_codes,
                                                            w_scales, D, up, (int)r, Y, ldy);
  else
    k_gemm_mxfp4<<<grid, dim3(kThreads), 0, s>>>(M, N, K, a_codes, a_scales, w_codes, w_scales,
                                                  D, up, (int)r, Y, ldy);
  return hipGetLastError();
}

}  // namespace svdq
