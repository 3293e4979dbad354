// Per-modality relative-L2 scoring against the unquantised bf16 layer ("MiniMax-H3 NVFP4 — what
// the smoothing scale should be calibrated on", section "The metric that picks the winner also
// hides the cost": relative L2 over a uniform sample of all rows and over each modality's rows).
//
// For the sampled rows, Y_ref = bf16(X·Wᵀ) is computed on bf16 MFMA (fp32 accumulation) with the
// X rows gathered by index (k_ref_rows).  Either the rows are stored (a sweep over several λ
// computes them once per batch: they do not depend on λ, and k_score_ref then scores each λ
// against them), or the epilogue forms (Y − Y_ref)² and Y_ref² per element and accumulates them
// per row group in fp64, adding each wave's eight sums to `sums`.  Both forms run the same MFMAs
// in the same order, so they see the same reference values.
#include "device.h"
#include "gemm_common.h"
#include "launch.h"

namespace svdq {

namespace {

// Sums against stored reference rows: sampled row i compares Y[rows[i], :] with Yref[i, :].  A
// wave takes one sampled row at a time (grid-stride over rows), its lanes 16-byte pieces of the
// two rows; each lane keeps fp64 sums per row group, the workgroup combines them in LDS and adds
// one value per (group, quantity) to `sums`.
__global__ __launch_bounds__(256) void k_score_ref(const uint16_t* __restrict__ Y, int64_t ldy,
                                                   const uint16_t* __restrict__ Yr, int64_t ldr,
                                                   int64_t M, int64_t N,
                                                   const int32_t* __restrict__ rows,
                                                   const int8_t* __restrict__ grp, int64_t n_rows,
                                                   double* __restrict__ sums) {
  __shared__ double red[4][8];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};  // [group][d2, r2]
  const int64_t n8 = N / 8;
  for (int64_t i = (int64_t)blockIdx.x * 4 + wave; i < n_rows; i += (int64_t)gridDim.x * 4) {
    int64_t m = rows[i];
    m = m < 0 ? 0 : (m < M ? m : M - 1);  // an out-of-range index reads a valid row
    const int g = grp[i];
    const u32x4_t* py = reinterpret_cast<const u32x4_t*>(Y + m * ldy);
    const u32x4_t* pr = reinterpret_cast<const u32x4_t*>(Yr + i * ldr);
    double d2 = 0.0, r2 = 0.0;
    for (int64_t p = lane; p < n8; p += 64) {
      const u32x4_t a = py[p], b = pr[p];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double r0 = (double)bf16_lo(b[e]), r1 = (double)bf16_hi(b[e]);
        const double e0 = (double)bf16_lo(a[e]) - r0, e1 = (double)bf16_hi(a[e]) - r1;
        d2 += e0 * e0 + e1 * e1;
        r2 += r0 * r0 + r1 * r1;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += q == g ? d2 : 0.0;
      acc[2 * q + 1] += q == g ? r2 : 0.0;
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    for (int off = 32; off > 0; off >>= 1) acc[q] += __shfl_xor(acc[q], off);
    if (lane == 0) red[wave][q] = acc[q];
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int q = threadIdx.x;
    const double v = (red[0][q] + red[1][q]) + (red[2][q] + red[3][q]);
    if (v != 0.0) atomicAdd(sums + q, v);
  }
}

// Reference rows on LDS-staged tiles (the store mode used for sweeps): workgroup tile 256
// sampled rows x 256 columns, 8 waves (two per SIMD) of 128 x 64, XCD-grouped tile order; K
// advances 64 per stage through two LDS buffers with one barrier per stage.  Each stage's bf16
// rows go global -> registers (one stage ahead; 8 lanes per 128-byte row, so every load
// instruction covers whole lines) -> LDS, chunk c of row R stored at c ^ swz(R), which keeps the
// 16-byte stores and the fragment reads (32 consecutive rows, one chunk) free of bank conflicts.
// The K mapping per MFMA is k_score's (lane h, step t: elements 32h + 8t .. + 8 of the stage),
// and the MFMAs run in the same order, so the rows are bit for bit those of k_score.
constexpr int kRThreads = 512;
constexpr int kRB = 256;                  // sampled rows and columns per workgroup tile
constexpr int kRRow = 128;                // bytes of a row per stage (64 bf16)
constexpr int kROp = kRB * kRRow;         // one operand, one buffer: 32 KB
constexpr int kRBuf = 2 * kROp;           // A then W

__device__ __forceinline__ int rswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ void rbarrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// kSums: instead of storing the rows, add Σ(Y[rows[i], n] − Y_ref[i, n])² and Σ Y_ref[i, n]² per
// row group to sums (fp64; one atomic per wave, group and quantity).
template <bool kSums>
__global__ __launch_bounds__(kRThreads) void k_ref_rows(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ W, int64_t ldw,
    int64_t M, int64_t N, int64_t K, const int32_t* __restrict__ rows, int64_t n_rows,
    uint16_t* __restrict__ Yr, int64_t ldr, const uint16_t* __restrict__ Y, int64_t ldy,
    const int8_t* __restrict__ grp, double* __restrict__ sums) {
  constexpr int FM = 4, FN = 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kRBuf];
  int64_t tm, tn;
  if (!tile_of_block((n_rows + kRB - 1) / kRB, N / kRB, tm, tn)) return;
  const int64_t i0 = tm * kRB, n0 = tn * kRB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int r32 = lane & 31, h = lane >> 5;
  const int64_t nstage = K / 64;

  // staging share: piece tid + 512 q (q = 0..3) of each operand, i.e. row tid / 8 + 64 q,
  // chunk tid % 8; the swizzle depends on the row's low four bits only, the same for every q
  const int prow = tid >> 3, pc = tid & 7;
  const int soff = prow * kRRow + 16 * (pc ^ rswz(prow));
  const uint16_t* pa[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int64_t idx = i0 + prow + 64 * q;
    idx = idx < n_rows ? idx : n_rows - 1;
    int64_t m = rows[idx];
    m = m < 0 ? 0 : (m < M ? m : M - 1);  // an out-of-range index reads a valid row
    pa[q] = X + m * ldx + 8 * pc;
  }
  const uint16_t* pw = W + (n0 + prow) * ldw + 8 * pc;
  u32x4_t ra[4], rw[4];
  auto load = [&](int64_t st) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = *reinterpret_cast<const u32x4_t*>(pa[q] + st * 64);
      rw[q] = *reinterpret_cast<const u32x4_t*>(pw + (int64_t)q * 64 * ldw + st * 64);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<u32x4_t*>(lds + buf * kRBuf + soff + q * 64 * kRRow) = ra[q];
      *reinterpret_cast<u32x4_t*>(lds + buf * kRBuf + kROp + soff + q * 64 * kRRow) = rw[q];
    }
  };
  // fragment bases: step t of the lane's row is logical chunk 4h + t
  const int x = rswz(r32);
  const int fa = (wm * 128 + r32) * kRRow, fb = kROp + (wn * 64 + r32) * kRRow;
  bf16x8_t a_op[FM], b_op[FN];
  auto read_frags = [&](int buf, int t, bf16x8_t (&fa_)[FM], bf16x8_t (&fb_)[FN]) {
    const int c = 16 * ((4 * h + t) ^ x);
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa_[i] = *reinterpret_cast<const bf16x8_t*>(lds + buf * kRBuf + fa + i * 32 * kRRow + c);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb_[j] = *reinterpret_cast<const bf16x8_t*>(lds + buf * kRBuf + fb + j * 32 * kRRow + c);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int64_t last = nstage - 1;
  load(0);
  store(0);
  load(last < 1 ? last : 1);
  rbarrier();
  read_frags(0, 0, a_op, b_op);
  for (int64_t s = 0; s < nstage; ++s) {
    const int cur = (int)(s & 1), nxt = cur ^ 1;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8_t na[FM], nb[FN];
      if (t < 3) read_frags(cur, t + 1, na, nb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_op[i], b_op[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (t == 1) {
        // the next buffer held stage s-1, which every wave finished reading before the
        // previous barrier; stage s+1 is in registers, stage s+2 is requested
        store(nxt);
        load(s + 2 < last ? s + 2 : last);
      }
      if (t < 3) {
#pragma unroll
        for (int i = 0; i < FM; ++i) a_op[i] = na[i];
#pragma unroll
        for (int j = 0; j < FN; ++j) b_op[j] = nb[j];
      }
    }
    rbarrier();
    read_frags(nxt, 0, a_op, b_op);
  }
  if (kSums) {
    // 32x32 accumulator layout: lane holds column r32 and rows (e/4)*8 + 4h + e%4
    double sd[4] = {0.0, 0.0, 0.0, 0.0}, sr[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t idx = i0 + wm * 128 + 32 * i + (e >> 2) * 8 + 4 * h + (e & 3);
        if (idx < n_rows) {
          int64_t m = rows[idx];
          m = m < 0 ? 0 : (m < M ? m : M - 1);
          const int gsel = grp[idx];
          double d2 = 0.0, r2 = 0.0;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const float yref = bf16_to_f32(f32_to_bf16(acc[i][j][e]));
            const float y = bf16_to_f32(Y[m * ldy + n0 + wn * 64 + 32 * j + r32]);
            const double d = (double)y - (double)yref;
            d2 += d * d;
            r2 += (double)yref * (double)yref;
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            sd[g] += gsel == g ? d2 : 0.0;
            sr[g] += gsel == g ? r2 : 0.0;
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      for (int off = 32; off > 0; off >>= 1) {
        sd[g] += __shfl_xor(sd[g], off);
        sr[g] += __shfl_xor(sr[g], off);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (sd[g] != 0.0) atomicAdd(sums + 2 * g, sd[g]);
        if (sr[g] != 0.0) atomicAdd(sums + 2 * g + 1, sr[g]);
      }
    }
    return;
  }
  // every wave's last fragment reads completed before the final barrier: the buffers are free
  // for the output staging (each wave its own 16 KB)
  static_assert(8 * gemm_store_bytes<FM, FN>() <= 2 * kRBuf, "output staging fits the LDS");
  gemm_store<FM, FN>(acc, 1.0f, lds + wave * gemm_store_bytes<FM, FN>(), lane, n_rows, N,
                     i0 + wm * 128, n0 + wn * 64, nullptr, nullptr, Yr, ldr);
}

}  // namespace

hipError_t launch_score_ref(const uint16_t* Y, int64_t ldy, const uint16_t* Yref, int64_t ldr,
                            int64_t M, int64_t N, const int32_t* rows, const int8_t* grp,
                            int64_t n_rows, double* sums, hipStream_t s) {
  int64_t blocks = (n_rows + 3) / 4;
  blocks = blocks < 2048 ? blocks : 2048;
  k_score_ref<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(Y, ldy, Yref, ldr, M, N, rows, grp,
                                                           n_rows, sums);
  return hipGetLastError();
}

hipError_t launch_score(const uint16_t* Y, int64_t ldy, const uint16_t* X, int64_t ldx,
                        const uint16_t* W, int64_t ldw, int64_t M, int64_t N, int64_t K,
                        const int32_t* rows, const int8_t* grp, int64_t n_rows, double* sums,
                        hipStream_t s) {
  // (N is a multiple of 256 and K of 64, as the entry point requires)
  const dim3 grid(grid_of_tiles((n_rows + kRB - 1) / kRB, N / kRB));
  k_ref_rows<true><<<grid, dim3(kRThreads), 0, s>>>(X, ldx, W, ldw, M, N, K, rows, n_rows,
                                                    nullptr, 0, Y, ldy, grp, sums);
  return hipGetLastError();
}

hipError_t launch_reference_rows(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                                 int64_t M, int64_t N, int64_t K, const int32_t* rows,
                                 int64_t n_rows, uint16_t* Yref, int64_t ldr, hipStream_t s) {
  // (N is a multiple of 256 and K of 64, as the entry points require)
  const dim3 grid(grid_of_tiles((n_rows + kRB - 1) / kRB, N / kRB));
  k_ref_rows<false><<<grid, dim3(kRThreads), 0, s>>>(X, ldx, W, ldw, M, N, K, rows, n_rows,
                                                     Yref, ldr, nullptr, 0, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace svdq
