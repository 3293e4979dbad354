// GPTQ rounding of the low-rank branch's residual ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32,
// GPTQ)", opening paragraph: the residual is GPTQ-rounded; GPTQ as published by Frantar et al.
// 2022: columns quantised in order, each column's rounding error compensated in the columns not
// yet quantised through the inverse Hessian).
//
// Hessian: H = Σ_m x̂_m x̂_mᵀ with x̂ = fl32(x · fl32(1/λ)), in fp64 (each product of two fp32
// values is exact), 64 x 64 tiles of the lower triangle mirrored to the upper.
//
// The sweep without an inverse.  With H = Ũ Ũᵀ, Ũ upper triangular (the Cholesky factor taken
// from the last row up), the published update (error of column j over the diagonal of the upper
// Cholesky factor of H⁻¹, along that factor's row) adds up to
//     w̃_k = w_k + Σ_{j<k} (w_j − q_j) · C_jk,      C_jk = Ũ_jk / Ũ_kk,
// where w is the residual before the sweep and q_j the dequantised code of column j: writing
// the published sweep's errors e and its unit-diagonal factor V (row j of the factor over its
// diagonal), w̃ = w − e(V − I) and e = w̃ − q give e·V = w − q, and V⁻¹ = Ũ·diag(1/Ũ_kk)
// column-normalised because the factor of H⁻¹ is Ũ⁻¹.  So only one Cholesky factorisation is
// needed: Ũ is the lower Cholesky factor of the index-reversed H, reversed back.
//
// Steps on the device, all fp64 except the fp32 residual and the quantiser:
//   damping H + 0.01 · mean(diag H) · I, copied index-reversed;  blocked lower Cholesky
//   (64-column panels: a one-workgroup diagonal factor, a forward-substituted panel, a rank-64
//   update of the trailing lower triangle);  C;  R32 (as the round-to-nearest path) and, for
//   NVFP4, its tensor scale;  then per block of 64 columns: 16 lanes per weight row quantise
//   the block's columns in order, keep w̃ of the block in registers and update it in-block,
//   and write the block's w − q;  a rank-64 product adds those to the running sums
//   T of all later columns.  A group's scale is fixed at its first column from the values the
//   published sweep holds there; those differ from the partial sums above for every column but
//   the first, and are recovered by a forward substitution inside the group (see the block
//   kernel).
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kB = 64;           // panel / sweep block width
typedef __attribute__((ext_vector_type(2))) double f64x2_t;
constexpr double kPercDamp = 0.01;
constexpr int kSuper = 4 * kB;   // columns whose w − q are carried to the later columns at once

int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// H (+)= X̂ᵀX̂ on one lower tile (ti >= tj) of 64 x 64, mirrored.  Thread (ty, tx) = 4 x 4
// outputs; rows of X̂ staged 32 at a time as fp32.
__global__ __launch_bounds__(256) void k_hessian(const uint16_t* __restrict__ X, int64_t M,
                                                 int64_t K, int64_t ldx,
                                                 const float* __restrict__ lambda,
                                                 int accumulate, double* __restrict__ H) {
  __shared__ float xi[32][kB];
  __shared__ float xj[32][kB];
  const int64_t b = blockIdx.x;
  int64_t ti = (int64_t)((__builtin_sqrt(8.0 * (double)b + 1.0) - 1.0) * 0.5);
  while (ti * (ti + 1) / 2 > b) --ti;
  while ((ti + 1) * (ti + 2) / 2 <= b) ++ti;
  const int64_t tj = b - ti * (ti + 1) / 2;
  const int64_t i0 = ti * kB, j0 = tj * kB;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0;
  for (int64_t m0 = 0; m0 < M; m0 += 32) {
    __syncthreads();
    for (int t = tid; t < 32 * kB; t += 256) {
      const int rr = t / kB, cc = t % kB;
      const int64_t m = m0 + rr;
      float vi = 0.0f, vj = 0.0f;
      if (m < M) {
        const float li = lambda ? 1.0f / lambda[i0 + cc] : 1.0f;
        const float lj = lambda ? 1.0f / lambda[j0 + cc] : 1.0f;
        vi = bf16_to_f32(X[m * ldx + i0 + cc]) * li;
        vj = bf16_to_f32(X[m * ldx + j0 + cc]) * lj;
      }
      xi[rr][cc] = vi;
      xj[rr][cc] = vj;
    }
    __syncthreads();
    const int mn = M - m0 < 32 ? (int)(M - m0) : 32;
    for (int mm = 0; mm < mn; ++mm) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&xi[mm][ty * 4]);
      const f32x4_t c = *reinterpret_cast<const f32x4_t*>(&xj[mm][tx * 4]);
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = __builtin_fma((double)a[p], (double)c[q], acc[p][q]);
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = i0 + ty * 4 + p, j = j0 + tx * 4 + q;
      double v = acc[p][q];
      if (accumulate) v += H[i * K + j];
      H[i * K + j] = v;
      if (ti != tj) H[j * K + i] = v;   // the mirrored entry: same sum, same order
    }
}

// damp = 0.01 · mean(diag H), or −1 when the diagonal is all zero (H taken as the identity)
__global__ __launch_bounds__(256) void k_damping(const double* __restrict__ H, int64_t K,
                                                 double* __restrict__ damp) {
  __shared__ double red[4];
  double s = 0.0;
  for (int64_t k = threadIdx.x; k < K; k += 256) s += H[k * K + k];
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double t = (red[0] + red[1]) + (red[2] + red[3]);
    *damp = t == 0.0 ? -1.0 : kPercDamp * (t / (double)K);
  }
}

// A[i][j] = Hd[K−1−i][K−1−j]: the damped Hessian with its indices reversed
__global__ __launch_bounds__(256) void k_reverse_damped(const double* __restrict__ H, int64_t K,
                                                        const double* __restrict__ damp,
                                                        double* __restrict__ A) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= K * K) return;
  const int64_t i = t / K, j = t % K;
  const double d = *damp;
  double v;
  if (d < 0.0) {
    v = i == j ? 1.0 : 0.0;
  } else {
    v = H[(K - 1 - i) * K + (K - 1 - j)];
    if (i == j) v += d;
  }
  A[t] = v;
}

// Lane l's value of x, as a wave-uniform value (l a compile-time constant after unrolling).
__device__ __forceinline__ double lane_value(double x, int l) {
  const int2 v = __builtin_bit_cast(int2, x);
  return __builtin_bit_cast(double, int2{__builtin_amdgcn_readlane(v.x, l),
                                         __builtin_amdgcn_readlane(v.y, l)});
}

// Unblocked Cholesky of the 64 x 64 diagonal block at (j0, j0) in one wave: lane i holds row i
// in registers; each step takes the pivot and the scaled column from their lanes as uniform
// values, so a step costs no barrier.  The upper part is written as zeros.
__global__ __launch_bounds__(64) void k_chol_diag(double* __restrict__ A, int64_t K, int64_t j0) {
  const int i = threadIdx.x;
  double* rowp = A + (j0 + i) * K + j0;
  double a[kB];
#pragma unroll
  for (int j = 0; j < kB; j += 2) {
    const f64x2_t v = *reinterpret_cast<const f64x2_t*>(rowp + j);
    a[j] = v[0];
    a[j + 1] = v[1];
  }
#pragma unroll
  for (int c = 0; c < kB; ++c) {
    const double d = __builtin_sqrt(lane_value(a[c], c));
    if (i == c) a[c] = d;
    if (i > c) a[c] = a[c] / d;
#pragma unroll
    for (int j = c + 1; j < kB; ++j) {
      const double ajc = lane_value(a[c], j);
      if (i >= j) a[j] = a[j] - a[c] * ajc;
    }
  }
#pragma unroll
  for (int j = 0; j < kB; j += 2)
    *reinterpret_cast<f64x2_t*>(rowp + j) = f64x2_t{j <= i ? a[j] : 0.0, j + 1 <= i ? a[j + 1] : 0.0};
}

// Panel rows i >= j0 + 64: L[i, j0 .. j0+64) by forward substitution against the factored
// diagonal block; one thread per row.
__global__ __launch_bounds__(64) void k_chol_panel(double* __restrict__ A, int64_t K, int64_t j0) {
  __shared__ double l[kB][kB + 1];
  const int tid = threadIdx.x;
  for (int t = tid; t < kB * kB; t += 64) l[t / kB][t % kB] = A[(j0 + t / kB) * K + j0 + t % kB];
  __syncthreads();
  const int64_t i = j0 + kB + (int64_t)blockIdx.x * 64 + tid;
  if (i >= K) return;
  double* row = A + i * K + j0;
  double x[kB];
#pragma unroll
  for (int c = 0; c < kB; ++c) x[c] = row[c];
#pragma unroll
  for (int c = 0; c < kB; ++c) {
    double v = x[c];
#pragma unroll
    for (int p = 0; p < c; ++p) v = __builtin_fma(-x[p], l[c][p], v);
    x[c] = v / l[c][c];
  }
#pragma unroll
  for (int c = 0; c < kB; ++c) row[c] = x[c];
}

// Out[i][j] += sign · Σ_{c < 64 nchunk} A[i][c] · B(c, j) on 64 x 64 output tiles, B(c, j) = B[c][j]
// (row-major, ldb) or, TRANSB, Bt[j][c].  LOWER: tiles above the diagonal (tile row < tile
// column) are skipped.  Thread (ty, tx) = 4 x 4 outputs; both operands staged in LDS with the
// output index contiguous.
template <bool TRANSB, bool LOWER>
__global__ __launch_bounds__(256) void k_rank64(const double* __restrict__ A, int64_t lda,
                                                const double* __restrict__ B, int64_t ldb,
                                                double* __restrict__ Out, int64_t ldo,
                                                double sign, int nchunk) {
  if (LOWER && blockIdx.y < blockIdx.x) return;
  __shared__ double as[kB][kB + 2];   // as[c][i]
  __shared__ double bs[kB][kB + 2];   // bs[c][j]
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t i0 = (int64_t)blockIdx.y * kB, j0 = (int64_t)blockIdx.x * kB;
  double acc[4][4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[p][q] = 0.0;
  // the inner dimension is nchunk x 64, staged 64 at a time
  for (int ch = 0; ch < nchunk; ++ch) {
    const int64_t c0 = (int64_t)ch * kB;
    __syncthreads();
    for (int t = tid; t < kB * kB; t += 256) {
      const int r = t / kB, c = t % kB;
      as[c][r] = A[(i0 + r) * lda + c0 + c];
      if (TRANSB) bs[c][r] = B[(j0 + r) * ldb + c0 + c];
      else bs[r][c] = B[(c0 + r) * ldb + j0 + c];
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < kB; ++c) {
      double a[4], b[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        a[p] = as[c][ty * 4 + p];
        b[p] = bs[c][tx * 4 + p];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = __builtin_fma(a[p], b[q], acc[p][q]);
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      double* o = Out + (i0 + ty * 4 + p) * ldo + j0 + tx * 4 + q;
      *o = __builtin_fma(sign, acc[p][q], *o);
    }
}

// C[j][k] = Ũ_jk / Ũ_kk for j < k (else 0), Ũ_jk = L[K−1−j][K−1−k]
__global__ __launch_bounds__(256) void k_make_c(const double* __restrict__ L, int64_t K,
                                                double* __restrict__ C) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= K * K) return;
  const int64_t j = t / K, k = t % K;
  C[t] = j < k ? L[(K - 1 - j) * K + (K - 1 - k)] / L[(K - 1 - k) * K + (K - 1 - k)] : 0.0;
}

__global__ __launch_bounds__(256) void k_fill_f64(double* __restrict__ p, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n) p[t] = 0.0;
}

// Scale of one quantiser group from the fp32 values x[0 .. G) of a row, and the element rule.
template <int FMT>
struct GroupQuant {
  float inv;        // NVFP4 / int4: inverse block scale
  double mult;      // exact value of one code unit
  int ex;           // MX exponent
  uint32_t stored;  // the stored scale (E4M3 byte, fp16 bits or E8M0 byte)

  __device__ __forceinline__ void set(float a, float g) {
    if (FMT == 0) {
      const float d6 = 6.0f * g;
      float sval;
      stored = e4m3_encode_pos(a / d6, &sval);
      const float S = sval * g;
      inv = S != 0.0f ? 1.0f / S : 0.0f;
      mult = (double)sval * (double)g;
    } else if (FMT == 1) {
      const __half s = __float2half_rn(a / 7.0f);
      const float sf = __half2float(s);
      inv = sf != 0.0f ? 1.0f / sf : 0.0f;
      mult = (double)sf;
      stored = (uint32_t)__builtin_bit_cast(uint16_t, s);
    } else {
      ex = mx_exponent(a, FMT == 2 ? 2 : 8);
      mult = ldexp(1.0, ex);
      stored = (uint32_t)(ex + 127);
    }
  }
  // element code of x and its exact value
  __device__ __forceinline__ uint32_t code(float x, double* val) const {
    if (FMT == 0 || FMT == 2) {
      const float y = FMT == 0 ? x * inv : __builtin_ldexpf(x, -ex);
      const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, 0.0f, 1.0f, 0) & 0xFu;
      *val = (FMT == 0 && inv == 0.0f) ? 0.0 : e2m1_value(c) * mult;
      return (FMT == 0 && inv == 0.0f) ? (c & 8u) : c;
    } else if (FMT == 1) {
      const uint32_t c = int4_code(x * inv);
      *val = (double)((int)c - (c >= 8u ? 16 : 0)) * mult;
      return c;
    } else {
      const uint32_t c = e4m3_encode_signed(__builtin_ldexpf(x, -ex));
      *val = e4m3_value(c) * mult;
      return c;
    }
  }
};

// One block of 64 columns of the sweep: 16 lanes per weight row, lane s of a row holding the
// columns 4s .. 4s + 3 of the block in registers (the residual w and the running value w̃).
// Column m is quantised by its owner lane and its w − q broadcast to the row's lanes, which fold
// it into their later columns with the in-block coefficients C[b0 + m][b0 + c] (shared by the
// workgroup in LDS).  At a group's first column the group's values as the published sweep holds
// them are recovered by the forward substitution z_j = y_j − Σ_{m<=l<j} C_lj·z_l (y = w̃ − w),
// one broadcast per column, and the group maximum by shuffles across the row's lanes.
template <int FMT>
__global__ __launch_bounds__(256) void k_gptq_block(const float* __restrict__ R32,
                                                    const double* __restrict__ T,
                                                    const double* __restrict__ C, int64_t N,
                                                    int64_t K, int64_t b0,
                                                    const float* __restrict__ tensor_g,
                                                    uint8_t* __restrict__ codes,
                                                    void* __restrict__ scales,
                                                    double* __restrict__ D, int64_t ldd) {
  constexpr int G = FMT == 0 ? 16 : (FMT == 1 ? 64 : 32);
  constexpr int GL = G / 4;   // lanes of a group
  __shared__ double cb[kB][kB + 1];
  const int tid = threadIdx.x;
  for (int t = tid; t < kB * kB; t += 256) cb[t / kB][t % kB] = C[(b0 + t / kB) * K + b0 + t % kB];
  __syncthreads();
  const int lane = tid & 63;
  const int sub = lane & 15, rbase = lane & 48;
  const int64_t n = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const bool live = n < N;
  const int64_t row = live ? n : N - 1;
  const int64_t off = row * K + b0 + 4 * sub;
  double w[4], v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w[e] = (double)R32[off + e];
    v[e] = w[e] + T[off + e];
  }
  const float g = FMT == 0 ? *tensor_g : 1.0f;
  GroupQuant<FMT> gq;
  uint32_t packed = 0u;
  for (int q = 0; q < kB / 4; ++q) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * q + e;
      if (e == 0 && q % GL == 0) {
        // group entry at column m: z over the group's columns (lanes q .. q + GL - 1)
        double y[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) y[k] = v[k] - w[k];
        for (int jq = 0; jq < GL; ++jq) {
#pragma unroll
          for (int ej = 0; ej < 4; ++ej) {
            const int j = m + 4 * jq + ej;   // block column, final in its owner after this
            const double zj = __shfl(y[ej], rbase + q + jq);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int c = 4 * sub + k;
              if (c > j && c < m + G) y[k] = __builtin_fma(-cb[j][c], zj, y[k]);
            }
          }
        }
        float a = 0.0f;
        if (sub >= q && sub < q + GL) {
#pragma unroll
          for (int k = 0; k < 4; ++k) a = fmaxf(a, fabsf((float)(w[k] + y[k])));
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
        gq.set(a, g);
        if (live && sub == q) {
          const int64_t gi = (b0 + m) / G;
          if (FMT == 1)
            reinterpret_cast<uint16_t*>(scales)[n * (K / G) + gi] = (uint16_t)gq.stored;
          else
            reinterpret_cast<uint8_t*>(scales)[n * (K / G) + gi] = (uint8_t)gq.stored;
        }
      }
      // column m: its owner's code; w − q to every lane of the row
      double qv;
      const uint32_t c = gq.code((float)v[e], &qv);
      const double d_own = w[e] - qv;
      if (sub == q) {
        packed |= FMT == 3 ? c << (8 * e) : c << (4 * e);
        if (live) D[n * ldd + m] = d_own;
      }
      const double d = __shfl(d_own, rbase + q);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int col = 4 * sub + k;
        if (col > m) v[k] = __builtin_fma(d, cb[m][col], v[k]);
      }
    }
  }
  if (!live) return;
  if (FMT == 3)
    *reinterpret_cast<uint32_t*>(codes + n * K + b0 + 4 * sub) = packed;
  else
    *reinterpret_cast<uint16_t*>(codes + n * (K / 2) + (b0 + 4 * sub) / 2) = (uint16_t)packed;
}

struct GptqWs {
  double *A, *C, *T, *D, *damp;
  float* R32;
  int64_t bytes;
};

GptqWs carve(void* base, int64_t N, int64_t K) {
  uint8_t* b = static_cast<uint8_t*>(base);
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    void* p = b ? b + off : nullptr;
    off += align256(bytes);
    return p;
  };
  GptqWs w;
  w.A = static_cast<double*>(take(K * K * 8));
  w.C = static_cast<double*>(take(K * K * 8));
  w.T = static_cast<double*>(take(N * K * 8));
  w.D = static_cast<double*>(take(N * kSuper * 8));
  w.R32 = static_cast<float*>(take(N * K * 4));
  w.damp = static_cast<double*>(take(8));
  w.bytes = off;
  return w;
}

}  // namespace

hipError_t launch_gptq_hessian(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                               const float* lambda, int accumulate, double* H, hipStream_t s) {
  const int64_t T = K / kB;
  k_hessian<<<dim3((unsigned)(T * (T + 1) / 2)), dim3(256), 0, s>>>(X, M, K, ldx, lambda,
                                                                   accumulate, H);
  return hipGetLastError();
}

int64_t gptq_workspace_bytes(int64_t N, int64_t K) { return carve(nullptr, N, K).bytes; }

hipError_t launch_gptq_quantize_weight(int fmt, const uint16_t* W, int64_t N, int64_t K,
                                       int64_t ldw, const float* lambda, const uint16_t* down,
                                       const uint16_t* up, int64_t r, const double* H,
                                       uint8_t* codes, void* scales, float* tensor_scale,
                                       void* workspace, hipStream_t s) {
  const GptqWs w = carve(workspace, N, K);
  hipError_t e;
#define SVDQ_TRY_HIP(x)                    \
  do {                                     \
    if ((e = (x)) != hipSuccess) return e; \
  } while (0)
  // Ũ from the index-reversed damped Hessian
  k_damping<<<dim3(1), dim3(256), 0, s>>>(H, K, w.damp);
  SVDQ_TRY_HIP(hipGetLastError());
  k_reverse_damped<<<dim3((unsigned)ceil_div(K * K, 256)), dim3(256), 0, s>>>(H, K, w.damp, w.A);
  SVDQ_TRY_HIP(hipGetLastError());
  for (int64_t j0 = 0; j0 < K; j0 += kB) {
    k_chol_diag<<<dim3(1), dim3(64), 0, s>>>(w.A, K, j0);
    SVDQ_TRY_HIP(hipGetLastError());
    const int64_t rest = K - j0 - kB;
    if (rest > 0) {
      k_chol_panel<<<dim3((unsigned)ceil_div(rest, 64)), dim3(64), 0, s>>>(w.A, K, j0);
      SVDQ_TRY_HIP(hipGetLastError());
      const unsigned tiles = (unsigned)(rest / kB);
      const int64_t p = (j0 + kB) * K + j0;   // the panel rows below the diagonal block
      k_rank64<true, true><<<dim3(tiles, tiles), dim3(256), 0, s>>>(
          w.A + p, K, w.A + p, K, w.A + (j0 + kB) * K + j0 + kB, K, -1.0, 1);
      SVDQ_TRY_HIP(hipGetLastError());
    }
  }
  k_make_c<<<dim3((unsigned)ceil_div(K * K, 256)), dim3(256), 0, s>>>(w.A, K, w.C);
  SVDQ_TRY_HIP(hipGetLastError());
  // the residual (the round-to-nearest path's own kernel), the NVFP4 tensor scale, and T = 0
  SVDQ_TRY_HIP(launch_residual_f32(W, N, K, ldw, lambda, down, up, r, w.R32,
                                   fmt == 0 ? tensor_scale : nullptr, s));
  k_fill_f64<<<dim3((unsigned)ceil_div(N * K, 256)), dim3(256), 0, s>>>(w.T, N * K);
  SVDQ_TRY_HIP(hipGetLastError());
  // the sweep.  Blocks are grouped in super-blocks of 256 columns: after a block, its w − q is
  // carried only into the rest of its super-block; at the end of a super-block the w − q of all
  // its columns is carried into every later column in one rank-256 update (the running sums T
  // are rewritten once per super-block instead of once per block).
  const dim3 rows_grid((unsigned)ceil_div(N, 16));
  for (int64_t b0 = 0; b0 < K; b0 += kB) {
    const int64_t sb0 = b0 - b0 % kSuper, sb1 = sb0 + kSuper < K ? sb0 + kSuper : K;
    double* Db = w.D + (b0 - sb0);
    if (fmt == 0)
      k_gptq_block<0><<<rows_grid, dim3(256), 0, s>>>(w.R32, w.T, w.C, N, K, b0, tensor_scale,
                                                      codes, scales, Db, kSuper);
    else if (fmt == 1)
      k_gptq_block<1><<<rows_grid, dim3(256), 0, s>>>(w.R32, w.T, w.C, N, K, b0, nullptr, codes,
                                                      scales, Db, kSuper);
    else if (fmt == 2)
      k_gptq_block<2><<<rows_grid, dim3(256), 0, s>>>(w.R32, w.T, w.C, N, K, b0, nullptr, codes,
                                                      scales, Db, kSuper);
    else
      k_gptq_block<3><<<rows_grid, dim3(256), 0, s>>>(w.R32, w.T, w.C, N, K, b0, nullptr, codes,
                                                      scales, Db, kSuper);
    SVDQ_TRY_HIP(hipGetLastError());
    const int64_t in_sb = sb1 - (b0 + kB);   // later columns of this super-block
    if (in_sb > 0) {
      k_rank64<false, false><<<dim3((unsigned)(in_sb / kB), (unsigned)(N / kB)), dim3(256), 0, s>>>(
          Db, kSuper, w.C + b0 * K + b0 + kB, K, w.T + b0 + kB, K, 1.0, 1);
      SVDQ_TRY_HIP(hipGetLastError());
    } else if (K - sb1 > 0) {
      k_rank64<false, false><<<dim3((unsigned)((K - sb1) / kB), (unsigned)(N / kB)), dim3(256), 0,
                               s>>>(w.D, kSuper, w.C + sb0 * K + sb1, K, w.T + sb1, K, 1.0,
                                    (int)((sb1 - sb0) / kB));
      SVDQ_TRY_HIP(hipGetLastError());
    }
  }
#undef SVDQ_TRY_HIP
  return hipSuccess;
}

}  // namespace svdq
