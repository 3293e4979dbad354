// Randomized rank-r factors of the smoothed weight A = diag(λ)·Wᵀ (K x N) on the GPU: the branch
// the layer adds in 16 bits ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening
// paragraph).  The pages give no method for computing it; this is the randomized range finder
// with power iterations followed by a small SVD (Halko, Martinsson and Tropp 2011, Algorithms 4.4
// and 5.1):
//   Y = A Ω, Q = orth(Y); q times: Q = orth(A · orth(Aᵀ Q));  Z = Aᵀ Q  (= Bᵀ, B = Qᵀ A)
//   ZᵀZ = B Bᵀ = U Σ² Uᵀ;  L1 = Q U_r Σ_r (K x r);  L2 = (Z U_r Σ_r⁻¹)ᵀ (r x N)
// Ω (N x ℓ) is the caller's.  The large products are fp32 (bf16 W exact, fp32 fused
// multiply-adds) split over their reduction dimension, the splits summed in a fixed order
// (deterministic).  orth() is Cholesky-QR applied twice: Gram matrix in fp64 from fp32 rows,
// Cholesky and triangular inverse in fp64 (one workgroup), rows times the inverse in fp64.  The
// ℓ x ℓ eigenproblem is parallel cyclic Jacobi in fp64 (one workgroup, round-robin pairs).
// None of this is on the layer's per-batch path; it prepares the factors that
// svdq_quantize_weight and the GEMM take.
#include "device.h"
#include "launch.h"

namespace svdq {

namespace {

constexpr int kMaxEll = 160;
constexpr int kColTile = 40;       // columns of the sketch handled by one thread
constexpr int kSplitWt = 128;      // reduction rows (of W) per partial sum of Wᵀ·X
constexpr int kSplitW = 256;       // reduction channels per partial sum of W·Q
constexpr int kGramRows = 64;      // rows per partial Gram matrix
constexpr int kJacobiThreads = 1024;
constexpr int kMaxSweeps = 40;
constexpr int kLdsEll = 80;        // the small factorisations run in LDS up to this ell
constexpr int kCholThreads = 512;  // threads of the small Cholesky-inverse workgroup
constexpr int kJacHLdsEll = 138;   // the Jacobi eigensolver keeps H in LDS up to this ell
constexpr int kJacVLdsEll = 64;    // and V as well up to this ell
constexpr int kJacItems = (kMaxEll / 2 * kMaxEll + kJacobiThreads - 1) / kJacobiThreads;  // per thread and pass
// odd row pitch of the Jacobi H in LDS: a column of H then spreads over the banks
__host__ __device__ constexpr int jacobi_pitch(int ell) { return ell | 1; }

// The matrix is either the bf16 weight (scaled by λ per channel) or an fp32 matrix (the refit
// target of the layer's low-rank branch).

// Stage a ROWS x COLS tile of W (rows r0 .. r_end, columns c0 .. c_end; the rest reads as 0)
// into LDS as fp32 with 16-byte loads, all of a thread's loads in flight before the first
// store.  COLS and c0 are multiples of the elements per 16 bytes and the rows are 16-byte
// aligned (ldw a multiple of 8); a 16-byte piece that crosses c_end is read element by element.
template <typename T, int ROWS, int COLS>
struct TileBuf {
  static constexpr int V = 16 / (int)sizeof(T);       // elements per 16 bytes
  static constexpr int PER = ROWS * COLS / V / 256;    // 16-byte loads per thread
  static_assert(PER * 256 * V == ROWS * COLS, "tile must split evenly over 256 threads");
  u32x4_t v[PER];
};

// Load a ROWS x COLS tile of W (rows r0 .. r_end, columns c0 .. c_end; the rest reads as 0) into
// registers with 16-byte loads.  COLS and c0 are multiples of the elements per 16 bytes and the
// rows are 16-byte aligned (ldw a multiple of 8); a piece that crosses c_end is read element by
// element.
template <typename T, int ROWS, int COLS>
__device__ __forceinline__ void load_tile(const T* __restrict__ W, int64_t ldw, int64_t r0,
                                          int64_t r_end, int64_t c0, int64_t c_end,
                                          TileBuf<T, ROWS, COLS>& b) {
  constexpr int V = TileBuf<T, ROWS, COLS>::V;
#pragma unroll
  for (int p = 0; p < TileBuf<T, ROWS, COLS>::PER; ++p) {
    const int idx = threadIdx.x + 256 * p;
    const int rr = idx / (COLS / V), cv = idx % (COLS / V);
    const int64_t c = c0 + cv * V;
    b.v[p] = u32x4_t{0u, 0u, 0u, 0u};
    if (r0 + rr < r_end) {
      const T* src = W + (r0 + rr) * ldw + c;
      if (c + V <= c_end) {
        b.v[p] = *reinterpret_cast<const u32x4_t*>(src);
      } else if (c < c_end) {
        T part[V];
#pragma unroll
        for (int e = 0; e < V; ++e) part[e] = c + e < c_end ? src[e] : (T)0;
        __builtin_memcpy(&b.v[p], part, 16);
      }
    }
  }
}

// ... and store it into LDS as fp32 (row pitch LDS_LD floats)
template <typename T, int ROWS, int COLS, int LDS_LD>
__device__ __forceinline__ void store_tile(const TileBuf<T, ROWS, COLS>& b, float* lds) {
  constexpr int V = TileBuf<T, ROWS, COLS>::V;
#pragma unroll
  for (int p = 0; p < TileBuf<T, ROWS, COLS>::PER; ++p) {
    const int idx = threadIdx.x + 256 * p;
    const int rr = idx / (COLS / V), cv = idx % (COLS / V);
    float* dst = lds + rr * LDS_LD + cv * V;
    if (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[2 * e] = bf16_lo(b.v[p][e]);
        dst[2 * e + 1] = bf16_hi(b.v[p][e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = __uint_as_float(b.v[p][e]);
    }
  }
}

template <typename T, int ROWS, int COLS, int LDS_LD>
__device__ __forceinline__ void stage_tile(const T* __restrict__ W, int64_t ldw, int64_t r0,
                                           int64_t r_end, int64_t c0, int64_t c_end,
                                           float* lds) {
  TileBuf<T, ROWS, COLS> b;
  load_tile<T, ROWS, COLS>(W, ldw, r0, r_end, c0, c_end, b);
  store_tile<T, ROWS, COLS, LDS_LD>(b, lds);
}

// Yp[s][k][j] = Σ_{n in split s} W[n, k] · X[n, j]: 256 columns k per workgroup (thread =
// column), 40 columns of X per workgroup (blockIdx.z); W and X staged 64 rows at a time.  (Loading
// the next chunk into registers while multiplying the current one timed slower.)
template <typename T>
__global__ __launch_bounds__(256) void k_sketch_wt(const T* __restrict__ W, int64_t N,
                                                   int64_t K, int64_t ldw,
                                                   const float* __restrict__ X, int ell,
                                                   float* __restrict__ Yp) {
  constexpr int kR = 64;
  // the W chunk [kR][256] while accumulating, then the block of sums [256][kColTile]
  __shared__ __attribute__((aligned(16))) float s_buf[kR * 256];
  static_assert(kR * 256 >= 256 * kColTile, "the sums fit the chunk buffer");
  float (*ws)[256] = reinterpret_cast<float (*)[256]>(s_buf);
  __shared__ float xs[kR][kColTile];
  const int64_t kb = (int64_t)blockIdx.x * 256;
  const int64_t s = blockIdx.y;
  const int j0 = blockIdx.z * kColTile;
  const int jn = ell - j0 < kColTile ? ell - j0 : kColTile;
  const int64_t n_begin = s * kSplitWt;
  const int64_t n_end = n_begin + kSplitWt < N ? n_begin + kSplitWt : N;
  float acc[kColTile];
#pragma unroll
  for (int c = 0; c < kColTile; ++c) acc[c] = 0.0f;
  for (int64_t n0 = n_begin; n0 < n_end; n0 += kR) {
    __syncthreads();
    stage_tile<T, kR, 256, 256>(W, ldw, n0, n_end, kb, K, &ws[0][0]);
    for (int t = threadIdx.x; t < kR * kColTile; t += 256) {
      const int rr = t / kColTile, c = t % kColTile;
      xs[rr][c] = (n0 + rr < n_end && c < jn) ? X[(n0 + rr) * ell + j0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < kR; ++rr) {
      const float w = ws[rr][threadIdx.x];
#pragma unroll
      for (int c = 0; c < kColTile; ++c) acc[c] = __builtin_fmaf(w, xs[rr][c], acc[c]);
    }
  }
  // The sums leave through LDS so that the stores are row-contiguous (a thread's 40 sums are
  // one row of the output; storing them directly would touch a cache line per lane).
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kColTile; ++c) s_buf[threadIdx.x * kColTile + ((c + threadIdx.x) % kColTile)] = acc[c];
  __syncthreads();
  auto sum_at = [&](int row, int c) { return s_buf[row * kColTile + ((c + row) % kColTile)]; };
  if (ell == kColTile && kb + 256 <= K) {
    // the block is one contiguous run of 256 x 40 floats
    float* dst = Yp + (s * K + kb) * ell;
    for (int t = threadIdx.x; t < 256 * kColTile / 4; t += 256) {
      const int e = 4 * t, row = e / kColTile, c = e % kColTile;
      *reinterpret_cast<f32x4_t*>(dst + e) =
          f32x4_t{sum_at(row, c), sum_at(row, c + 1), sum_at(row, c + 2), sum_at(row, c + 3)};
    }
  } else {
    for (int t = threadIdx.x; t < 256 * kColTile; t += 256) {
      const int row = t / kColTile, c = t % kColTile;
      const int64_t k = kb + row;
      if (k < K && c < jn) Yp[(s * K + k) * ell + j0 + c] = sum_at(row, c);
    }
  }
}

// Zp[s][n][j] = Σ_{k in split s} W[n, k] · λ_k · Q[k, j]: 128 rows n x 40 columns per
// workgroup; thread = 4 rows (tid / 8) x 5 columns (tid % 8 + 8m), W and λ∘Q staged 64 channels
// at a time.
template <typename T>
__global__ __launch_bounds__(256) void k_sketch_w(const T* __restrict__ W, int64_t N,
                                                  int64_t K, int64_t ldw,
                                                  const float* __restrict__ lambda,
                                                  const float* __restrict__ Q, int ell,
                                                  float* __restrict__ Zp) {
  constexpr int kRows = 128, kPr = 4, kPc = kColTile / 8;
  __shared__ float ws[kRows][65];
  __shared__ float qs[64][kColTile];
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t s = blockIdx.y;
  const int j0 = blockIdx.z * kColTile;
  const int jn = ell - j0 < kColTile ? ell - j0 : kColTile;
  const int64_t k_begin = s * kSplitW;
  const int64_t k_end = k_begin + kSplitW < K ? k_begin + kSplitW : K;
  const int rg = threadIdx.x >> 3, cg = threadIdx.x & 7;
  float acc[kPr][kPc];
#pragma unroll
  for (int a = 0; a < kPr; ++a)
#pragma unroll
    for (int m = 0; m < kPc; ++m) acc[a][m] = 0.0f;
  for (int64_t k0 = k_begin; k0 < k_end; k0 += 64) {
    const int kn = k_end - k0 < 64 ? (int)(k_end - k0) : 64;
    __syncthreads();
    stage_tile<T, kRows, 64, 65>(W, ldw, n0, N, k0, k_end, &ws[0][0]);
    for (int t = threadIdx.x; t < 64 * kColTile; t += 256) {
      const int kk = t / kColTile, c = t % kColTile;
      float v = 0.0f;
      if (kk < kn && c < jn) {
        v = Q[(k0 + kk) * ell + j0 + c];
        if (lambda) v *= lambda[k0 + kk];
      }
      qs[kk][c] = v;
    }
    __syncthreads();
    for (int kk = 0; kk < kn; ++kk) {
      float w[kPr], q[kPc];
#pragma unroll
      for (int a = 0; a < kPr; ++a) w[a] = ws[rg * kPr + a][kk];
#pragma unroll
      for (int m = 0; m < kPc; ++m) q[m] = qs[kk][cg + 8 * m];
#pragma unroll
      for (int a = 0; a < kPr; ++a)
#pragma unroll
        for (int m = 0; m < kPc; ++m) acc[a][m] = __builtin_fmaf(w[a], q[m], acc[a][m]);
    }
  }
#pragma unroll
  for (int a = 0; a < kPr; ++a) {
    const int64_t n = n0 + rg * kPr + a;
    if (n < N) {
#pragma unroll
      for (int m = 0; m < kPc; ++m) {
        const int c = cg + 8 * m;
        if (c < jn) Zp[(s * N + n) * ell + j0 + c] = acc[a][m];
      }
    }
  }
}

// out[i] = scale(row) · Σ_s P[s][i] (splits in ascending order), i over rows x ell
__global__ __launch_bounds__(256) void k_reduce_splits(const float* __restrict__ P, int64_t rows,
                                                       int ell, int64_t nsplit,
                                                       const float* __restrict__ row_scale,
                                                       float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = rows * ell;
  if (i >= total) return;
  float acc = 0.0f;
  for (int64_t s = 0; s < nsplit; ++s) acc += P[s * total + i];
  if (row_scale) acc *= row_scale[i / ell];
  out[i] = acc;
}

// Gp[b][i][j] = Σ over rows of chunk b (64 rows) of M[row][i]·M[row][j] in fp64 (both triangles)
__global__ __launch_bounds__(256) void k_gram_partial(const float* __restrict__ M, int64_t rows,
                                                      int ell, double* __restrict__ Gp) {
  __shared__ float ms[kGramRows][kMaxEll];
  const int64_t r0 = (int64_t)blockIdx.x * kGramRows;
  const int rn = rows - r0 < kGramRows ? (int)(rows - r0) : kGramRows;
  for (int t = threadIdx.x; t < kGramRows * ell; t += 256) {
    const int rr = t / ell, c = t % ell;
    ms[rr][c] = rr < rn ? M[(r0 + rr) * ell + c] : 0.0f;
  }
  __syncthreads();
  double* g = Gp + (int64_t)blockIdx.x * ell * ell;
  const int npairs = ell * (ell + 1) / 2;
  for (int p = threadIdx.x; p < npairs; p += 256) {
    // pair p -> (i, j), i <= j, row-major over the upper triangle
    int i = 0, rem = p;
    while (rem >= ell - i) {
      rem -= ell - i;
      ++i;
    }
    const int j = i + rem;
    double acc = 0.0;
    for (int rr = 0; rr < rn; ++rr) acc += (double)ms[rr][i] * (double)ms[rr][j];
    g[i * ell + j] = acc;
    g[j * ell + i] = acc;
  }
}

// G = Σ_b Gp[b] (ascending b)
__global__ __launch_bounds__(256) void k_gram_reduce(const double* __restrict__ Gp, int64_t nb,
                                                     int ell, double* __restrict__ G) {
  // one wave per element: lane l sums the partials l, l + 64, ... in order, then the wave adds
  // its lanes in a fixed tree (deterministic)
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (i >= ell * ell) return;
  double acc = 0.0;
  for (int64_t b = lane; b < nb; b += 64) acc += Gp[b * ell * ell + i];
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) G[i] = acc;
}

// Cholesky G = RᵀR (R upper) and Rinv = R⁻¹ (upper), fp64, one workgroup.  A pivot that is not
// positive (a rank-deficient block) is raised to a tiny positive value relative to the trace,
// which keeps every value finite; such directions have singular values at rounding level and
// end up at the bottom of the spectrum.  Both factorisations are right-looking: every step is a
// pivot, a scaled row and a rank-1 update of the trailing part, each spread over the workgroup,
// so a step costs a few barriers instead of a serial dot product.
__global__ __launch_bounds__(kCholThreads) void k_chol_inv(const double* __restrict__ G, int ell,
                                                  double* __restrict__ Rg,
                                                  double* __restrict__ Rinvg) {
  __shared__ double s_tiny;
  __shared__ double s_r[kLdsEll * kLdsEll], s_ri[kLdsEll * kLdsEll];
  // R and R⁻¹ are built in LDS when they fit, in the output buffers otherwise (same arithmetic)
  const bool in_lds = ell <= kLdsEll;
  double* R = in_lds ? s_r : Rg;
  double* X = in_lds ? s_ri : Rinvg;
  const int tid = threadIdx.x;
  if (tid == 0) {
    double tr = 0.0;
    for (int i = 0; i < ell; ++i) tr += G[i * ell + i];
    s_tiny = (tr > 1e-300 ? tr : 1e-300) * 1e-28;
  }
  // R starts as the upper triangle of G, X as the identity
  for (int t = tid; t < ell * ell; t += kCholThreads) {
    const int i = t / ell, j = t % ell;
    R[t] = j >= i ? G[t] : 0.0;
    X[t] = i == j ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int j = 0; j < ell; ++j) {
    if (tid == 0) {
      const double d = R[j * ell + j];
      R[j * ell + j] = sqrt(d > s_tiny ? d : s_tiny);
    }
    __syncthreads();
    const double rjj = R[j * ell + j];
    for (int i = j + 1 + tid; i < ell; i += kCholThreads) R[j * ell + i] /= rjj;
    __syncthreads();
    const int n = ell - 1 - j;   // trailing upper triangle: rows/columns j+1 .. ell-1
    for (int t = tid; t < n * n; t += kCholThreads) {
      const int k = j + 1 + t / n, i = j + 1 + t % n;
      if (i >= k) R[k * ell + i] -= R[j * ell + k] * R[j * ell + i];
    }
    __syncthreads();
  }
  // X = R⁻¹ from the bottom row up: row k of X is divided by R_kk, then removed from the rows
  // above it in proportion to column k of R
  for (int k = ell - 1; k >= 0; --k) {
    const double rkk = R[k * ell + k];
    for (int c = k + tid; c < ell; c += kCholThreads) X[k * ell + c] /= rkk;
    __syncthreads();
    for (int t = tid; t < k * (ell - k); t += kCholThreads) {
      const int i = t / (ell - k), c = k + t % (ell - k);
      X[i * ell + c] -= R[i * ell + k] * X[k * ell + c];
    }
    __syncthreads();
  }
  if (in_lds) {
    for (int t = tid; t < ell * ell; t += kCholThreads) {
      Rg[t] = s_r[t];
      Rinvg[t] = s_ri[t];
    }
  }
}

// Mo[row][j] = Σ_{i <= j} M[row][i] · Rinv[i][j]  (fp64 accumulation)
__global__ __launch_bounds__(256) void k_apply_rinv(const float* __restrict__ M, int64_t rows,
                                                    int ell, const double* __restrict__ Rinv,
                                                    float* __restrict__ Mo) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * ell) return;
  const int64_t row = t / ell;
  const int j = (int)(t % ell);
  double acc = 0.0;
  for (int i = 0; i <= j; ++i) acc += (double)M[row * ell + i] * Rinv[i * ell + j];
  Mo[t] = (float)acc;
}

// Parallel cyclic Jacobi on the symmetric H (ell x ell, fp64), eigenvectors accumulated as the
// rows of Vt (Vt = Vᵀ); then the eigenpairs sorted by decreasing eigenvalue: eig[i], U[:, i].
// Rounds pair the indices by the circle method (index 0 fixed, the others rotating); an odd ell
// gets a dummy index that sits out its pairs.  A round applies its rotations in place: rows p
// and q of H and of Vt, a barrier, then columns p and q of H.  H lives in LDS up to kJacHLdsEll
// with an odd row pitch (the column pass then reads and writes across the banks instead of
// one bank in sixteen), Vt too up to kJacVLdsEll; larger ones stay in the caller's buffers
// (same arithmetic).
__global__ __launch_bounds__(kJacobiThreads) void k_jacobi(double* __restrict__ Hg, int ell,
                                                           double* __restrict__ Vg,
                                                           double* __restrict__ U,
                                                           double* __restrict__ eig) {
  extern __shared__ double s_dyn[];  // H (ell x jacobi_pitch, when in LDS), then Vt (ell²)
  __shared__ double s_c[kMaxEll / 2], s_s[kMaxEll / 2];
  __shared__ int s_p[kMaxEll / 2], s_q[kMaxEll / 2];
  __shared__ double s_red[2][kJacobiThreads / 64];
  __shared__ int s_order[kMaxEll];
  __shared__ int s_done;
  __shared__ double s_prev;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_prev = 0.0;
  const bool h_lds = ell <= kJacHLdsEll, v_lds = ell <= kJacVLdsEll;
  const int ldh = h_lds ? jacobi_pitch(ell) : ell;
  double* H = h_lds ? s_dyn : Hg;
  double* Vt = v_lds ? s_dyn + (h_lds ? ell * ldh : 0) : Vg;
  if (h_lds)
    for (int t = tid; t < ell * ell; t += kJacobiThreads) H[(t / ell) * ldh + t % ell] = Hg[t];
  const int m = (ell + 1) & ~1;  // even player count
  const int half = m / 2;
  for (int t = tid; t < ell * ell; t += kJacobiThreads) Vt[t] = (t / ell == t % ell) ? 1.0 : 0.0;
  // One rotation pass of a round over A (row pitch ld): rows p, q (by_row) or columns p, q of
  // every pair of the round, for every position along them.  Item t of the pass is (pair
  // t / ell, position t % ell); a thread's items are fixed for the whole solve, so their
  // coordinates are computed once.
  int item_pr[kJacItems], item_x[kJacItems];
#pragma unroll
  for (int k = 0; k < kJacItems; ++k) {
    const int t = tid + k * kJacobiThreads;
    item_pr[k] = t < half * ell ? t / ell : -1;
    item_x[k] = t < half * ell ? t % ell : 0;
  }
  auto rotate = [&](double* A, int ld, bool by_row) {
#pragma unroll
    for (int k = 0; k < kJacItems; ++k) {
      const int pr = item_pr[k];
      if (pr < 0) break;
      const int p = s_p[pr], q = s_q[pr];
      if (q < 0) continue;
      const int x = item_x[k];
      const int ip = by_row ? p * ld + x : x * ld + p;
      const int iq = by_row ? q * ld + x : x * ld + q;
      const double ap = A[ip], aq = A[iq];
      const double c = s_c[pr], sn = s_s[pr];
      A[ip] = c * ap - sn * aq;
      A[iq] = sn * ap + c * aq;
    }
  };
  __syncthreads();
  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    // convergence: off-diagonal mass against the whole matrix
    double off = 0.0, all = 0.0;
    for (int t = tid; t < ell * ell; t += kJacobiThreads) {
      const int a = t / ell, b = t % ell;
      const double h = H[a * ldh + b];
      all += h * h;
      if (a != b) off += h * h;
    }
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o);
      all += __shfl_xor(all, o);
    }
    if (lane == 0) {
      s_red[0][wave] = off;
      s_red[1][wave] = all;
    }
    __syncthreads();
    if (tid == 0) {
      double so = 0.0, sa = 0.0;
      for (int w = 0; w < kJacobiThreads / 64; ++w) {
        so += s_red[0][w];
        sa += s_red[1][w];
      }
      // done at 1e-15 of the norm, or once the off-diagonal mass, already below 1e-10 of the
      // norm (the quadratic phase), no longer falls 4x per sweep: it has reached the rounding
      // floor of the rotations, which for larger ell lies above 1e-15
      s_done = (so <= 1e-30 * sa || (so <= 1e-20 * sa && so >= 0.25 * s_prev)) ? 1 : 0;
      s_prev = so;
    }
    __syncthreads();
    if (s_done) break;
    for (int round = 0; round < m - 1; ++round) {
      if (tid < half) {
        int a, b;
        if (tid == 0) {
          a = 0;
          b = 1 + round % (m - 1);
        } else {
          a = 1 + (round + tid) % (m - 1);
          b = 1 + (round - tid + (m - 1)) % (m - 1);
        }
        const int p = a < b ? a : b, q = a < b ? b : a;
        double c = 1.0, sn = 0.0;
        if (q < ell) {
          const double hpq = H[p * ldh + q];
          if (hpq != 0.0) {
            const double tau = (H[q * ldh + q] - H[p * ldh + p]) / (2.0 * hpq);
            const double tt = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
            c = 1.0 / sqrt(1.0 + tt * tt);
            sn = tt * c;
          }
        }
        s_p[tid] = p;
        s_q[tid] = q < ell ? q : -1;
        s_c[tid] = c;
        s_s[tid] = sn;
      }
      __syncthreads();
      // rows p, q of H and of Vt: p <- c·p − s·q, q <- s·p + c·q
      rotate(H, ldh, true);
      rotate(Vt, ell, true);
      __syncthreads();
      // columns p, q of H
      rotate(H, ldh, false);
      __syncthreads();
    }
  }
  // sort by decreasing eigenvalue (ties by index)
  if (tid == 0) {
    for (int i = 0; i < ell; ++i) s_order[i] = i;
    for (int i = 0; i < ell; ++i) {
      int best = i;
      for (int j = i + 1; j < ell; ++j)
        if (H[s_order[j] * ldh + s_order[j]] > H[s_order[best] * ldh + s_order[best]]) best = j;
      const int tmp = s_order[i];
      s_order[i] = s_order[best];
      s_order[best] = tmp;
    }
  }
  __syncthreads();
  for (int t = tid; t < ell * ell; t += kJacobiThreads) {
    const int i = t / ell, c = t % ell;
    U[i * ell + c] = Vt[s_order[c] * ell + i];
  }
  for (int c = tid; c < ell; c += kJacobiThreads) eig[c] = H[s_order[c] * ldh + s_order[c]];
}

size_t jacobi_lds_bytes(int ell) {
  size_t n = 0;
  if (ell <= kJacHLdsEll) n += (size_t)ell * jacobi_pitch(ell) * 8;
  if (ell <= kJacVLdsEll) n += (size_t)ell * ell * 8;
  return n;
}

// lora_down[i][k] = bf16(σ_i Σ_j Q[k][j] U[j][i]);  lora_up[n][i] = bf16(Σ_j Z[n][j] U[j][i] / σ_i)
// (0 when σ_i == 0);  sigma[i] = σ_i = sqrt(max(eig_i, 0)).
__global__ __launch_bounds__(256) void k_factors(const float* __restrict__ Q,
                                                 const float* __restrict__ Z, int64_t N,
                                                 int64_t K, int ell, int r,
                                                 const double* __restrict__ U,
                                                 const double* __restrict__ eig,
                                                 uint16_t* __restrict__ down,
                                                 uint16_t* __restrict__ up,
                                                 float* __restrict__ sigma) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nd = (int64_t)r * K, nu = N * (int64_t)r;
  if (t < nd) {
    const int i = (int)(t / K);
    const int64_t k = t % K;
    const double sg = sqrt(eig[i] > 0.0 ? eig[i] : 0.0);
    double acc = 0.0;
    for (int j = 0; j < ell; ++j) acc += (double)Q[k * ell + j] * U[j * ell + i];
    down[(int64_t)i * K + k] = f32_to_bf16((float)(acc * sg));
    if (sigma && k == 0) sigma[i] = (float)sg;
  } else if (t < nd + nu) {
    const int64_t u = t - nd;
    const int64_t n = u / r;
    const int i = (int)(u % r);
    const double sg = sqrt(eig[i] > 0.0 ? eig[i] : 0.0);
    double acc = 0.0;
    for (int j = 0; j < ell; ++j) acc += (double)Z[n * ell + j] * U[j * ell + i];
    up[n * r + i] = f32_to_bf16(sg > 0.0 ? (float)(acc / sg) : 0.0f);
  }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

struct Workspace {
  float *y, *yt, *z, *zt, *p;
  double *gp, *g, *r, *rinv, *v, *u, *eig;
};

Workspace carve(void* base, int64_t N, int64_t K, int64_t ell) {
  uint8_t* b = static_cast<uint8_t*>(base);
  Workspace w;
  auto take = [&](int64_t bytes) {
    uint8_t* p = b;
    b += align256(bytes);
    return p;
  };
  w.y = reinterpret_cast<float*>(take(K * ell * 4));
  w.yt = reinterpret_cast<float*>(take(K * ell * 4));
  w.z = reinterpret_cast<float*>(take(N * ell * 4));
  w.zt = reinterpret_cast<float*>(take(N * ell * 4));
  const int64_t splits = ceil_div(N, kSplitWt) * K > ceil_div(K, kSplitW) * N
                             ? ceil_div(N, kSplitWt) * K
                             : ceil_div(K, kSplitW) * N;
  w.p = reinterpret_cast<float*>(take(splits * ell * 4));
  const int64_t nb = ceil_div(K > N ? K : N, kGramRows);
  w.gp = reinterpret_cast<double*>(take(nb * ell * ell * 8));
  w.g = reinterpret_cast<double*>(take(ell * ell * 8));
  w.r = reinterpret_cast<double*>(take(ell * ell * 8));
  w.rinv = reinterpret_cast<double*>(take(ell * ell * 8));
  w.v = reinterpret_cast<double*>(take(ell * ell * 8));
  w.u = reinterpret_cast<double*>(take(ell * ell * 8));
  w.eig = reinterpret_cast<double*>(take(ell * 8));
  return w;
}

}  // namespace

int64_t lowrank_workspace_bytes(int64_t N, int64_t K, int64_t ell) {
  int64_t total = 0;
  total += 2 * align256(K * ell * 4) + 2 * align256(N * ell * 4);
  const int64_t splits = ceil_div(N, kSplitWt) * K > ceil_div(K, kSplitW) * N
                             ? ceil_div(N, kSplitWt) * K
                             : ceil_div(K, kSplitW) * N;
  total += align256(splits * ell * 4);
  total += align256(ceil_div(K > N ? K : N, kGramRows) * ell * ell * 8);
  total += 5 * align256(ell * ell * 8) + align256(ell * 8);
  return total;
}

int lowrank_max_ell() { return kMaxEll; }

namespace {

template <typename T>
hipError_t lowrank_impl(const T* W, int64_t N, int64_t K, int64_t ldw, const float* lambda,
                        const float* omega, int64_t ell, int64_t r, int power_iters,
                        uint16_t* lora_down, uint16_t* lora_up, float* sigma, void* workspace,
                        hipStream_t s) {
  Workspace w = carve(workspace, N, K, ell);
  const int e = (int)ell;
  const unsigned ztiles = (unsigned)ceil_div(ell, kColTile);
  hipError_t err;
#define SVDQ_CHECK_LAUNCH() \
  do {                      \
    err = hipGetLastError(); \
    if (err != hipSuccess) return err; \
  } while (0)

  // Y (K x ell) = diag(λ) Wᵀ X  for X (N x ell)
  auto a_times = [&](const float* X, float* Y) -> hipError_t {
    const int64_t nsplit = ceil_div(N, kSplitWt);
    k_sketch_wt<<<dim3((unsigned)ceil_div(K, 256), (unsigned)nsplit, ztiles), dim3(256), 0, s>>>(
        W, N, K, ldw, X, e, w.p);
    SVDQ_CHECK_LAUNCH();
    k_reduce_splits<<<dim3((unsigned)ceil_div(K * ell, 256)), dim3(256), 0, s>>>(
        w.p, K, e, nsplit, lambda, Y);
    SVDQ_CHECK_LAUNCH();
    return hipSuccess;
  };
  // Z (N x ell) = W diag(λ) Q  for Q (K x ell)
  auto at_times = [&](const float* Qm, float* Z) -> hipError_t {
    const int64_t nsplit = ceil_div(K, kSplitW);
    k_sketch_w<<<dim3((unsigned)ceil_div(N, 128), (unsigned)nsplit, ztiles), dim3(256), 0, s>>>(
        W, N, K, ldw, lambda, Qm, e, w.p);
    SVDQ_CHECK_LAUNCH();
    k_reduce_splits<<<dim3((unsigned)ceil_div(N * ell, 256)), dim3(256), 0, s>>>(
        w.p, N, e, nsplit, nullptr, Z);
    SVDQ_CHECK_LAUNCH();
    return hipSuccess;
  };
  auto gram = [&](const float* M, int64_t rows, double* G) -> hipError_t {
    const int64_t nb = ceil_div(rows, kGramRows);
    k_gram_partial<<<dim3((unsigned)nb), dim3(256), 0, s>>>(M, rows, e, w.gp);
    SVDQ_CHECK_LAUNCH();
    k_gram_reduce<<<dim3((unsigned)ceil_div(ell * ell, 4)), dim3(256), 0, s>>>(w.gp, nb, e, G);
    SVDQ_CHECK_LAUNCH();
    return hipSuccess;
  };
  // M (rows x ell) <- an orthonormal basis of its columns (Cholesky-QR twice); tmp is scratch
  auto orth = [&](float*& M, float*& tmp, int64_t rows) -> hipError_t {
    for (int pass = 0; pass < 2; ++pass) {
      if ((err = gram(M, rows, w.g)) != hipSuccess) return err;
      k_chol_inv<<<dim3(1), dim3(kCholThreads), 0, s>>>(w.g, e, w.r, w.rinv);
      SVDQ_CHECK_LAUNCH();
      k_apply_rinv<<<dim3((unsigned)ceil_div(rows * ell, 256)), dim3(256), 0, s>>>(M, rows, e,
                                                                                  w.rinv, tmp);
      SVDQ_CHECK_LAUNCH();
      float* t = M;
      M = tmp;
      tmp = t;
    }
    return hipSuccess;
  };

  float *y = w.y, *yt = w.yt, *z = w.z, *zt = w.zt;
  if ((err = a_times(omega, y)) != hipSuccess) return err;
  if ((err = orth(y, yt, K)) != hipSuccess) return err;
  for (int it = 0; it < power_iters; ++it) {
    if ((err = at_times(y, z)) != hipSuccess) return err;
    if ((err = orth(z, zt, N)) != hipSuccess) return err;
    if ((err = a_times(z, y)) != hipSuccess) return err;
    if ((err = orth(y, yt, K)) != hipSuccess) return err;
  }
  if ((err = at_times(y, z)) != hipSuccess) return err;       // Z = Aᵀ Q = Bᵀ
  if ((err = gram(z, N, w.g)) != hipSuccess) return err;      // B Bᵀ
  {
    const size_t lds = jacobi_lds_bytes(e);
    if ((err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_jacobi),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) !=
        hipSuccess)
      return err;
    k_jacobi<<<dim3(1), dim3(kJacobiThreads), lds, s>>>(w.g, e, w.v, w.u, w.eig);
  }
  SVDQ_CHECK_LAUNCH();
  const int64_t nout = (r * K) + (N * r);
  k_factors<<<dim3((unsigned)ceil_div(nout, 256)), dim3(256), 0, s>>>(
      y, z, N, K, e, (int)r, w.u, w.eig, lora_down, lora_up, sigma);
  SVDQ_CHECK_LAUNCH();
#undef SVDQ_CHECK_LAUNCH
  return hipSuccess;
}

}  // namespace

hipError_t launch_lowrank(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                          const float* lambda, const float* omega, int64_t ell, int64_t r,
                          int power_iters, uint16_t* lora_down, uint16_t* lora_up, float* sigma,
                          void* workspace, hipStream_t s) {
  return lowrank_impl(W, N, K, ldw, lambda, omega, ell, r, power_iters, lora_down, lora_up, sigma,
                      workspace, s);
}

hipError_t launch_lowrank_f32(const float* E, int64_t N, int64_t K, int64_t lde,
                              const float* omega, int64_t ell, int64_t r, int power_iters,
                              uint16_t* lora_down, uint16_t* lora_up, float* sigma,
                              void* workspace, hipStream_t s) {
  return lowrank_impl(E, N, K, lde, nullptr, omega, ell, r, power_iters, lora_down, lora_up,
                      sigma, workspace, s);
}

}  // namespace svdq
