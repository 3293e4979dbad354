"""Low-rank branch and weight residual.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph.  The layer
keeps a rank-32 branch in 16-bit precision beside a 4-bit residual weight.  Here the branch is
the rank-r truncated SVD of the smoothed weight W' = diag(λ)·W, the weight that meets the
smoothed activation X̂ = X/λ, so X·W = X̂·W' = X̂·L1·L2 + X̂·R.

Storage here is [out, in] = [N, K]: W'[n, k] = λ_k · W[n, k].  With W'ᵀ (K x N) = U Σ Vᵀ:
    L1 = U_r Σ_r  (K x r),   L2 = V_rᵀ  (r x N)
    lora_down = bf16(L1ᵀ)  [r, K],   lora_up = bf16(L2ᵀ)  [N, r]
Readings: the split puts Σ on L1 and both factors are stored in bf16 (round to nearest even).
The residual uses the ROUNDED factors:
    R = W' − Σ_i lora_up[:, i] ⊗ lora_down[i, :]    (float64, i ascending; each product exact)
    R32 = float32(R)
SVD factors are not unique (signs, rotations of equal singular values), so both the oracle and
the GPU path take lora_down / lora_up as inputs.

Randomized factors (computing the branch on the GPU; the pages give no method for it, so the
reading is the randomized range finder with power iterations and a small SVD, Halko, Martinsson
and Tropp 2011, Algorithms 4.4 and 5.1):
    A = W'ᵀ (K x N),  Ω (N x ℓ, ℓ = r + oversampling) a given random matrix
    Q = orth(A Ω);  q times: Q = orth(A · orth(Aᵀ Q))
    B = Qᵀ A = U_B Σ V_Bᵀ,   L1 = Q U_B[:, :r] Σ_r,   L2 = V_B[:, :r]ᵀ
Ω is an input (both sides draw nothing).  The span of each Q, hence L1·L2 and Σ, does not
depend on how a basis is orthonormalised; the factors themselves are compared only through
these unique quantities.
"""
import numpy as np

from .formats import bf16_bits_to_f32, bf16_rne

F32 = np.float32


def smoothed_weight(W_bits, lam):
    """W'[n, k] = λ_k · W[n, k] in float64 (exact: 24-bit × 8-bit significands)."""
    W = bf16_bits_to_f32(W_bits).astype(np.float64)
    if lam is None:
        return W
    return W * np.asarray(lam, dtype=F32).astype(np.float64)[None, :]


def truncated_svd(A, r):
    """Rank-r truncated SVD of a float64 matrix A: (U_r, σ_r, V_rᵀ), σ descending.

    A library SVD is the step: LAPACK's full SVD for moderate sizes, ARPACK's partial SVD
    (scipy.sparse.linalg.svds) when both dimensions exceed 2048.
    """
    A = np.asarray(A, dtype=np.float64)
    if r == 0:
        return (np.zeros((A.shape[0], 0)), np.zeros(0), np.zeros((0, A.shape[1])))
    if min(A.shape) > 2048:
        from scipy.sparse.linalg import svds
        U, s, Vt = svds(A, k=r, tol=0, random_state=0)
        order = np.argsort(s)[::-1]
        return U[:, order], s[order], Vt[order, :]
    U, s, Vt = np.linalg.svd(A, full_matrices=False)
    return U[:, :r], s[:r], Vt[:r, :]


def lowrank_factors(W_bits, lam, r):
    """bf16 factors (lora_down [r, K], lora_up [N, r]) of the rank-r SVD of W'ᵀ = diag(λ)Wᵀ."""
    Wp = smoothed_weight(W_bits, lam)              # [N, K]
    U, s, Vt = truncated_svd(Wp.T, r)              # W'ᵀ is K x N
    L1 = U * s[None, :]                            # K x r
    L2 = Vt                                        # r x N
    return bf16_rne(L1.T), bf16_rne(L2.T)


def _orth(M):
    """An orthonormal basis of the columns of M (a library QR is the step)."""
    return np.linalg.qr(M)[0]


def randomized_factors(W_bits, lam, r, omega, power_iters):
    """Randomized rank-r factors: (lora_down bf16 bits [r, K], lora_up bf16 bits [N, r],
    σ float64 [r], the unrounded L1 [K, r] and L2 [r, N] in float64)."""
    return randomized_factors_of(smoothed_weight(W_bits, lam).T, r, omega, power_iters)


def randomized_factors_of(A, r, omega, power_iters):
    """The same factors for any K x N matrix A (float64)."""
    A = np.asarray(A, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)        # N x ℓ
    Q = _orth(A @ omega)
    for _ in range(power_iters):
        Q = _orth(A @ _orth(A.T @ Q))
    B = Q.T @ A                                        # ℓ x N
    Ub, s, Vt = np.linalg.svd(B, full_matrices=False)
    L1 = (Q @ Ub[:, :r]) * s[None, :r]
    L2 = Vt[:r]
    return bf16_rne(L1.T), bf16_rne(L2.T), s[:r], L1, L2


def residual_f32(W_bits, lam, lora_down_bits, lora_up_bits):
    """R32 = float32(W' − Σ_i up[:, i] ⊗ down[i, :]) with the subtraction in float64, i ascending."""
    R = smoothed_weight(W_bits, lam)
    down = bf16_bits_to_f32(lora_down_bits).astype(np.float64)   # [r, K]
    up = bf16_bits_to_f32(lora_up_bits).astype(np.float64)       # [N, r]
    r = down.shape[0]
    for i in range(r):
        R -= up[:, i:i + 1] * down[i:i + 1, :]
    return R.astype(F32)
