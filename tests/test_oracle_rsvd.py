"""Pins of the oracle's randomized low-rank factors (reading: randomized range finder with power
iterations, Halko, Martinsson and Tropp 2011) against facts independent of it: an exactly
low-rank matrix is recovered exactly; the singular values never exceed the exact ones and
approach them with power iterations; the approximation error is close to the optimal (exact
truncated SVD) on a decaying spectrum; the right factor is orthonormal."""
import numpy as np
import pytest

from oracle import svd as OS
from oracle.formats import bf16_rne, bf16_bits_to_f32


def _weight_bits(N, K, s, seed):
    rng = np.random.default_rng(seed)
    U = np.linalg.qr(rng.standard_normal((N, len(s))))[0]
    V = np.linalg.qr(rng.standard_normal((K, len(s))))[0]
    return bf16_rne(U @ np.diag(s) @ V.T)


def _A(W_bits, lam):
    return OS.smoothed_weight(W_bits, lam).T


def test_exactly_low_rank_matrix_is_recovered():
    # small-integer factors: every entry of their product is an integer of magnitude <= 24,
    # exact in bf16, so W has rank 6 exactly
    rng = np.random.default_rng(0)
    N, K, r, ell = 96, 128, 6, 12
    Wb = bf16_rne((rng.integers(-2, 3, (N, r)) @ rng.integers(-2, 3, (r, K))).astype(np.float64))
    lam = np.ones(K, np.float32)
    A = _A(Wb, lam)
    rank = np.linalg.matrix_rank(A)
    omega = rng.standard_normal((N, ell))
    _, _, s, L1, L2 = OS.randomized_factors(Wb, lam, rank, omega, 0)
    assert np.allclose(L1 @ L2, A, rtol=0, atol=1e-10 * np.abs(A).max())
    assert np.allclose(s, np.linalg.svd(A, compute_uv=False)[:rank], rtol=1e-10)


def test_singular_values_are_lower_bounds_that_tighten_with_power_iterations():
    rng = np.random.default_rng(1)
    N, K, r, ell = 200, 160, 10, 16
    s_true = 0.9 ** np.arange(min(N, K))
    Wb = _weight_bits(N, K, s_true, 1)
    lam = np.exp(rng.normal(0, 0.3, K)).astype(np.float32)
    exact = np.linalg.svd(_A(Wb, lam), compute_uv=False)[:r]
    omega = rng.standard_normal((N, ell))
    errs = []
    for q in (0, 1, 2):
        s = OS.randomized_factors(Wb, lam, r, omega, q)[2]
        assert np.all(s <= exact * (1 + 1e-12))          # Rayleigh-Ritz values: lower bounds
        errs.append(np.abs(s - exact).max() / exact[0])
    assert errs[2] < errs[0] and errs[2] < 1e-3


def test_error_is_near_optimal_and_the_right_factor_orthonormal():
    rng = np.random.default_rng(2)
    N, K, r, ell = 256, 192, 8, 16
    s_true = np.concatenate([10.0 / (1 + np.arange(8)), 0.05 * np.ones(184)])
    Wb = _weight_bits(N, K, s_true, 2)
    lam = np.ones(K, np.float32)
    A = _A(Wb, lam)
    sv = np.linalg.svd(A, compute_uv=False)
    optimal = np.sqrt((sv[r:] ** 2).sum())
    down, up, s, L1, L2 = OS.randomized_factors(Wb, lam, r, rng.standard_normal((N, ell)), 2)
    err = np.linalg.norm(A - L1 @ L2)
    assert optimal <= err <= 1.01 * optimal
    assert np.allclose(L2 @ L2.T, np.eye(r), atol=1e-12)
    # the bf16 factors: error within the rounding of the factors
    Ab = bf16_bits_to_f32(down).astype(np.float64).T @ bf16_bits_to_f32(up).astype(np.float64).T
    assert np.linalg.norm(A - Ab) <= 1.02 * optimal
