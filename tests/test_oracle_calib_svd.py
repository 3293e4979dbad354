"""Pins of the oracle's calibration, smoothing and low-rank steps: brute-force loops, closed
forms, the smoothing identity, brute-force rank-1 approximation and Eckart-Young."""
import itertools

import numpy as np

from oracle import calib as C
from oracle import svd as S
from oracle import formats as F
import synth

F32 = np.float32


def _tiny_inputs(seed=0, M=12, K=16, N=5):
    rng = np.random.default_rng(seed)
    X = synth.to_bf16_bits(rng.standard_normal((M, K)) * np.exp(rng.standard_normal(K)))
    W = synth.to_bf16_bits(rng.standard_normal((N, K)))
    return X, W, (0, 2, 9, M)


def test_channel_absmax_brute_force_loops():
    X, W, seg = _tiny_inputs()
    ax = C.channel_absmax_per_modality(X, seg)
    xf = F.bf16_bits_to_f32(X)
    for mu in range(3):
        for k in range(X.shape[1]):
            m = 0.0
            for row in range(seg[mu], seg[mu + 1]):
                m = max(m, abs(float(xf[row, k])))
            assert ax[mu, k] == m
    aw = C.weight_absmax(W)
    wf = F.bf16_bits_to_f32(W)
    for k in range(W.shape[1]):
        assert aw[k] == max(abs(float(wf[n, k])) for n in range(W.shape[0]))


def test_lambda_closed_forms_and_guards():
    ax = np.array([[4.0, 0.0, 9.0, 1.0], [1.0, 1.0, 1.0, 1.0], [0.0, 0.0, 0.0, 0.0]], dtype=F32)
    aw = np.array([1.0, 1.0, 4.0, 0.0], dtype=F32)
    lam = C.lambda_from_stats(ax, aw, 1)             # text only
    assert lam.tolist() == [2.0, 1.0, 1.5, 1.0]       # sqrt(4/1), guard ax=0, sqrt(9/4), guard aw=0
    assert np.all(C.lambda_from_stats(ax, aw, 0) == 1.0)
    lam_v = C.lambda_from_stats(ax, aw, 2)            # video only
    assert lam_v.tolist() == [1.0, 1.0, 0.5, 1.0]
    lam_all = C.lambda_from_stats(ax, aw, 7)
    assert lam_all.tolist() == [2.0, 1.0, 1.5, 1.0]
    lam_a = C.lambda_from_stats(ax, aw, 7, alpha=0.25)
    assert np.isclose(lam_a[0], 4.0 ** 0.25, rtol=1e-7) and np.isclose(lam_a[2], 9 ** .25 / 4 ** .75)


def test_mask_ignores_rows_of_other_modalities():
    X, W, seg = _tiny_inputs(1)
    _, _, lam_t, _ = C.calibrate(X, seg, W, 1)
    X2 = X.copy()
    X2[seg[1]:seg[2]] = synth.to_bf16_bits(np.full((seg[2] - seg[1], X.shape[1]), 1e4))
    _, _, lam_t2, _ = C.calibrate(X2, seg, W, 1)
    assert np.array_equal(lam_t, lam_t2)
    _, _, lam_v2, _ = C.calibrate(X2, seg, W, 2)
    assert not np.array_equal(lam_t, lam_v2)


def test_static_act_amax_equals_dynamic_max_of_smoothed():
    X, W, seg = _tiny_inputs(2, M=40, K=64)
    for mask in (0, 1, 2, 4, 7):
        ax, aw, lam, amax = C.calibrate(X, seg, W, mask)
        xhat = C.smooth(X, lam)
        assert amax == np.abs(xhat).max()


def test_smoothing_identity_and_unit_lambda():
    X, W, seg = _tiny_inputs(3, M=20, K=32, N=7)
    _, _, lam, _ = C.calibrate(X, seg, W, 7)
    x64 = F.bf16_bits_to_f32(X).astype(np.float64)
    w64 = F.bf16_bits_to_f32(W).astype(np.float64)
    lhs = (x64 / lam.astype(np.float64)) @ S.smoothed_weight(W, lam).T
    rhs = x64 @ w64.T
    assert np.max(np.abs(lhs - rhs)) <= 1e-13 * np.max(np.abs(rhs))
    xhat = C.smooth(X, lam).astype(np.float64)
    assert np.all(np.abs(xhat - x64 / lam) <= np.abs(x64 / lam) * 2.0 ** -23)
    assert np.array_equal(C.smooth(X, np.ones(X.shape[1], F32)), F.bf16_bits_to_f32(X))


def test_rank1_svd_beats_brute_force_grid_2x2_and_3x3():
    rng = np.random.default_rng(4)
    for n in (2, 3):
        A = rng.standard_normal((n, n))
        U, s, Vt = S.truncated_svd(A, 1)
        err = np.linalg.norm(A - (U * s) @ Vt)
        sv = np.sqrt(np.sort(np.linalg.eigvalsh(A @ A.T))[::-1])
        assert np.isclose(err, np.sqrt((sv[1:] ** 2).sum()), rtol=1e-10)
        # brute force over unit vectors u, v (angle grids); best σ for fixed u, v is uᵀAv
        angles = np.linspace(0, np.pi, 181)
        if n == 2:
            units = [np.array([np.cos(a), np.sin(a)]) for a in angles]
        else:
            units = [np.array([np.sin(a) * np.cos(b), np.sin(a) * np.sin(b), np.cos(a)])
                     for a, b in itertools.product(angles[::6], np.linspace(0, 2 * np.pi, 61))]
        Uu = np.array(units)
        sig = Uu @ A @ Uu.T                     # best σ for each (u, v) pair is uᵀAv
        iu, iv = np.unravel_index(np.argmax(np.abs(sig)), sig.shape)
        best = np.linalg.norm(A - sig[iu, iv] * np.outer(Uu[iu], Uu[iv]))
        for j in range(0, len(units), max(1, len(units) // 40)):   # direct norms on a subset
            assert np.linalg.norm(A - sig[j, j] * np.outer(Uu[j], Uu[j])) >= err - 1e-12
        assert err <= best + 1e-12
        assert best <= err * 1.05 + 1e-3


def test_eckart_young_orthonormality_and_factor_layout():
    rng = np.random.default_rng(5)
    A = rng.standard_normal((40, 30))
    for r in (1, 5, 12):
        U, s, Vt = S.truncated_svd(A, r)
        assert np.allclose(U.T @ U, np.eye(r), atol=1e-12)
        assert np.allclose(Vt @ Vt.T, np.eye(r), atol=1e-12)
        sv = np.sqrt(np.sort(np.linalg.eigvalsh(A.T @ A))[::-1])
        assert np.isclose(np.linalg.norm(A - (U * s) @ Vt) ** 2, (sv[r:] ** 2).sum(), rtol=1e-9)


def test_partial_svd_path_matches_full_svd_path(monkeypatch):
    rng = np.random.default_rng(6)
    A = rng.standard_normal((2100, 64)) @ rng.standard_normal((64, 2100)) * 0.01
    A += rng.standard_normal(A.shape) * 1e-3
    U1, s1, V1 = S.truncated_svd(A, 8)
    assert np.allclose(s1, np.linalg.svd(A[:, :], compute_uv=False)[:8], rtol=1e-9)
    assert np.allclose(np.abs(U1.T @ U1), np.eye(8), atol=1e-9)


def test_lowrank_factors_and_residual_reconstruct_smoothed_weight():
    X, W, seg = _tiny_inputs(7, M=16, K=48, N=24)
    _, _, lam, _ = C.calibrate(X, seg, W, 7)
    down, up = S.lowrank_factors(W, lam, 6)
    assert down.shape == (6, 48) and up.shape == (24, 6)
    R32 = S.residual_f32(W, lam, down, up)
    Wp = S.smoothed_weight(W, lam)
    recon = F.bf16_bits_to_f32(up).astype(np.float64) @ F.bf16_bits_to_f32(down).astype(np.float64)
    assert np.all(np.abs(Wp - recon - R32) <= np.abs(Wp - recon) * 2.0 ** -24 + 1e-300)
    # rank-6 branch captures most of W' (residual well below W')
    assert np.linalg.norm(R32) < 0.8 * np.linalg.norm(Wp)
    assert np.array_equal(S.residual_f32(W, lam, down[:0], up[:, :0]), Wp.astype(F32))
