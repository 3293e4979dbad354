"""Pins of the oracle's λ grid search ("MiniMax-H3 NVFP4 — what the smoothing scale should be
calibrated on", sections "Calibration" and "The metric that picks the winner also hides the
cost") against facts the method fixes: a layer whose operands sit on the quantiser's grid has
zero error where λ = 1; a λ made of powers of two that are constant over each quantiser block
changes nothing (dividing X by 2^j and multiplying W by 2^j is exact and moves only the block
scales); the winner is
the first α of smallest score; quantisation is per row, so scoring sampled rows equals
sampling the full layer's rows; the rank-r branch lowers the error on outlier data."""
import numpy as np
import pytest

import synth
from oracle import search as OSe, calib as OC, layer as OL, score as OSc
from oracle.formats import bf16_rne

F32 = np.float32


def _grid_operand(rng, R, K, values, block, top):
    """R x K values drawn from `values`, with ±top at the start of every block of each row."""
    x = rng.choice(values, size=(R, K)) * rng.choice([-1.0, 1.0], size=(R, K))
    x[:, ::block] = top * rng.choice([-1.0, 1.0], size=(R, K // block))
    return bf16_rne(x)


def test_grid_has_39_points_inside_the_unit_interval_with_one_half_among_them():
    a = OSe.alpha_grid()
    assert a.dtype == F32 and len(a) == 39
    assert np.all(np.diff(a.astype(np.float64)) > 0) and a[0] > 0 and a[-1] < 1
    assert F32(0.5) in a
    assert np.allclose(np.diff(a.astype(np.float64)), 1 / 40, rtol=0, atol=2.0 ** -23)


@pytest.mark.parametrize("fmt,values,block,top", [
    ("mxfp4", [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], 32, 6.0),
    ("int4", list(range(8)), 64, 7.0),
])
def test_operands_on_the_quantiser_grid_have_zero_error_at_lambda_one(fmt, values, block, top):
    rng = np.random.default_rng(0)
    M, N, K = 96, 64, 256
    X = _grid_operand(rng, M, K, values, block, top)
    W = _grid_operand(rng, N, K, values, block, top)
    ax = np.full((3, K), top, F32)           # equal activation and weight maxima: λ(½) = 1
    aw = np.full(K, top, F32)
    rows = np.sort(rng.choice(M, 40, replace=False))
    alphas = OSe.alpha_grid()
    scores, lam, best = OSe.lambda_search(X, W, ax, aw, 7, alphas, fmt, rows)
    half = int(np.flatnonzero(alphas == F32(0.5))[0])
    assert scores[half] == 0.0
    assert np.all(scores >= 0)
    assert best == int(np.flatnonzero(scores == 0.0)[0])       # the first of the zero scores
    assert np.array_equal(lam, OC.lambda_from_stats(ax, aw, 7, alphas[best]))


def test_blockwise_power_of_two_lambda_changes_no_mx_score():
    rng = np.random.default_rng(1)
    cfg = synth.config(0)
    X = synth.gen.x_bits(cfg)
    W = synth.gen.weight_bits(cfg["N"], cfg["K"])
    K = cfg["K"]
    j = rng.integers(-3, 4, K // 32)                          # λ = 2^j on each 32-block
    aw = np.exp(rng.normal(0, 0.3, K)).astype(F32)
    aw = np.ldexp(np.round(np.frexp(aw)[0] * 256) / 256, np.frexp(aw)[1]).astype(F32)
    ax = np.tile(np.ldexp(aw, np.repeat(2 * j, 32)), (3, 1)).astype(F32)   # ax/aw = 4^j
    rows = np.sort(rng.choice(cfg["M"], 64, replace=False))
    lam = OC.lambda_from_stats(ax, aw, 7, 0.5)
    assert np.array_equal(lam, np.ldexp(F32(1), np.repeat(j, 32)).astype(F32))
    for fmt in ("mxfp4", "mxfp8"):
        s_pow2, _ = OSe.candidate(X, W, ax, aw, 7, F32(0.5), fmt, rows)
        s_one, lam1 = OSe.candidate(X, W, ax, aw, 0, F32(0.5), fmt, rows)   # mask 0: λ = 1
        assert np.all(lam1 == 1)
        assert s_pow2 > 0 and abs(s_pow2 - s_one) <= 1e-12 * s_one, (fmt, s_pow2, s_one)


def test_first_of_equal_scores_wins():
    cfg = synth.config(0)
    X = synth.gen.x_bits(cfg)
    W = synth.gen.weight_bits(cfg["N"], cfg["K"])
    ax, aw, _, _ = OC.calibrate(X, cfg["seg"], W, 7)
    rows = np.arange(0, cfg["M"], 3)
    a = [F32(0.3), F32(0.6), F32(0.3), F32(0.6)]
    scores, lam, best = OSe.lambda_search(X, W, ax, aw, 7, a, "nvfp4", rows)
    assert scores[0] == scores[2] and scores[1] == scores[3] and scores[0] != scores[1]
    assert best == (0 if scores[0] < scores[1] else 1)


def test_scoring_sampled_rows_equals_sampling_the_full_layer():
    cfg = synth.config(0)
    X = synth.gen.x_bits(cfg)
    W = synth.gen.weight_bits(cfg["N"], cfg["K"])
    ax, aw, _, _ = OC.calibrate(X, cfg["seg"], W, 7)
    rng = np.random.default_rng(2)
    rows = rng.choice(cfg["M"], 100, replace=False)
    for fmt in ("nvfp4", "int4", "mxfp8"):
        s, lam = OSe.candidate(X, W, ax, aw, 7, F32(0.35), fmt, rows)
        amax = OC.act_amax_from_stats(ax, lam)
        K, N = cfg["K"], cfg["N"]
        down, up = np.zeros((0, K), np.uint16), np.zeros((N, 0), np.uint16)
        wt = OL.prepare_weight(W, lam, down, up, fmt)
        act = OL.prepare_activation(X, lam, amax, down, fmt)        # every row, then sample
        _, Y = OL.forward(act, wt, up, fmt, rows=rows)
        sums = OSc.modal_sums(Y, OSc.reference_rows(X, W, rows), np.full(len(rows), 3))
        full = float(np.sqrt(sums[3, 0]) / np.sqrt(sums[3, 1]))
        assert abs(s - full) <= 1e-12 * full, (fmt, s, full)
        s_perm, _ = OSe.candidate(X, W, ax, aw, 7, F32(0.35), fmt, rows[::-1].copy())
        assert abs(s_perm - s) <= 1e-12 * s


def test_the_low_rank_branch_lowers_the_error_on_outlier_data():
    cfg = synth.config(0)
    X = synth.gen.x_bits(cfg)
    W = synth.gen.weight_bits(cfg["N"], cfg["K"])
    ax, aw, _, _ = OC.calibrate(X, cfg["seg"], W, 7)
    rows = np.arange(cfg["M"])
    omega = np.random.default_rng(3).standard_normal((cfg["N"], 16)).astype(F32)
    alphas = [F32(0.25), F32(0.5), F32(0.75)]
    s0, _, _ = OSe.lambda_search(X, W, ax, aw, 7, alphas, "nvfp4", rows)
    s8, _, _ = OSe.lambda_search(X, W, ax, aw, 7, alphas, "nvfp4", rows, omega, 8, 2)
    assert np.all(s8 < s0), (s0, s8)


@pytest.mark.parametrize("fmt", ["nvfp4", "int4", "mxfp4"])
def test_each_refit_step_lowers_the_weight_error_for_the_fixed_quantised_residual(fmt):
    # iterate t + 1 takes the best rank-r approximation of E_t = W' − deq(Q(R_t)), so for that
    # fixed quantised residual it is no worse than iterate t's branch (Eckart–Young; the power
    # iterations make the randomized factors optimal to rounding at this size), up to the bf16
    # rounding of the new factors
    from oracle import svd as OS
    from oracle.formats import bf16_bits_to_f32
    cfg = synth.config(0)
    X = synth.gen.x_bits(cfg)
    W = synth.gen.weight_bits(cfg["N"], cfg["K"])
    ax, aw, _, _ = OC.calibrate(X, cfg["seg"], W, 7)
    r = 8
    omega = np.random.default_rng(4).standard_normal((cfg["N"], 24)).astype(F32)
    s, lam, facs = OSe.candidate_iterates(X, W, ax, aw, 7, F32(0.5), fmt, np.arange(64), omega,
                                          r, power_iters=6, refit_iters=3)
    Wp = OS.smoothed_weight(W, lam)

    def branch(f):
        d = bf16_bits_to_f32(f[0]).astype(np.float64)
        u = bf16_bits_to_f32(f[1]).astype(np.float64)
        return u @ d                                          # [N, K]

    for t in range(3):
        wt = OL.prepare_weight(W, lam, facs[t][0], facs[t][1], fmt)
        E = Wp - OSe.dequantized_weight(wt, fmt)
        # bf16 rounding moves each factor by at most 2^-9 of itself, so the branch moves by at
        # most about 2^-8 · ||up||_F · ||down||_F
        d = bf16_bits_to_f32(facs[t + 1][0]).astype(np.float64)
        u = bf16_bits_to_f32(facs[t + 1][1]).astype(np.float64)
        rounding = 1.01 * 2.0 ** -8 * np.linalg.norm(u) * np.linalg.norm(d)
        before = np.linalg.norm(E - branch(facs[t]))
        after = np.linalg.norm(E - branch(facs[t + 1]))
        assert after <= before + rounding, (fmt, t, before, after, rounding)
        # the unrounded new branch is the best rank-r approximation of E_t (an exact SVD; the
        # singular values fall from about 20 to about 2 after the r-th, so it is unique)
        U, sv, Vt = np.linalg.svd(E, full_matrices=False)
        best_r = (U[:, :r] * sv[:r]) @ Vt[:r]
        assert sv[r - 1] > 5 * sv[r]
        assert np.linalg.norm(facs[t + 1][2] - best_r) <= 1e-9 * np.linalg.norm(best_r)
    assert len(s) == 4 and np.all(np.isfinite(s))


def test_refit_needs_a_branch_and_zero_iterations_is_the_plain_candidate():
    cfg = synth.config(0)
    X = synth.gen.x_bits(cfg)
    W = synth.gen.weight_bits(cfg["N"], cfg["K"])
    ax, aw, _, _ = OC.calibrate(X, cfg["seg"], W, 7)
    with pytest.raises(ValueError):
        OSe.candidate(X, W, ax, aw, 7, F32(0.5), "nvfp4", np.arange(8), refit_iters=2)
    omega = np.random.default_rng(5).standard_normal((cfg["N"], 16)).astype(F32)
    s3, _, f3 = OSe.candidate_iterates(X, W, ax, aw, 7, F32(0.5), "nvfp4", np.arange(64), omega,
                                       8, 2, 3)
    s0, _, f0 = OSe.candidate_iterates(X, W, ax, aw, 7, F32(0.5), "nvfp4", np.arange(64), omega,
                                       8, 2, 0)
    assert s3[0] == s0[0] and np.array_equal(f3[0][0], f0[0][0])
    sc, _ = OSe.candidate(X, W, ax, aw, 7, F32(0.5), "nvfp4", np.arange(64), omega, 8, 2, 3)
    assert sc == s3.min()
