"""GPU parity of the λ grid search (svdq_lambda_search) with the oracle's search on the same
seeded inputs, random matrix Ω and sampled rows.

Tolerance, derived from the layer's own parity bar: the GPU output Y of a candidate is within
rel-L2 1e-3 of the oracle's, and |rel(Y) − rel(Y')| <= ||Y − Y'|| / ||Y_ref||, so without the
rank-r branch each score agrees with the oracle's to 1e-3 · (1 + score) absolute.  With the
branch the factors come from fp32 arithmetic on the GPU and float64 in the oracle and are
unique only up to bf16 rounding, so a few residual codes may move; there the bound is 2 % of
the score plus the same 1e-3 · (1 + score).  The winner must be the oracle's winner or score
within that tolerance of it, and the λ returned must be the winner's λ (to the one float32 ulp
by which float64 powers of two math libraries may differ)."""
import numpy as np
import pytest

import synth
from oracle import search as OSe, calib as OC
from tests.gpu_common import dev_bf16, dev, torch_mod

pytestmark = pytest.mark.gpu

F32 = np.float32
FMT = {"nvfp4": 0, "int4": 1, "mxfp4": 2, "mxfp8": 3}


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _case(M, K, N, seed=0):
    cfg = dict(synth.config(0), M=M, K=K, N=N, seg=synth.segments(M, 16, 16))
    X = synth.x_bits(cfg, seed=seed)
    W = synth.weight_bits(N, K, seed=seed)
    ax, aw, _, _ = OC.calibrate(X, cfg["seg"], W, 7)
    return X, W, ax, aw


def _run(L, X, W, ax, aw, alphas, fmt, rows, omega, r, q, mask=7):
    torch = torch_mod()
    state = dict(ax=dev(ax), aw=dev(aw))
    om = dev(omega) if r > 0 else None
    scores, best, idx = L.lambda_search(dev_bf16(X), dev_bf16(W), state, [float(a) for a in alphas],
                                        dev(rows.astype(np.int32)), FMT[fmt], om, r, q, mask)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), best.cpu().numpy(), int(idx.cpu().numpy()[0])


def _check(L, X, W, ax, aw, alphas, fmt, rows, r, q=2, ell=None, mask=7, seed=5):
    N = W.shape[0]
    ell = ell or r + 8
    omega = np.random.default_rng(seed).standard_normal((N, ell)).astype(F32) if r else None
    g_scores, g_lam, g_idx = _run(L, X, W, ax, aw, alphas, fmt, rows, omega, r, q, mask)
    o_scores, o_lam, o_idx = OSe.lambda_search(X, W, ax, aw, mask, alphas, fmt, rows, omega, r, q)
    tol = 1e-3 * (1 + o_scores) + (0.02 * o_scores if r else 0.0)
    worst = np.max(np.abs(g_scores - o_scores) / o_scores)
    print(f"[search] {fmt} r={r} {X.shape}x{W.shape} rows={len(rows)} n_alpha={len(alphas)}: "
          f"worst relative score difference {worst:.3e}, GPU best {g_idx} ({g_scores[g_idx]:.5f})"
          f", oracle best {o_idx} ({o_scores[o_idx]:.5f})", flush=True)
    assert np.all(np.abs(g_scores - o_scores) <= tol), (g_scores, o_scores)
    assert g_idx == int(np.argmin(g_scores))
    assert o_scores[g_idx] <= o_scores[o_idx] + 2 * tol[o_idx]
    # λ of a general α comes from float64 powers, which the GPU's and the host's math
    # libraries may round differently in the last place: within one float32 ulp
    o_lam = OC.lambda_from_stats(ax, aw, mask, F32(alphas[g_idx]))
    ulp = np.abs(g_lam.view(np.int32).astype(np.int64) - o_lam.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1


@pytest.fixture(scope="module")
def small():
    return _case(640, 512, 256)


def test_full_grid_nvfp4_without_branch(L, small):
    X, W, ax, aw = small
    rows = np.sort(np.random.default_rng(1).choice(X.shape[0], 200, replace=False))
    _check(L, X, W, ax, aw, OSe.alpha_grid(), "nvfp4", rows, r=0)


def test_full_grid_nvfp4_rank8(L, small):
    X, W, ax, aw = small
    rows = np.sort(np.random.default_rng(2).choice(X.shape[0], 200, replace=False))
    _check(L, X, W, ax, aw, OSe.alpha_grid(), "nvfp4", rows, r=8, ell=16)


@pytest.mark.parametrize("fmt,r", [("int4", 8), ("int4", 0), ("mxfp4", 0), ("mxfp4", 16),
                                   ("mxfp8", 8)])
def test_other_formats_on_every_fourth_point(L, small, fmt, r):
    X, W, ax, aw = small
    rows = np.random.default_rng(3).choice(X.shape[0], 130, replace=False)   # unsorted
    _check(L, X, W, ax, aw, OSe.alpha_grid()[1::4], fmt, rows, r=r)


def test_single_modality_mask_and_repeated_rows(L, small):
    X, W, ax, aw = small
    rows = np.random.default_rng(4).integers(0, X.shape[0], 77)            # with repeats
    _check(L, X, W, ax, aw, [F32(0.2), F32(0.5), F32(0.8)], "nvfp4", rows, r=8, mask=2)


def test_one_sampled_row_and_one_candidate(L, small):
    X, W, ax, aw = small
    _check(L, X, W, ax, aw, [F32(0.5)], "nvfp4", np.array([17]), r=0)


def test_full_size_attention_projection(L):
    """5120 x 5120, rank 32, 1024 uniform rows of a 16384-row packed sequence: three candidates
    against the oracle, then the whole 39-point grid timed."""
    torch = torch_mod()
    cfg = synth.config(1)
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    print(f"[search] full size {cfg['name']}", flush=True)
    X = synth.x_bits(cfg)
    W = synth.weight_bits(N, K)
    ax, aw, _, _ = OC.calibrate(X, cfg["seg"], W, 7)
    rows = np.sort(np.random.default_rng(6).choice(M, 1024, replace=False))
    _check(L, X, W, ax, aw, [F32(0.25), F32(0.5), F32(0.75)], "nvfp4", rows, r=32, ell=40)

    omega = np.random.default_rng(7).standard_normal((N, 40)).astype(F32)
    Xd, Wd, od = dev_bf16(X), dev_bf16(W), dev(omega)
    state = dict(ax=dev(ax), aw=dev(aw))
    rd = dev(rows.astype(np.int32))
    grid = [float(a) for a in OSe.alpha_grid()]
    L.lambda_search(Xd, Wd, state, grid, rd, 0, od, 32, 2)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    scores, best, idx = L.lambda_search(Xd, Wd, state, grid, rd, 0, od, 32, 2)
    t1.record()
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    assert np.all(np.isfinite(s)) and int(idx.cpu()[0]) == int(np.argmin(s))
    print(f"[search] 39 candidates at 5120x5120 r=32, 1024 rows: {t0.elapsed_time(t1):.1f} ms, "
          f"best α = {grid[int(idx.cpu()[0])]:.3f} (score {s.min():.5f}, α=0.5: {s[19]:.5f})",
          flush=True)
