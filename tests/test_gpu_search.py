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


def _run(L, X, W, ax, aw, alphas, fmt, rows, omega, r, q, mask=7, refit=0):
    torch = torch_mod()
    state = dict(ax=dev(ax), aw=dev(aw))
    om = dev(omega) if r > 0 else None
    out = L.lambda_search(dev_bf16(X), dev_bf16(W), state, [float(a) for a in alphas],
                          dev(rows.astype(np.int32)), FMT[fmt], om, r, q, mask, refit_iters=refit,
                          per_iterate=True)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


def _check(L, X, W, ax, aw, alphas, fmt, rows, r, q=2, ell=None, mask=7, seed=5, refit=0):
    N = W.shape[0]
    ell = ell or r + 8
    omega = np.random.default_rng(seed).standard_normal((N, ell)).astype(F32) if r else None
    g = _run(L, X, W, ax, aw, alphas, fmt, rows, omega, r, q, mask, refit)
    g_scores, g_lam, g_idx = g["scores"].numpy(), g["lam"].numpy(), int(g["index"][0])
    o_scores, o_lam, o_idx, det = OSe.lambda_search(X, W, ax, aw, mask, alphas, fmt, rows, omega,
                                                    r, q, refit, details=True)
    g_it, o_it = g["iter_scores"].numpy(), det["iter_scores"]
    tol_it = 1e-3 * (1 + o_it) + (0.02 * o_it if r else 0.0)
    tol = 1e-3 * (1 + o_scores) + (0.02 * o_scores if r else 0.0)
    worst = np.max(np.abs(g_it - o_it) / o_it)
    print(f"[search] {fmt} r={r} refit={refit} {X.shape}x{W.shape} rows={len(rows)} "
          f"n_alpha={len(alphas)}: worst relative score difference {worst:.3e}, GPU best {g_idx} "
          f"({g_scores[g_idx]:.5f}), oracle best {o_idx} ({o_scores[o_idx]:.5f})", flush=True)
    assert np.all(np.abs(g_it - o_it) <= tol_it), (g_it, o_it)
    assert np.array_equal(g_scores, g_it.min(axis=1))
    assert np.all(np.abs(g_scores - o_scores) <= tol), (g_scores, o_scores)
    assert g_idx == int(np.argmin(g_scores))
    assert o_scores[g_idx] <= o_scores[o_idx] + 2 * tol[o_idx]
    # λ of a general α comes from float64 powers, which the GPU's and the host's math
    # libraries may round differently in the last place: within one float32 ulp
    o_lam = OC.lambda_from_stats(ax, aw, mask, F32(alphas[g_idx]))
    ulp = np.abs(g_lam.view(np.int32).astype(np.int64) - o_lam.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1
    return g, det, (o_scores, o_idx)


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


@pytest.mark.parametrize("fmt,r", [("nvfp4", 8), ("int4", 8), ("mxfp4", 16), ("mxfp8", 8)])
def test_refit_iterations(L, small, fmt, r):
    X, W, ax, aw = small
    rows = np.sort(np.random.default_rng(8).choice(X.shape[0], 160, replace=False))
    g, det, _ = _check(L, X, W, ax, aw, OSe.alpha_grid()[3::9], fmt, rows, r=r, refit=4)
    assert g["lora_down"].shape == (r, X.shape[1]) and g["lora_up"].shape == (W.shape[0], r)


@pytest.mark.parametrize("fmt,r", [("nvfp4", 8), ("int4", 8), ("mxfp4", 16), ("mxfp8", 8)])
def test_best_factors_reproduce_the_best_score(L, small, fmt, r):
    """The factors the search returns (possibly from a refit iterate) are scored twice: through
    the layer's own entry points with the winner's λ, and through the oracle's layer with the
    same λ and factors.  Both must give the GPU's winning score to the layer tolerance
    1e-3 · (1 + score): with the factors fixed, the only differences left are the GPU GEMM's
    fp32 accumulation, which the layer parity bar covers."""
    torch = torch_mod()
    X, W, ax, aw = small
    rows = np.sort(np.random.default_rng(9).choice(X.shape[0], 192, replace=False))
    omega = np.random.default_rng(10).standard_normal((W.shape[0], r + 8)).astype(F32)
    g = _run(L, X, W, ax, aw, OSe.alpha_grid()[::6], fmt, rows, omega, r, 2, refit=5)
    i = int(g["index"][0])
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    lam = g["lam"].cuda()
    lam_h = g["lam"].numpy()
    amax_h = OC.act_amax_from_stats(ax, lam_h)
    amax = torch.tensor([amax_h], device="cuda")
    down, up = g["lora_down"].cuda(), g["lora_up"].cuda()
    pw = L.prepare_weight(Wd, lam, down, up, FMT[fmt])
    Xs = Xd[torch.from_numpy(rows).long().cuda()].contiguous()
    codes, scales, ga, D = L.quantize_activation(Xs, lam, amax, down, FMT[fmt])
    Y = L.gemm(codes, scales, ga, D, pw, len(rows))
    torch.cuda.synchronize()
    from oracle import score as OSc
    from tests.gpu_common import host_bits
    Yref = OSc.reference_rows(X, W, rows)
    sums = OSc.modal_sums(host_bits(Y), Yref, np.full(len(rows), 3))
    again = np.sqrt(sums[3, 0]) / np.sqrt(sums[3, 1])
    down_h = g["lora_down"].view(torch.int16).numpy().view(np.uint16)
    up_h = g["lora_up"].view(torch.int16).numpy().view(np.uint16)
    oracle_score, _ = OSe._score(X, W, lam_h, amax_h, down_h, up_h, fmt, rows, Yref)
    best = float(g["scores"][i])
    print(f"[search] {fmt} r={r} best factors: search score {best:.6f}, layer again "
          f"{again:.6f}, oracle with the same factors {oracle_score:.6f}", flush=True)
    assert abs(again - best) <= 1e-3 * (1 + best)
    assert abs(oracle_score - best) <= 1e-3 * (1 + best)


def test_full_size_attention_projection(L):
    """5120 x 5120, rank 32, 1024 uniform rows of a 16384-row packed sequence: three candidates,
    and one with two refit iterations, against the oracle; then the whole 39-point grid and 100
    refit iterations of one candidate timed."""
    torch = torch_mod()
    cfg = synth.config(1)
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    print(f"[search] full size {cfg['name']}", flush=True)
    X = synth.x_bits(cfg)
    W = synth.weight_bits(N, K)
    ax, aw, _, _ = OC.calibrate(X, cfg["seg"], W, 7)
    rows = np.sort(np.random.default_rng(6).choice(M, 1024, replace=False))
    _check(L, X, W, ax, aw, [F32(0.25), F32(0.5), F32(0.75)], "nvfp4", rows, r=32, ell=40)
    _check(L, X, W, ax, aw, [F32(0.5)], "nvfp4", rows, r=32, ell=40, refit=2)

    omega = np.random.default_rng(7).standard_normal((N, 40)).astype(F32)
    Xd, Wd, od = dev_bf16(X), dev_bf16(W), dev(omega)
    state = dict(ax=dev(ax), aw=dev(aw))
    rd = dev(rows.astype(np.int32))
    grid = [float(a) for a in OSe.alpha_grid()]
    L.lambda_search(Xd, Wd, state, grid, rd, 0, od, 32, 2)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    out = L.lambda_search(Xd, Wd, state, grid, rd, 0, od, 32, 2)
    t1.record()
    torch.cuda.synchronize()
    s, i = out["scores"].cpu().numpy(), int(out["index"].cpu()[0])
    assert np.all(np.isfinite(s)) and i == int(np.argmin(s))
    print(f"[search] 39 candidates at 5120x5120 r=32, 1024 rows: {t0.elapsed_time(t1):.1f} ms, "
          f"best α = {grid[i]:.3f} (score {s.min():.5f}, α=0.5: {s[19]:.5f})", flush=True)

    # 100 refit iterations of the branch for one candidate, timed
    t0.record()
    out = L.lambda_search(Xd, Wd, state, [0.5], rd, 0, od, 32, 2, refit_iters=100,
                          per_iterate=True)
    t1.record()
    torch.cuda.synchronize()
    it = out["iter_scores"].cpu().numpy()[0]
    assert np.all(np.isfinite(it)) and out["scores"].cpu().numpy()[0] == it.min()
    print(f"[search] α=0.5 with 100 refits at 5120x5120 r=32: {t0.elapsed_time(t1):.1f} ms; "
          f"score {it[0]:.5f} -> best {it.min():.5f} at iterate {int(np.argmin(it))} "
          f"(iterates 1-5: {np.round(it[1:6], 5).tolist()})", flush=True)
