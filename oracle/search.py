"""λ grid search against the layer's output error.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on", sections "Calibration"
(a grid of 39 candidate λ, built from the activation statistics accumulated under a modality
mask, each scored with the OutputsError objective) and "The metric that picks the winner also
hides the cost" (the objective: relative L2 of the layer's output against the bf16 layer over a
uniform sample of all rows, with the rank-32 branch in the output).

Readings where the pages are silent:
  * the grid is the migration strength α of λ_k = a_k^α / w_k^(1−α) (a_k the masked
    activation absmax, w_k the weight absmax) at α_i = i/40, i = 1..39: 39 points strictly
    inside (0, 1), α = 1/2 among them;
  * for every candidate the whole layer is rebuilt from λ_α: the static activation amax of
    λ_α, rank-r factors of diag(λ_α)·Wᵀ (the randomized factors, Ω an input; none when r = 0),
    the quantised residual, and the quantised sampled rows;
  * the score of a candidate is rel = sqrt(Σ(Y − Y_ref)²) / sqrt(Σ Y_ref²) over the sampled
    rows (Y_ref = bf16(X·Wᵀ)), +inf when Σ Y_ref² = 0; the winner is the first α of smallest
    score;
  * the low-rank refit the page runs for each candidate (100 iterations, against the same
    objective) is not defined there; the reading is the alternating refit: iterate t + 1 takes
    the rank-r factors (randomized, the same Ω) of E_t = W' − deq(Q(R_t)), what the quantised
    residual of iterate t leaves of the smoothed weight W' = λ·W, exact in float64; iterate 0
    is the factors of W' itself; every iterate is scored like the first and the candidate's
    score is the smallest over its iterates (the first of equal ones is kept).
"""
import numpy as np

from . import calib, layer, score, svd, quant, mx

F32 = np.float32


def alpha_grid(n=39):
    """α_i = i/(n+1), i = 1..n, as float32."""
    return (np.arange(1, n + 1, dtype=np.float64) / (n + 1)).astype(F32)


def dequantized_weight(wt, fmt):
    """Exact float64 values of a prepared weight's codes [N, K]."""
    if fmt in layer.MX_ELEM:
        return mx.mx_dequantize(wt["codes"], wt["scales"], layer.MX_ELEM[fmt])
    if fmt == "int4":
        return quant.int4_dequantize(wt["codes"], wt["scales"])
    return quant.nvfp4_dequantize(wt["codes"], wt["scales"], wt["g"])


def _score(X_bits, W_bits, lam, act_amax, down, up, fmt, rows, Yref):
    wt = layer.prepare_weight(W_bits, lam, down, up, fmt)
    act = layer.prepare_activation(np.asarray(X_bits)[rows], lam, act_amax, down, fmt)
    _, Y = layer.forward(act, wt, up, fmt)
    sums = score.modal_sums(Y, Yref, np.full(len(rows), 3))
    d, ref = sums[3]
    rel = float(np.sqrt(d) / np.sqrt(ref)) if ref > 0 else float("inf")
    return rel, wt


def candidate_iterates(X_bits, W_bits, ax, aw, mask, alpha, fmt, rows, omega=None, r=0,
                       power_iters=2, refit_iters=0):
    """All iterates of one α: (scores float64 [refit_iters + 1], λ float32 [K],
    factors [(lora_down bits, lora_up bits, unrounded branch L1·L2 as [N, K] float64 or None)]
    per iterate)."""
    W_bits = np.asarray(W_bits)
    N, K = W_bits.shape
    if refit_iters and not r:
        raise ValueError("refit iterations need a low-rank branch")
    lam = calib.lambda_from_stats(ax, aw, mask, alpha)
    act_amax = calib.act_amax_from_stats(ax, lam)
    if r > 0:
        down, up, _, L1, L2 = svd.randomized_factors(W_bits, lam, r, omega, power_iters)
        branch = (L1 @ L2).T
    else:
        down = np.zeros((0, K), np.uint16)
        up = np.zeros((N, 0), np.uint16)
        branch = None
    Yref = score.reference_rows(X_bits, W_bits, rows)
    Wp = svd.smoothed_weight(W_bits, lam)
    scores, factors = [], []
    for t in range(refit_iters + 1):
        rel, wt = _score(X_bits, W_bits, lam, act_amax, down, up, fmt, rows, Yref)
        scores.append(rel)
        factors.append((down, up, branch))
        if t < refit_iters:
            E = Wp - dequantized_weight(wt, fmt)          # [N, K]
            down, up, _, L1, L2 = svd.randomized_factors_of(E.T, r, omega, power_iters)
            branch = (L1 @ L2).T
    return np.array(scores), lam, factors


def _first_min(scores):
    best = 0
    for i in range(1, len(scores)):
        if scores[i] < scores[best] or np.isnan(scores[best]):
            best = i
    return best


def candidate(X_bits, W_bits, ax, aw, mask, alpha, fmt, rows, omega=None, r=0, power_iters=2,
              refit_iters=0):
    """Score of one α (the smallest over its iterates): (rel float64, λ float32 [K])."""
    s, lam, _ = candidate_iterates(X_bits, W_bits, ax, aw, mask, alpha, fmt, rows, omega, r,
                                   power_iters, refit_iters)
    return float(s[_first_min(s)]), lam


def lambda_search(X_bits, W_bits, ax, aw, mask, alphas, fmt, rows, omega=None, r=0,
                  power_iters=2, refit_iters=0, details=False):
    """(scores float64 [n], best λ float32 [K], best index): the first α of smallest score.
    With details, a fourth item: dict(iter_scores [n, refit_iters + 1], factors of the winner's
    best iterate)."""
    scores, lams, its, facs = [], [], [], []
    for a in alphas:
        s, lam, f = candidate_iterates(X_bits, W_bits, ax, aw, mask, F32(a), fmt, rows, omega, r,
                                       power_iters, refit_iters)
        t = _first_min(s)
        scores.append(s[t])
        lams.append(lam)
        its.append(s)
        facs.append(f[t][:2])
    scores = np.array(scores)
    best = _first_min(scores)
    if details:
        return scores, lams[best], best, dict(iter_scores=np.array(its), factors=facs[best])
    return scores, lams[best], best
