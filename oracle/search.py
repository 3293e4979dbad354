"""λ grid search against the layer's output error.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on", sections "Calibration"
(a grid of 39 candidate λ, built from the activation statistics accumulated under a modality
mask, each scored with the OutputsError objective) and "The metric that picks the winner also
hides the cost" (that objective is the relative L2 of the layer output against bf16, on rows
drawn uniformly from the packed sequence, the rank-32 branch included).

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
  * the 100 iterations of low-rank refit that the page runs for each candidate are not part of
    this search (the page does not define them).
"""
import numpy as np

from . import calib, layer, score, svd

F32 = np.float32


def alpha_grid(n=39):
    """α_i = i/(n+1), i = 1..n, as float32."""
    return (np.arange(1, n + 1, dtype=np.float64) / (n + 1)).astype(F32)


def candidate(X_bits, W_bits, ax, aw, mask, alpha, fmt, rows, omega=None, r=0, power_iters=2):
    """Score of one α: (rel float64, λ float32 [K])."""
    W_bits = np.asarray(W_bits)
    N, K = W_bits.shape
    lam = calib.lambda_from_stats(ax, aw, mask, alpha)
    act_amax = calib.act_amax_from_stats(ax, lam)
    if r > 0:
        down, up = svd.randomized_factors(W_bits, lam, r, omega, power_iters)[:2]
    else:
        down = np.zeros((0, K), np.uint16)
        up = np.zeros((N, 0), np.uint16)
    wt = layer.prepare_weight(W_bits, lam, down, up, fmt)
    Xs = np.asarray(X_bits)[rows]
    act = layer.prepare_activation(Xs, lam, act_amax, down, fmt)
    _, Y = layer.forward(act, wt, up, fmt)
    Yref = score.reference_rows(X_bits, W_bits, rows)
    sums = score.modal_sums(Y, Yref, np.full(len(rows), 3))
    d, ref = sums[3]
    rel = float(np.sqrt(d) / np.sqrt(ref)) if ref > 0 else float("inf")
    return rel, lam


def lambda_search(X_bits, W_bits, ax, aw, mask, alphas, fmt, rows, omega=None, r=0,
                  power_iters=2):
    """(scores float64 [n], best λ float32 [K], best index): the first α of smallest score."""
    scores, lams = [], []
    for a in alphas:
        rel, lam = candidate(X_bits, W_bits, ax, aw, mask, F32(a), fmt, rows, omega, r,
                             power_iters)
        scores.append(rel)
        lams.append(lam)
    scores = np.array(scores)
    best = 0
    for i in range(1, len(scores)):
        if scores[i] < scores[best] or np.isnan(scores[best]):
            best = i
    return scores, lams[best], best
