"""Per-modality relative-L2 scoring against the unquantised bf16 layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on", section "The metric that
picks the winner also hides the cost": relative L2 against bf16, once over a uniform sample of
all rows of the packed sequence (the column the calibration itself reports) and once per modality.

    rel_μ = sqrt(Σ (Y − Y_ref)²) / sqrt(Σ Y_ref²)   over the sampled rows of group μ,
    Y_ref = bf16(X @ Wᵀ) from the unsmoothed bf16 X and W (product in float64).
Groups: 0 text, 1 video, 2 audio, 3 uniform rows.  Sums are accumulated in float64.
"""
import numpy as np

from .formats import bf16_bits_to_f32
from .gemm import reference_bf16_linear

N_GROUPS = 4


def modal_sums(Y_bits_rows, Yref_bits_rows, row_group):
    """sums[μ] = (Σ (Y − Y_ref)², Σ Y_ref²) over the rows whose group is μ; float64 [4, 2]."""
    Y = bf16_bits_to_f32(Y_bits_rows).astype(np.float64)
    R = bf16_bits_to_f32(Yref_bits_rows).astype(np.float64)
    d2 = ((Y - R) ** 2).sum(axis=1)
    r2 = (R ** 2).sum(axis=1)
    sums = np.zeros((N_GROUPS, 2))
    for mu in range(N_GROUPS):
        sel = np.asarray(row_group) == mu
        sums[mu, 0] = d2[sel].sum()
        sums[mu, 1] = r2[sel].sum()
    return sums


def reference_rows(X_bits, W_bits, rows):
    """Y_ref for the given rows."""
    return reference_bf16_linear(np.asarray(X_bits)[rows], W_bits)


def rel_l2(sums):
    """rel_μ from the sums (NaN for an empty group)."""
    sums = np.asarray(sums, dtype=np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.sqrt(sums[:, 0]) / np.sqrt(sums[:, 1])
