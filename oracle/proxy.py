"""Statistics-only "bits lost" proxy of a smoothing scale, per modality.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on", section "Why".
The rule, restated: a block scale is fixed by the largest magnitude in its block, so each
channel's resolution shrinks by the ratio of the block maximum to its own maximum, measured in
bits as log2(block max / channel max) after smoothing; changing λ changes those ratios.  The
page ranks candidate λ per modality by this count alone, from calibration statistics.

Readings where the page is silent:
  * the channel absmax of modality μ after smoothing is c_k = fl(ax_μ[k] · fl(1/λ_k)) in
    float32 (the activation kernel's smoothing multiply; the maximum of |X̂| over the rows of μ
    equals it because rounding is monotonic);
  * groups are the quantiser's blocks of consecutive channels (16 for NVFP4, 32 for the MX
    formats, 64 for int4);
  * channel k loses log2(max_{j in its group} c_j / c_k) bits, evaluated in float64; channels
    with c_k = 0 carry no signal and are left out, and the proxy of a modality is the mean over
    the remaining channels (0 when none remain);
  * the page quotes differences of the proxy between two λ; the function returns the proxy
    itself, so a difference is two calls.
"""
import numpy as np

from .calib import inv_lambda

F32 = np.float32


def smoothed_channel_absmax(ax, lam):
    """c[μ, k] = fl(ax[μ, k] · fl(1/λ_k)) in float32 (λ None: λ = 1)."""
    ax = np.asarray(ax, dtype=F32)
    if lam is None:
        return ax.copy()
    return (ax * inv_lambda(lam)[None, :]).astype(F32)


def bits_lost(ax, lam, block=16):
    """Mean bits lost per channel for each modality: float64 [n_modalities]."""
    c = smoothed_channel_absmax(ax, lam).astype(np.float64)
    n_mod, K = c.shape
    if K % block:
        raise ValueError(f"K={K} is not a multiple of the block size {block}")
    groups = c.reshape(n_mod, K // block, block)
    gmax = groups.max(axis=2, keepdims=True)
    live = groups > 0
    bits = np.zeros_like(groups)
    bits[live] = np.log2(np.broadcast_to(gmax, groups.shape)[live] / groups[live])
    out = np.zeros(n_mod)
    for mu in range(n_mod):
        n = int(live[mu].sum())
        out[mu] = float(bits[mu].sum() / n) if n else 0.0
    return out
