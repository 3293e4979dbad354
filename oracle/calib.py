"""λ calibration reduction and smoothing.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on":
  * section "Calibration": the per-channel activation statistics are accumulated under a
    modality mask, and the selected absmax feeds λ;
  * opening section: one λ per input channel is shared by every modality, since the layer's
    single weight (W·λ) serves all of them;
  * section "Why": the kernel sees X / λ.

Readings where the pages are silent:
  * λ formula: the SmoothQuant α-migration, λ_k = ax_k^α / aw_k^(1-α), with ax the selected
    per-channel activation absmax and aw the per-input-channel absmax of the original weight.
    For α = 0.5 it is computed as sqrt(ax / aw) in float32 (division and square root each
    correctly rounded); other α use float64 powers rounded once to float32.  α itself is a
    float32 value (the migration strength as the layer stores it), and both exponents α and
    1 − α are exact in float64.
  * zero guard: λ_k = 1 when ax_k == 0 or aw_k == 0; modality mask 0 means λ = 1.
  * mask selection: ax_sel = max over the modalities whose bit is set (bit 0 text, bit 1 video,
    bit 2 audio) of that modality's absmax (rows of the other modalities are ignored).
  * smoothing divide: X̂ = X * (1/λ) with the reciprocal rounded to float32 once per channel.
  * static activation tensor amax: max_k (ax_all_k * (1/λ_k)) over ALL rows, which equals
    max |X̂| over all rows because rounding is monotonic.
"""
import numpy as np

from .formats import bf16_bits_to_f32

F32 = np.float32
N_MODALITIES = 3          # text, video, audio (packed in that order)


def channel_absmax_per_modality(X_bits, seg):
    """ax[μ, k] = max over the rows of modality μ of |X[m, k]| (0 for an empty modality).

    X_bits: uint16 bf16 [M, K]; seg: 4 offsets {0, n_text, n_text + n_video, M}.
    """
    X_bits = np.asarray(X_bits, dtype=np.uint16)
    M, K = X_bits.shape
    seg = [int(v) for v in seg]
    if seg[0] != 0 or seg[3] != M or not (seg[0] <= seg[1] <= seg[2] <= seg[3]):
        raise ValueError("bad segment offsets")
    ax = np.zeros((N_MODALITIES, K), dtype=F32)
    for mu in range(N_MODALITIES):
        lo, hi = seg[mu], seg[mu + 1]
        for c0 in range(lo, hi, 4096):                      # row chunks bound memory only
            c1 = min(hi, c0 + 4096)
            blk = np.abs(bf16_bits_to_f32(X_bits[c0:c1]))
            ax[mu] = np.maximum(ax[mu], blk.max(axis=0))
    return ax


def weight_absmax(W_bits):
    """aw[k] = max_n |W[n, k]| for W stored [N, K] (out, in)."""
    return np.abs(bf16_bits_to_f32(W_bits)).max(axis=0).astype(F32)


def select_absmax(ax, mask):
    """Max over the modalities whose bit is set in `mask`."""
    K = ax.shape[1]
    sel = np.zeros(K, dtype=F32)
    for mu in range(N_MODALITIES):
        if mask & (1 << mu):
            sel = np.maximum(sel, ax[mu])
    return sel


def lambda_from_stats(ax, aw, mask, alpha=0.5):
    """Per-channel smoothing scale λ (float32 [K])."""
    K = ax.shape[1]
    if mask == 0:
        return np.ones(K, dtype=F32)
    sel = select_absmax(ax, mask)
    aw = np.asarray(aw, dtype=F32)
    ok = (sel != 0) & (aw != 0)
    lam = np.ones(K, dtype=F32)
    alpha = float(F32(alpha))                 # the float32 α, widened exactly
    if alpha == 0.5:
        ratio = (sel[ok] / aw[ok]).astype(F32)
        lam[ok] = np.sqrt(ratio).astype(F32)
    else:
        a64 = sel[ok].astype(np.float64) ** alpha / aw[ok].astype(np.float64) ** (1.0 - alpha)
        lam[ok] = a64.astype(F32)
    return lam


def inv_lambda(lam):
    """1/λ rounded to float32 once per channel."""
    return (F32(1.0) / np.asarray(lam, dtype=F32)).astype(F32)


def act_amax_from_stats(ax, lam):
    """Static activation tensor amax: max_k (ax_all_k * (1/λ_k)) in float32."""
    ax_all = ax.max(axis=0).astype(F32)
    return F32((ax_all * inv_lambda(lam)).astype(F32).max())


def calibrate(X_bits, seg, W_bits, mask, alpha=0.5):
    """The full calibration reduction: (ax [3,K], aw [K], λ [K], act_amax)."""
    ax = channel_absmax_per_modality(X_bits, seg)
    if W_bits is None:
        aw = np.ones(ax.shape[1], dtype=F32)
    else:
        aw = weight_absmax(W_bits)
    lam = lambda_from_stats(ax, aw, mask, alpha)
    return ax, aw, lam, act_amax_from_stats(ax, lam)


def smooth(X_bits, lam):
    """X̂ = X * (1/λ) in float32, [M, K]."""
    return (bf16_bits_to_f32(X_bits) * inv_lambda(lam)[None, :]).astype(F32)
