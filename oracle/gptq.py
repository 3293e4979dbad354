"""GPTQ rounding of the low-rank branch's residual.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph (the residual left by the
16-bit low-rank branch is GPTQ-rounded to int4) and the conversion-cost line (calibration and
GPTQ are the two steps of converting the DiT).  GPTQ itself is the published algorithm of
Frantar, Ashkboos, Hoefler and Alistarh (2022): with H the Hessian of the layer's squared output
error and U the upper Cholesky factor of H⁻¹ (H⁻¹ = UᵀU), the columns are quantised in order;
the error of column k, divided by U_kk, is subtracted from the not yet quantised columns along
row k of U.

Readings where the pages are silent:
  * the residual multiplies the smoothed activation, so H = Σ over calibration rows of x̂·x̂ᵀ
    with x̂ = fl32(x · fl32(1/λ)) (the activation quantiser's input), in float64;
  * damping as published: H_kk += 0.01 · mean_k H_kk; an all-zero H is taken as the identity;
  * natural column order; a group's scale (the quantiser's block: 64 columns for int4, 16 for
    NVFP4, 32 for the MX formats) is fixed when the sweep reaches the group's first column,
    from the current values of the group's columns;
  * the sweep starts from R32, the float32 residual the round-to-nearest path quantises; the
    working values are float64 and each decision quantises fl32 of the current value with the
    round-to-nearest path's own element rule; the NVFP4 tensor scale is that path's,
    g = max|R32| / 2688, fixed before the sweep;
  * codes and scales are stored exactly as the round-to-nearest path stores them.
"""
import numpy as np

from . import calib, quant, mx
from .formats import bf16_bits_to_f32, e2m1_decode, e4m3_decode, pack_nibbles

F32 = np.float32
GROUP = {"int4": 64, "nvfp4": 16, "mxfp4": 32, "mxfp8": 32}
MX_ELEM = {"mxfp4": "e2m1", "mxfp8": "e4m3"}
PERCDAMP = 0.01


def hessian(X_bits, lam):
    """H = X̂ᵀ X̂ over the given rows, float64 [K, K] (lam None: λ = 1, X̂ = X)."""
    if lam is None:
        xhat = bf16_bits_to_f32(X_bits).astype(np.float64)
    else:
        xhat = calib.smooth(X_bits, lam).astype(np.float64)
    return xhat.T @ xhat


def damped(H, percdamp=PERCDAMP):
    """H + percdamp · mean(diag H) · I (the identity when H is all zero)."""
    H = np.array(H, dtype=np.float64)
    d = float(np.mean(np.diag(H)))
    if d == 0.0:
        return np.eye(H.shape[0])
    H[np.diag_indices_from(H)] += percdamp * d
    return H


def _group_scale(x32, fmt, g):
    """Per-row scale of one group from its float32 values [N, G]:
    (stored scale, element quantiser of a float32 column -> (element codes, exact values))."""
    a = np.abs(x32).max(axis=1)
    if fmt == "int4":
        s16 = quant.int4_scale(a)

        def enc(x):
            c = quant.int4_codes(x, s16)
            return c, c.astype(np.float64) * s16.astype(np.float64)
        return s16, enc
    if fmt == "nvfp4":
        s, S = quant.nvfp4_block_scales(a, g)

        def enc(x):
            nib = quant.nvfp4_nibbles(x, S)
            return nib, e2m1_decode(nib) * e4m3_decode(s) * np.float64(F32(g))
        return s.astype(np.uint8), enc
    elem = MX_ELEM[fmt]
    e = mx.mx_exponent(a, elem)

    def enc(x):
        c = mx.mx_element_codes(x, e, elem)
        v = e2m1_decode(c) if elem == "e2m1" else e4m3_decode(c)
        return c, v * np.ldexp(1.0, e)
    return (e + 127).astype(np.uint8), enc


def gptq_quantize(R32, H, fmt, amax=None):
    """GPTQ codes and scales of the residual R32 [N, K] under the Hessian H [K, K] (damped here):
    dict(codes, scales, g (NVFP4) / None, deq (exact float64 values of the codes)).  Rows are
    independent given H, so R32 may be a subset of a residual's rows; amax is then the whole
    residual's max|R32| for the NVFP4 tensor scale (default: this R32's)."""
    W = np.asarray(R32, dtype=F32).astype(np.float64)
    N, K = W.shape
    G = GROUP[fmt]
    if K % G:
        raise ValueError(f"K={K} is not a multiple of the group size {G}")
    if amax is None:
        amax = np.abs(np.asarray(R32, dtype=F32)).max()
    g = quant.nvfp4_tensor_scale(amax) if fmt == "nvfp4" else None
    U = np.linalg.cholesky(np.linalg.inv(damped(H))).T          # H⁻¹ = UᵀU, U upper
    el = np.zeros((N, K), dtype=np.int16)
    deq = np.zeros((N, K))
    scales = []
    enc = None
    for k in range(K):
        if k % G == 0:
            sc, enc = _group_scale(W[:, k:k + G].astype(F32), fmt, g)
            scales.append(sc)
        c, v = enc(W[:, k].astype(F32))
        el[:, k] = c
        deq[:, k] = v
        err = (W[:, k] - v) / U[k, k]
        W[:, k + 1:] -= np.outer(err, U[k, k + 1:])
    scales = np.stack(scales, axis=1)
    if fmt == "mxfp8":
        codes = el.astype(np.uint8)
    else:
        codes = pack_nibbles((el.astype(np.int64) & 0xF).astype(np.uint8))
    return dict(codes=codes, scales=scales, g=g, deq=deq)


def output_error(R32, deq, H):
    """tr((R − Q) H (R − Q)ᵀ): the squared output error of the rounding over the calibration
    rows H was accumulated from."""
    D = np.asarray(R32, dtype=F32).astype(np.float64) - deq
    return float(np.einsum("nk,kj,nj->", D, H, D))
