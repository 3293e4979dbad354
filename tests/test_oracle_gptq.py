"""Pins of the oracle's GPTQ rounding ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)",
opening paragraph; GPTQ as published by Frantar et al. 2022) against facts that fix it: with a
diagonal Hessian no column can compensate another, so GPTQ is round-to-nearest; two coupled
columns have the closed-form update w1 += (w0 − q0)·H01/H11; the rounding lowers the output
error it minimises on correlated activations; a scaled Hessian changes nothing (the damping is
relative); the Hessian is the sum of the rows' outer products."""
import numpy as np
import pytest

import synth
from oracle import gptq as OG, quant as OQ, mx as OM, calib as OC, svd as OS
from oracle.formats import bf16_rne, bf16_bits_to_f32

F32 = np.float32
FMTS = ["int4", "nvfp4", "mxfp4", "mxfp8"]


def _rtn(R32, fmt):
    if fmt == "int4":
        c, s = OQ.int4_quantize(R32)
        return c, s
    if fmt == "nvfp4":
        c, s, _, _ = OQ.nvfp4_quantize(R32, np.abs(R32).max())
        return c, s
    return OM.mx_quantize(R32, OG.MX_ELEM[fmt])


def _residual(N, K, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, K)) * np.exp(rng.normal(0, 0.5, K))[None, :]).astype(F32)


@pytest.mark.parametrize("fmt", FMTS)
def test_diagonal_hessian_is_round_to_nearest(fmt):
    R = _residual(24, 128)
    H = np.diag(np.random.default_rng(1).uniform(0.5, 3.0, 128))
    out = OG.gptq_quantize(R, H, fmt)
    c, s = _rtn(R, fmt)
    assert np.array_equal(out["codes"], c)
    assert np.array_equal(np.asarray(out["scales"]).view(np.uint8), np.asarray(s).view(np.uint8))


@pytest.mark.parametrize("fmt", FMTS)
def test_two_coupled_columns_follow_the_closed_form(fmt):
    K = 64
    R = _residual(40, K, seed=2)
    H = np.eye(K)
    H[0, 1] = H[1, 0] = 0.9
    out = OG.gptq_quantize(R, H, fmt)
    Hd = OG.damped(H)
    # column 0 and every uncoupled column round to nearest; column 1 takes w1 + (w0 − q0)·b/c
    # under the scale its group fixed at column 0
    ref = OG.gptq_quantize(R, np.diag(np.diag(H)), fmt)
    w1 = R[:, 1].astype(np.float64) + (R[:, 0] - ref["deq"][:, 0]) * Hd[0, 1] / Hd[1, 1]
    R1 = R.copy()
    R1[:, 1] = w1.astype(F32)
    G = OG.GROUP[fmt]
    # quantise with the group scale of the ORIGINAL group values: rebuild it from R
    sc, enc = OG._group_scale(R[:, :G], fmt, OQ.nvfp4_tensor_scale(np.abs(R).max()))
    c1, v1 = enc(w1.astype(F32))
    assert np.array_equal(out["deq"][:, 1], v1)
    keep = np.ones(K, bool)
    keep[1] = False
    assert np.array_equal(out["deq"][:, keep], ref["deq"][:, keep])
    assert not np.array_equal(out["deq"][:, 1], ref["deq"][:, 1])     # the update mattered


@pytest.mark.parametrize("fmt", FMTS)
def test_gptq_lowers_the_output_error_on_outlier_activations(fmt):
    cfg = synth.config(0)
    X = synth.gen.x_bits(cfg)
    W = synth.gen.weight_bits(cfg["N"], cfg["K"])
    _, _, lam, _ = OC.calibrate(X, cfg["seg"], W, 7)
    down, up = OS.lowrank_factors(W, lam, 8)
    R32 = OS.residual_f32(W, lam, down, up)
    H = OG.hessian(X, lam)
    out = OG.gptq_quantize(R32, H, fmt)
    c, s = _rtn(R32, fmt)
    g = OQ.nvfp4_tensor_scale(np.abs(R32).max())
    if fmt == "int4":
        rtn = OQ.int4_dequantize(c, s)
    elif fmt == "nvfp4":
        rtn = OQ.nvfp4_dequantize(c, s, g)
    else:
        rtn = OM.mx_dequantize(c, s, OG.MX_ELEM[fmt])
    e_g, e_r = OG.output_error(R32, out["deq"], H), OG.output_error(R32, rtn, H)
    assert e_g < 0.9 * e_r, (fmt, e_g, e_r)


def test_scaled_hessian_changes_nothing():
    R = _residual(16, 128, seed=3)
    X = np.random.default_rng(4).standard_normal((300, 128))
    H = X.T @ X
    a = OG.gptq_quantize(R, H, "int4")
    b = OG.gptq_quantize(R, 4.0 * H, "int4")
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


def test_hessian_is_the_sum_of_row_outer_products():
    rng = np.random.default_rng(5)
    X = bf16_rne(rng.standard_normal((7, 32)))
    lam = rng.uniform(0.5, 2.0, 32).astype(F32)
    H = OG.hessian(X, lam)
    inv = (F32(1) / lam).astype(F32)
    ref = np.zeros((32, 32))
    for m in range(7):
        x = (bf16_bits_to_f32(X[m]) * inv).astype(F32).astype(np.float64)
        for i in range(32):
            for j in range(32):
                ref[i, j] += x[i] * x[j]
    assert np.allclose(H, ref, rtol=1e-15, atol=0)
    assert np.array_equal(OG.damped(np.zeros((4, 4))), np.eye(4))
