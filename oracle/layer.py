"""The oracle's steps of the W4A4 layer put together in the order the layer runs them.

TEST INFRASTRUCTURE ONLY (see the package docstring).

    calibrate (ax, aw, λ, act_amax)  ->  weight prep (R32 = W' − L1L2, quantised with its own
    dynamic tensor amax max|R32|)  ->  activation prep (X̂ = X/λ quantised with the static
    act_amax for NVFP4, or per 64-group for int4, or per 32-block for the MX formats (mxfp4,
    mxfp8: no tensor scale); D = bf16(X̂)·L1 unrounded)  ->  GEMM.
"""
import numpy as np

from . import calib, svd, quant, gemm, mx

MX_ELEM = {"mxfp4": "e2m1", "mxfp8": "e4m3"}

F32 = np.float32


def prepare_weight(W_bits, lam, lora_down_bits, lora_up_bits, fmt):
    """Quantised residual weight: dict(codes, scales, g (NVFP4 only), R32)."""
    R32 = svd.residual_f32(W_bits, lam, lora_down_bits, lora_up_bits)
    if fmt in MX_ELEM:
        codes, scales = mx.mx_quantize(R32, MX_ELEM[fmt])
        return dict(codes=codes, scales=scales, g=None, R32=R32)
    if fmt == "int4":
        codes, scales = quant.int4_quantize(R32)
        return dict(codes=codes, scales=scales, g=None, R32=R32)
    amax = F32(np.abs(R32).max())
    codes, scales, g, _ = quant.nvfp4_quantize(R32, amax)
    return dict(codes=codes, scales=scales, g=g, R32=R32)


def prepare_activation(X_bits, lam, act_amax, lora_down_bits, fmt):
    """Quantised activation: dict(codes, scales, g (NVFP4), n_sat (NVFP4), D float64, xhat)."""
    xhat = calib.smooth(X_bits, lam)
    D = gemm.lowrank_down(xhat, lora_down_bits)
    if fmt in MX_ELEM:
        codes, scales = mx.mx_quantize(xhat, MX_ELEM[fmt])
        return dict(codes=codes, scales=scales, g=None, n_sat=0, D=D, xhat=xhat)
    if fmt == "int4":
        codes, scales = quant.int4_quantize(xhat)
        return dict(codes=codes, scales=scales, g=None, n_sat=0, D=D, xhat=xhat)
    codes, scales, g, n_sat = quant.nvfp4_quantize(xhat, act_amax)
    return dict(codes=codes, scales=scales, g=g, n_sat=n_sat, D=D, xhat=xhat)


def forward(act, wt, lora_up_bits, fmt, rows=None):
    """Layer output (Y64, Y bits) from prepared activation / weight; optionally only `rows`."""
    sel = slice(None) if rows is None else rows
    if fmt in MX_ELEM:
        return gemm.linear_mx(act["codes"][sel], act["scales"][sel], wt["codes"], wt["scales"],
                              act["D"][sel], lora_up_bits, MX_ELEM[fmt])
    if fmt == "int4":
        return gemm.linear_int4(act["codes"][sel], act["scales"][sel], wt["codes"], wt["scales"],
                                act["D"][sel], lora_up_bits)
    return gemm.linear_nvfp4(act["codes"][sel], act["scales"][sel], act["g"], wt["codes"],
                             wt["scales"], wt["g"], act["D"][sel], lora_up_bits)
