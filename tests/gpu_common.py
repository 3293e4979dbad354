"""Shared helpers of the GPU parity tests: device transfer of bf16 bit patterns, the oracle
side of a layer case, and the comparison rules (bit-exact codes; bf16 outputs within
rel-L2 <= 1e-3 and |Δ| <= 2^-7·|y| + 1e-3·rms(y) of the oracle's bf16 output; the fp32
low-rank intermediate D within 2^-16·|d| + 1e-5·rms(D) of the float64 product)."""
import numpy as np

from oracle import calib as OC, svd as OS, quant as OQ, gemm as OG, layer as OL
from oracle.formats import bf16_bits_to_f32

Y_REL_L2 = 1e-3
Y_ELEM_REL = 2.0 ** -7
Y_ELEM_RMS = 1e-3
D_ELEM_RMS = 1e-5
D_ELEM_REL = 2.0 ** -16


def torch_mod():
    import torch
    return torch


def dev_bf16(bits):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t):
    torch = torch_mod()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_y(y_gpu_bits, y_ref_bits, what="Y"):
    g = bf16_bits_to_f32(y_gpu_bits).astype(np.float64)
    y = bf16_bits_to_f32(y_ref_bits).astype(np.float64)
    rms = np.sqrt(np.mean(y * y))
    rel = np.linalg.norm(g - y) / np.linalg.norm(y)
    bad = np.abs(g - y) > Y_ELEM_REL * np.abs(y) + Y_ELEM_RMS * rms
    assert rel <= Y_REL_L2, f"{what}: rel-L2 {rel:.3e} > {Y_REL_L2}"
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance, worst "
                           f"{np.abs(g - y)[bad].max():.3e} (rms {rms:.3e})")
    return rel


def check_d(d_gpu, d_ref):
    """D (fp32 accumulation of exact bf16 products) against the float64 product."""
    g = np.asarray(d_gpu, dtype=np.float64)
    d = np.asarray(d_ref, dtype=np.float64)
    if d.size == 0:
        return
    rms = np.sqrt(np.mean(d * d))
    bad = np.abs(g - d) > D_ELEM_REL * np.abs(d) + D_ELEM_RMS * rms
    assert not bad.any(), f"D: {bad.sum()} elements out of tolerance, worst {np.abs(g - d).max():.3e}"


def oracle_case(X, seg, W, mask, r, fmt, alpha=0.5, factors=None, rows=None):
    """Everything the oracle computes for one layer case (rows: optional row sample for the
    activation-side outputs)."""
    ax, aw, lam, amax = OC.calibrate(X, seg, W, mask, alpha)
    if factors is None:
        down, up = OS.lowrank_factors(W, lam, r)
    else:
        down, up = factors
    wt = OL.prepare_weight(W, lam, down, up, fmt)
    Xs = X if rows is None else X[rows]
    act = OL.prepare_activation(Xs, lam, amax, down, fmt)
    y64, y = OL.forward(act, wt, up, fmt)
    return dict(ax=ax, aw=aw, lam=lam, amax=amax, down=down, up=up, wt=wt, act=act, y=y)
