"""Allocating helpers over the C ABI for the W4A4 layer (torch provides memory and streams).

Every numeric step runs in libsvdq.so; these functions only allocate outputs and call the
entry points in order: calibration -> weight preparation -> activation quantisation with the
low-rank down-projection -> W4A4 GEMM.
"""
from dataclasses import dataclass

from . import _lib
from ._lib import NVFP4, INT4_G64, MXFP4, MXFP8  # noqa: F401


def _torch():
    import torch
    return torch


@dataclass
class PreparedWeight:
    fmt: int
    N: int
    K: int
    r: int
    codes: object        # uint8 [N, K/2] (MXFP8: [N, K])
    scales: object       # uint8 [N, K/16] (E4M3), float16 [N, K/64] or uint8 [N, K/32] (E8M0)
    g: object            # float32 [1] (NVFP4) or None
    lora_up: object      # bf16 [N, r] or None


def _alloc_codes_scales(fmt, rows, K, dev):
    """Code and scale tensors of one format; the NVFP4 tensor scale (else None)."""
    torch = _torch()
    codes = torch.empty(rows, K if fmt == MXFP8 else K // 2, dtype=torch.uint8, device=dev)
    g = None
    if fmt == NVFP4:
        scales = torch.empty(rows, K // 16, dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
    elif fmt == INT4_G64:
        scales = torch.empty(rows, K // 64, dtype=torch.float16, device=dev)
    else:
        scales = torch.empty(rows, K // 32, dtype=torch.uint8, device=dev)
    return codes, scales, g


def calibrate(X, seg, W=None, mask=7, alpha=0.5, state=None):
    """λ calibration on X [M, K]; pass the previous result as `state` to accumulate batches."""
    torch = _torch()
    K = X.shape[1]
    dev = X.device
    if state is None:
        state = dict(ax=torch.empty(3, K, device=dev), aw=torch.empty(K, device=dev),
                     **{"lambda": torch.empty(K, device=dev)},
                     act_amax=torch.empty(1, device=dev))
        acc = 0
    else:
        acc = 1
    _lib.svdq_calibrate_lambda(X, seg, W, mask, alpha, acc, state["ax"], state["aw"],
                               state["lambda"], state["act_amax"])
    return state


def bits_lost(ax, lam=None, block=16):
    """Bits-lost proxy per modality (float64 [3]) of the smoothing λ for per-modality channel
    maxima ax [3, K] (the `ax` of a calibration state); block = the quantiser's group size."""
    torch = _torch()
    out = torch.empty(3, dtype=torch.float64, device=ax.device)
    _lib.svdq_bits_lost(ax, lam, block, out)
    return out


def lowrank_factors(W, lam, omega, r, power_iters=2):
    """Randomized rank-r factors of diag(λ)·Wᵀ on the GPU: (lora_down [r, K], lora_up [N, r],
    sigma [r]).  omega [N, ell] fp32 is the caller's random matrix (ell >= r)."""
    torch = _torch()
    N, K = W.shape
    ell = omega.shape[1]
    dev = W.device
    down = torch.empty(r, K, dtype=torch.bfloat16, device=dev)
    up = torch.empty(N, r, dtype=torch.bfloat16, device=dev)
    sigma = torch.empty(r, dtype=torch.float32, device=dev)
    nbytes = _lib.svdq_lowrank_workspace_bytes(N, K, ell)
    if nbytes < 0:
        raise ValueError(f"unsupported sketch width {ell}")
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    off = (-ws.data_ptr()) % 256
    _lib.svdq_lowrank_factors(W, lam, omega, r, power_iters, down, up, sigma,
                              ws[off:off + nbytes])
    return down, up, sigma


# The 39 migration strengths α = i/40 of the λ grid (λ_k = a_k^α / w_k^(1−α)).
ALPHA_GRID = tuple(i / 40.0 for i in range(1, 40))


def lambda_search(X, W, state, alphas, rows, fmt=NVFP4, omega=None, r=32, power_iters=2,
                  mask=7, refit_iters=0, per_iterate=False):
    """λ grid search on the GPU: for each α the layer's output error on the sampled rows
    (device int32 indices into X), the smallest over refit_iters refits of the low-rank branch.
    Returns dict(scores fp64 [n_alpha], lam (the winner's λ), index, and when r > 0 the
    winner's best factors lora_down [r, K] / lora_up [N, r]; with per_iterate the score of
    every iterate, fp64 [n_alpha, refit_iters + 1])."""
    torch = _torch()
    N, K = W.shape
    dev = X.device
    ell = omega.shape[1] if omega is not None else 0
    n = len(alphas)
    out = dict(scores=torch.empty(n, dtype=torch.float64, device=dev),
               lam=torch.empty(K, dtype=torch.float32, device=dev),
               index=torch.empty(1, dtype=torch.int32, device=dev))
    if per_iterate:
        out["iter_scores"] = torch.empty(n, refit_iters + 1, dtype=torch.float64, device=dev)
    if r > 0:
        out["lora_down"] = torch.empty(r, K, dtype=torch.bfloat16, device=dev)
        out["lora_up"] = torch.empty(N, r, dtype=torch.bfloat16, device=dev)
    nbytes = _lib.svdq_lambda_search_workspace_bytes(fmt, N, K, ell, r, rows.numel(), n,
                                                     refit_iters)
    if nbytes < 0:
        raise ValueError("unsupported search shape")
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    off = (-ws.data_ptr()) % 256
    _lib.svdq_lambda_search(X, W, state["ax"], state["aw"], mask, alphas, fmt, omega, r,
                            power_iters, refit_iters, rows, out["scores"], out.get("iter_scores"),
                            out["lam"], out["index"], out.get("lora_down"), out.get("lora_up"),
                            ws[off:off + nbytes])
    return out


def prepare_weight(W, lam, lora_down, lora_up, fmt=NVFP4, workspace=None):
    """Quantised residual of diag(λ)·W − L1·L2 (W [N, K] bf16).  With `workspace` (uint8, at
    least quantize_weight_workspace_bytes, 256-byte aligned) the NVFP4 residual is formed once."""
    torch = _torch()
    N, K = W.shape
    r = 0 if lora_down is None else lora_down.shape[0]
    codes, scales, g = _alloc_codes_scales(fmt, N, K, W.device)
    if workspace is None:
        _lib.svdq_quantize_weight(fmt, W, lam, lora_down, lora_up, r, codes, scales, g)
    else:
        _lib.svdq_quantize_weight_ws(fmt, W, lam, lora_down, lora_up, r, codes, scales, g,
                                     workspace)
    return PreparedWeight(fmt, N, K, r, codes, scales, g, lora_up)


def quantize_weight_workspace(N, K, fmt=NVFP4, device="cuda"):
    """A 256-byte aligned workspace for prepare_weight(..., workspace=...)."""
    torch = _torch()
    nb = _lib.svdq_quantize_weight_workspace_bytes(fmt, N, K)
    buf = torch.empty(nb + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nb]


def gptq_hessian(X, lam, H=None):
    """H [K, K] fp64 (+)= X̂ᵀX̂ of the calibration rows X; pass H back to accumulate batches."""
    torch = _torch()
    K = X.shape[1]
    if H is None:
        H = torch.empty(K, K, dtype=torch.float64, device=X.device)
        _lib.svdq_gptq_hessian(X, lam, H, accumulate=False)
    else:
        _lib.svdq_gptq_hessian(X, lam, H, accumulate=True)
    return H


def prepare_weight_gptq(W, lam, lora_down, lora_up, H, fmt=NVFP4):
    """prepare_weight with the residual GPTQ-rounded under the Hessian H."""
    torch = _torch()
    N, K = W.shape
    r = 0 if lora_down is None else lora_down.shape[0]
    codes, scales, g = _alloc_codes_scales(fmt, N, K, W.device)
    nbytes = _lib.svdq_gptq_workspace_bytes(N, K)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=W.device)
    off = (-ws.data_ptr()) % 256
    _lib.svdq_gptq_quantize_weight(fmt, W, lam, lora_down, lora_up, r, H, codes, scales, g,
                                   ws[off:off + nbytes])
    return PreparedWeight(fmt, N, K, r, codes, scales, g, lora_up)


def quantize_activation(X, lam, act_amax, lora_down, fmt=NVFP4, sat_count=None):
    """(codes, scales, g_a, D) of X [M, K]."""
    torch = _torch()
    M, K = X.shape
    r = 0 if lora_down is None else lora_down.shape[0]
    dev = X.device
    codes, scales, g = _alloc_codes_scales(fmt, M, K, dev)
    D = torch.empty(M, r, dtype=torch.float32, device=dev) if r else None
    _lib.svdq_quant_act_lowrank_down(fmt, X, lam, act_amax, lora_down, r, codes, scales, g, D,
                                     sat_count)
    return codes, scales, g, D


def cube_geometry(T, H, W, ct, ch, cw, n_text, n_audio, cube1d, device="cuda"):
    """DeltaQuant geometry on the host, uploaded: dict(row_to_cube, cube_ptr, cube_rows,
    group_ptr (device int32), n_cubes, host (the numpy arrays))."""
    import numpy as np
    torch = _torch()
    r2c, ptr, rows = _lib.svdq_cube_geometry(T, H, W, ct, ch, cw, n_text, n_audio, cube1d)
    gp = _lib.svdq_cube_groups(ptr)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
    return dict(row_to_cube=up(r2c), cube_ptr=up(ptr), cube_rows=up(rows), group_ptr=up(gp),
                n_cubes=len(ptr) - 1, host=dict(row_to_cube=r2c, cube_ptr=ptr, cube_rows=rows,
                                                group_ptr=gp))


def delta_quantize_activation(X, lam, act_amax, geo, lora_down, out=None, sat_count=None):
    """DeltaQuant activations of X [M, K] for the cube geometry `geo` (cube_geometry, or a dict
    with device cube_ptr / cube_rows / group_ptr and n_cubes): dict with core codes cc
    [n_cubes, K], core scales cs [n_cubes], delta codes dc [M, K/2] and scales dsc [M, K/16],
    g_delta gd [1], D [M, r] (fp32) and the fp32 core workspace ws.  Pass `out` to reuse its
    tensors."""
    torch = _torch()
    M, K = X.shape
    r = 0 if lora_down is None else lora_down.shape[0]
    dev = X.device
    u8 = torch.uint8
    nc = geo["n_cubes"]
    if out is None:
        nbytes = _lib.svdq_delta_workspace_bytes(nc, K)
        ws = torch.empty(nbytes + 256, dtype=u8, device=dev)
        off = (-ws.data_ptr()) % 256
        out = dict(cc=torch.empty(nc, K, dtype=u8, device=dev),
                   cs=torch.empty(nc, device=dev),
                   dc=torch.empty(M, K // 2, dtype=u8, device=dev),
                   dsc=torch.empty(M, K // 16, dtype=u8, device=dev),
                   gd=torch.empty(1, device=dev),
                   D=torch.empty(M, r, device=dev) if r else None,
                   ws=ws[off:off + nbytes])
    _lib.svdq_delta_quant_act(X, lam, act_amax, geo["cube_ptr"], geo["cube_rows"], nc,
                              geo["group_ptr"], lora_down, r, out["cc"], out["cs"], out["dc"],
                              out["dsc"], out["gd"], out.get("D"), sat_count, out["ws"])
    return out


def gemm(codes, scales, g_a, D, pw, M, out=None, core_out=None, row_to_cube=None):
    torch = _torch()
    Y = out if out is not None else torch.empty(M, pw.N, dtype=torch.bfloat16, device=codes.device)
    _lib.svdq_w4a4_gemm(pw.fmt, M, pw.N, pw.K, codes, scales, g_a, pw.codes, pw.scales, pw.g, D,
                        pw.lora_up, pw.r, Y, core_out, row_to_cube)
    return Y


def forward(X, pw, act_amax, lam, lora_down, out=None):
    """Y = X̂·L1·L2 + Q(X̂)·Q(R) for X [..., K]; leading dimensions are flattened exactly once."""
    lead = X.shape[:-1]
    X2 = X.reshape(-1, X.shape[-1])
    codes, scales, g, D = quantize_activation(X2, lam, act_amax, lora_down, pw.fmt)
    Y = gemm(codes, scales, g, D, pw, X2.shape[0], out=out)
    return Y.reshape(*lead, pw.N)
