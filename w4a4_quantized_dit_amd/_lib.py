"""ctypes binding of libsvdq.so: argument marshalling only.

Every function below has the name of the C entry point it calls and takes torch tensors (device
memory owned by the caller) plus sizes; it checks dtypes / devices / shapes, passes raw pointers
and the current torch stream, and raises SvdqError on a non-zero status.  No step of the layer
runs in Python: when the library is missing, loading fails loudly.
"""
import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsvdq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "svdq.h")

NVFP4, INT4_G64, MXFP4, MXFP8 = 0, 1, 2, 3

_c_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_SIGS = {
    "svdq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "svdq_last_error": (ctypes.c_char_p, []),
    "svdq_abi_version": (ctypes.c_int, []),
    "svdq_calibrate_lambda": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, _c_p, _i64, _i64,
                                             ctypes.c_uint32, ctypes.c_float, ctypes.c_int,
                                             _c_p, _c_p, _c_p, _c_p, _c_p]),
    "svdq_bits_lost": (ctypes.c_int, [_c_p, _c_p, _i64, _i64, _c_p, _c_p]),
    "svdq_lowrank_workspace_bytes": (_i64, [_i64, _i64, _i64]),
    "svdq_gptq_hessian": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, ctypes.c_int, _c_p,
                                         _c_p]),
    "svdq_gptq_workspace_bytes": (_i64, [_i64, _i64]),
    "svdq_gptq_quantize_weight": (ctypes.c_int, [ctypes.c_int, _c_p, _i64, _i64, _i64, _c_p, _c_p,
                                                 _c_p, _i64, _c_p, _c_p, _c_p, _c_p, _c_p, _i64,
                                                 _c_p]),
    "svdq_lambda_search_workspace_bytes": (_i64, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                                  _i64, ctypes.c_int]),
    "svdq_lambda_search": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, _i64, _i64, _c_p, _c_p,
                                          ctypes.c_uint32, _c_p, _i64, ctypes.c_int, _c_p, _i64,
                                          _i64, ctypes.c_int, ctypes.c_int, _c_p, _i64, _c_p, _c_p,
                                          _c_p, _c_p, _c_p, _c_p, _c_p, _i64, _c_p]),
    "svdq_lowrank_factors": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, _c_p, _i64, _i64,
                                            ctypes.c_int, _c_p, _c_p, _c_p, _c_p, _i64, _c_p]),
    "svdq_quantize_weight": (ctypes.c_int, [ctypes.c_int, _c_p, _i64, _i64, _i64, _c_p, _c_p,
                                            _c_p, _i64, _c_p, _c_p, _c_p, _c_p]),
    "svdq_quantize_weight_workspace_bytes": (_i64, [ctypes.c_int, _i64, _i64]),
    "svdq_quantize_weight_ws": (ctypes.c_int, [ctypes.c_int, _c_p, _i64, _i64, _i64, _c_p, _c_p,
                                               _c_p, _i64, _c_p, _c_p, _c_p, _c_p, _i64, _c_p]),
    "svdq_quant_act_lowrank_down": (ctypes.c_int, [ctypes.c_int, _c_p, _i64, _i64, _i64, _c_p,
                                                   _c_p, _c_p, _i64, _c_p, _c_p, _c_p, _c_p,
                                                   _c_p, _c_p]),
    "svdq_w4a4_gemm": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _c_p, _c_p, _c_p, _c_p,
                                      _c_p, _c_p, _c_p, _c_p, _i64, _c_p, _c_p, _c_p, _i64,
                                      _c_p]),
    "svdq_cube_geometry": (ctypes.c_int, [_i64] * 9 + [_c_p, _c_p, _c_p, _c_p]),
    "svdq_cube_divisor_aligned": (ctypes.c_int, [_i64] * 6 + [_c_p]),
    "svdq_cube_schedule": (ctypes.c_int, [_c_p, _i64, _i64, _c_p]),
    "svdq_cube_groups": (ctypes.c_int, [_c_p, _i64, _c_p, _c_p]),
    "svdq_delta_workspace_bytes": (_i64, [_i64, _i64]),
    "svdq_delta_quant_act": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, _c_p, _c_p, _c_p,
                                            _i64, _c_p, _i64, _c_p, _i64, _c_p, _c_p, _c_p,
                                            _c_p, _c_p, _c_p, _c_p, _c_p, _i64, _c_p]),
    "svdq_delta_quant_act_noalloc": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, _c_p, _c_p,
                                                    _c_p, _i64, _c_p, _i64, _c_p, _i64, _c_p,
                                                    _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "svdq_gemm_core": (ctypes.c_int, [_i64, _i64, _i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                      _c_p]),
    "svdq_score_modal_rel_l2": (ctypes.c_int, [_c_p, _i64, _c_p, _i64, _c_p, _i64, _i64, _i64,
                                               _i64, _c_p, _c_p, _i64, _c_p, _c_p]),
    "svdq_score_reference_rows": (ctypes.c_int, [_c_p, _i64, _c_p, _i64, _i64, _i64, _i64, _c_p,
                                                 _i64, _c_p, _i64, _c_p]),
    "svdq_score_modal_rel_l2_ref": (ctypes.c_int, [_c_p, _i64, _c_p, _i64, _i64, _i64, _c_p, _c_p,
                                                   _i64, _c_p, _c_p]),
}

_lib = None


class SvdqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} ({status_string(status)})")
        self.status = status


def load():
    """Load libsvdq.so (built in-tree by w4a4_quantized_dit_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m w4a4_quantized_dit_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_entry_points():
    """Names of the functions declared in include/svdq.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(svdq_\w+)\s*\(", text, re.M)))


def status_string(status):
    return load().svdq_status_string(status).decode()


def last_error():
    return load().svdq_last_error().decode()


def _check(status):
    if status != 0:
        raise SvdqError(status, last_error())


# ------------------------------------------------------------------------------------------
# tensor marshalling
# ------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, name="tensor", numel=None, rows=False):
    """Device pointer of a cuda tensor (None -> NULL).  The tensor must be contiguous, or with
    rows=True a 2-D view whose rows are contiguous (stride(1) == 1): its row stride is then
    passed as the matrix's leading dimension, which the library validates."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if rows:
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError(f"{name} must be a 2-D matrix with contiguous rows")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _ld(t):
    """Leading dimension (row stride, elements) of a matrix passed with rows=True."""
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _bf16():
    torch = _torch()
    return (torch.bfloat16, torch.int16)


def _scale_dtype(fmt):
    torch = _torch()
    return torch.float16 if fmt == INT4_G64 else torch.uint8


def _block(fmt):
    """Elements per scale along K."""
    return {NVFP4: 16, INT4_G64: 64, MXFP4: 32, MXFP8: 32}[int(fmt)]


def _code_bytes(fmt, rows, K):
    """Bytes of codes for rows x K elements (MXFP8: one per element, else two per byte)."""
    return rows * K if int(fmt) == MXFP8 else rows * K // 2


# ------------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------------

def svdq_calibrate_lambda(X, seg, W, modality_mask, alpha, accumulate, ax, aw, lam, act_amax,
                          stream=None):
    """λ calibration reduction; X [M, K] bf16, seg 4 ints, W [N, K] bf16 or None; outputs fp32."""
    torch = _torch()
    M, K = X.shape
    N = W.shape[0] if W is not None else 0
    seg_arr = (ctypes.c_int64 * 4)(*[int(v) for v in seg])
    f32 = torch.float32
    _check(load().svdq_calibrate_lambda(
        _ptr(X, _bf16(), "X", rows=True), M, K, _ld(X), ctypes.cast(seg_arr, _c_p),
        _ptr(W, _bf16(), "W", rows=True), N, _ld(W) if W is not None else K,
        int(modality_mask), float(alpha), int(accumulate),
        _ptr(ax, f32, "ax", 3 * K), _ptr(aw, f32, "aw", K), _ptr(lam, f32, "lambda", K),
        _ptr(act_amax, f32, "act_amax", 1), _stream(stream)))


def svdq_bits_lost(ax, lam, block, out, stream=None):
    """Bits-lost proxy per modality; ax [3, K] fp32, lam [K] fp32 or None; out [3] fp64."""
    torch = _torch()
    K = ax.shape[1]
    _check(load().svdq_bits_lost(
        _ptr(ax, torch.float32, "ax", 3 * K), _ptr(lam, torch.float32, "lambda", K), K,
        int(block), _ptr(out, torch.float64, "out", 3), _stream(stream)))


def svdq_lowrank_workspace_bytes(N, K, ell):
    return int(load().svdq_lowrank_workspace_bytes(int(N), int(K), int(ell)))


def svdq_lowrank_factors(W, lam, omega, r, power_iters, lora_down, lora_up, sigma, workspace,
                         stream=None):
    """Randomized rank-r factors of diag(λ)·Wᵀ; W [N, K] bf16, omega [N, ell] fp32; outputs
    lora_down [r, K] bf16, lora_up [N, r] bf16, sigma [r] fp32 or None; workspace uint8."""
    torch = _torch()
    N, K = W.shape
    ell = omega.shape[1]
    _check(load().svdq_lowrank_factors(
        _ptr(W, _bf16(), "W", rows=True), N, K, _ld(W), _ptr(lam, torch.float32, "lambda", K),
        _ptr(omega, torch.float32, "omega", N * ell), ell, int(r), int(power_iters),
        _ptr(lora_down, _bf16(), "lora_down", r * K), _ptr(lora_up, _bf16(), "lora_up", N * r),
        _ptr(sigma, torch.float32, "sigma", r), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream)))


def svdq_gptq_hessian(X, lam, H, accumulate=False, stream=None):
    torch = _torch()
    M, K = X.shape
    _check(load().svdq_gptq_hessian(
        _ptr(X, _bf16(), "X", rows=True), M, K, _ld(X),
        _ptr(lam, torch.float32, "lambda", K) if lam is not None else None, int(bool(accumulate)),
        _ptr(H, torch.float64, "H", K * K), _stream(stream)))


def svdq_gptq_workspace_bytes(N, K):
    return int(load().svdq_gptq_workspace_bytes(int(N), int(K)))


def svdq_gptq_quantize_weight(fmt, W, lam, lora_down, lora_up, r, H, codes, scales, tensor_scale,
                              workspace, stream=None):
    torch = _torch()
    N, K = W.shape
    _check(load().svdq_gptq_quantize_weight(
        int(fmt), _ptr(W, _bf16(), "W", rows=True), N, K, _ld(W),
        _ptr(lam, torch.float32, "lambda", K) if lam is not None else None,
        _ptr(lora_down, _bf16(), "lora_down", r * K) if r else None,
        _ptr(lora_up, _bf16(), "lora_up", N * r) if r else None, int(r),
        _ptr(H, torch.float64, "H", K * K),
        _ptr(codes, torch.uint8, "codes", _code_bytes(fmt, N, K)),
        _ptr(scales, _scale_dtype(fmt), "scales", N * K // _block(fmt)),
        _ptr(tensor_scale, torch.float32, "tensor_scale", 1) if tensor_scale is not None else None,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def svdq_lambda_search_workspace_bytes(fmt, N, K, ell, r, n_rows, n_alpha, refit_iters=0):
    return int(load().svdq_lambda_search_workspace_bytes(int(fmt), int(N), int(K), int(ell),
                                                         int(r), int(n_rows), int(n_alpha),
                                                         int(refit_iters)))


def svdq_lambda_search(X, W, ax, aw, mask, alphas, fmt, omega, r, power_iters, refit_iters, rows,
                       scores, iter_scores, best_lambda, best_index, best_down, best_up,
                       workspace, stream=None):
    """λ grid search (alphas: host floats) scored by the output error on the sampled rows."""
    torch = _torch()
    M, K = X.shape
    N = W.shape[0]
    ell = omega.shape[1] if omega is not None else 0
    n = len(alphas)
    arr = (ctypes.c_float * n)(*[float(a) for a in alphas])
    _check(load().svdq_lambda_search(
        _ptr(X, _bf16(), "X", rows=True), M, K, _ld(X), _ptr(W, _bf16(), "W", rows=True), N, _ld(W),
        _ptr(ax, torch.float32, "ax", 3 * K), _ptr(aw, torch.float32, "aw", K), int(mask),
        ctypes.cast(arr, _c_p), n, int(fmt),
        _ptr(omega, torch.float32, "omega", N * ell) if omega is not None else None, ell, int(r),
        int(power_iters), int(refit_iters), _ptr(rows, torch.int32, "rows"), rows.numel(),
        _ptr(scores, torch.float64, "scores", n),
        _ptr(iter_scores, torch.float64, "iter_scores", n * (refit_iters + 1))
        if iter_scores is not None else None,
        _ptr(best_lambda, torch.float32, "best_lambda", K),
        _ptr(best_index, torch.int32, "best_index", 1),
        _ptr(best_down, _bf16(), "best_down", r * K) if best_down is not None else None,
        _ptr(best_up, _bf16(), "best_up", N * r) if best_up is not None else None,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def svdq_quantize_weight_workspace_bytes(fmt, N, K):
    return int(load().svdq_quantize_weight_workspace_bytes(int(fmt), int(N), int(K)))


def svdq_quantize_weight_ws(fmt, W, lam, lora_down, lora_up, r, codes, scales, tensor_scale,
                            workspace, stream=None):
    """svdq_quantize_weight with the caller's workspace (uint8, 256-byte aligned; the NVFP4
    residual is formed once and kept there)."""
    torch = _torch()
    N, K = W.shape
    blk = _block(fmt)
    _check(load().svdq_quantize_weight_ws(
        int(fmt), _ptr(W, _bf16(), "W", rows=True), N, K, _ld(W), _ptr(lam, torch.float32, "lambda", K),
        _ptr(lora_down if r else None, _bf16(), "lora_down", r * K),
        _ptr(lora_up if r else None, _bf16(), "lora_up", N * r), int(r),
        _ptr(codes, torch.uint8, "codes", _code_bytes(fmt, N, K)),
        _ptr(scales, _scale_dtype(fmt), "scales", N * K // blk),
        _ptr(tensor_scale, torch.float32, "tensor_scale", 1),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def svdq_quantize_weight(fmt, W, lam, lora_down, lora_up, r, codes, scales, tensor_scale,
                         stream=None):
    """Residual weight quantisation; W [N, K] bf16; outputs codes [N, K/2] u8, scales, g_w."""
    torch = _torch()
    N, K = W.shape
    blk = _block(fmt)
    _check(load().svdq_quantize_weight(
        int(fmt), _ptr(W, _bf16(), "W", rows=True), N, K, _ld(W), _ptr(lam, torch.float32, "lambda", K),
        _ptr(lora_down if r else None, _bf16(), "lora_down", r * K),
        _ptr(lora_up if r else None, _bf16(), "lora_up", N * r), int(r),
        _ptr(codes, torch.uint8, "codes", _code_bytes(fmt, N, K)),
        _ptr(scales, _scale_dtype(fmt), "scales", N * K // blk),
        _ptr(tensor_scale, torch.float32, "tensor_scale", 1), _stream(stream)))


def svdq_quant_act_lowrank_down(fmt, X, lam, act_amax, lora_down, r, codes, scales,
                                tensor_scale, D, sat_count=None, stream=None):
    """Activation quantisation + D = bf16(X̂)·L1 (fp32 [M, r]); X [M, K] bf16."""
    torch = _torch()
    M, K = X.shape
    blk = _block(fmt)
    _check(load().svdq_quant_act_lowrank_down(
        int(fmt), _ptr(X, _bf16(), "X", rows=True), M, K, _ld(X),
        _ptr(lam, torch.float32, "lambda", K), _ptr(act_amax, torch.float32, "act_amax", 1),
        _ptr(lora_down if r else None, _bf16(), "lora_down", r * K), int(r),
        _ptr(codes, torch.uint8, "codes", _code_bytes(fmt, M, K)),
        _ptr(scales, _scale_dtype(fmt), "scales", M * K // blk),
        _ptr(tensor_scale, torch.float32, "tensor_scale", 1),
        _ptr(D if r else None, torch.float32, "D", M * r),
        _ptr(sat_count, (torch.int32,), "sat_count", 1), _stream(stream)))


def svdq_w4a4_gemm(fmt, M, N, K, a_codes, a_scales, g_a, w_codes, w_scales, g_w, D, lora_up, r,
                   Y, core_out=None, row_to_cube=None, stream=None):
    """Y [M, N] bf16 = W4A4 GEMM + D·L2 (+ core term)."""
    torch = _torch()
    blk = _block(fmt)
    _check(load().svdq_w4a4_gemm(
        int(fmt), M, N, K, _ptr(a_codes, torch.uint8, "a_codes", _code_bytes(fmt, M, K)),
        _ptr(a_scales, _scale_dtype(fmt), "a_scales", M * K // blk),
        _ptr(g_a, torch.float32, "g_a", 1), _ptr(w_codes, torch.uint8, "w_codes", _code_bytes(fmt, N, K)),
        _ptr(w_scales, _scale_dtype(fmt), "w_scales", N * K // blk),
        _ptr(g_w, torch.float32, "g_w", 1), _ptr(D if r else None, torch.float32, "D", M * r),
        _ptr(lora_up if r else None, _bf16(), "lora_up", N * r), int(r),
        _ptr(core_out, torch.float32, "core_out"), _ptr(row_to_cube, torch.int32, "row_to_cube", M),
        _ptr(Y, _bf16(), "Y", M * N, rows=True), _ld(Y), _stream(stream)))


def svdq_cube_geometry(T, H, W, ct, ch, cw, n_text, n_audio, cube1d):
    """Host geometry: returns numpy (row_to_cube, cube_ptr, cube_rows)."""
    import numpy as np
    lib = load()
    n = ctypes.c_int64(0)
    _check(lib.svdq_cube_geometry(T, H, W, ct, ch, cw, n_text, n_audio, cube1d, None, None, None,
                                  ctypes.cast(ctypes.pointer(n), _c_p)))
    M = n_text + T * H * W + n_audio
    r2c = np.zeros(M, np.int32)
    ptr = np.zeros(n.value + 1, np.int32)
    rows = np.zeros(M, np.int32)
    _check(lib.svdq_cube_geometry(T, H, W, ct, ch, cw, n_text, n_audio, cube1d,
                                  r2c.ctypes.data, ptr.ctypes.data, rows.ctypes.data,
                                  ctypes.cast(ctypes.pointer(n), _c_p)))
    return r2c, ptr, rows


def svdq_cube_divisor_aligned(T, H, W, ct, ch, cw):
    """Host: divisor-aligned cube edges (ct', ch', cw')."""
    out = (ctypes.c_int64 * 3)()
    _check(load().svdq_cube_divisor_aligned(T, H, W, ct, ch, cw, ctypes.cast(out, _c_p)))
    return tuple(out)


def svdq_cube_schedule(table, step):
    """Host: cube edges of `step` under a schedule of (first_step, ct, ch, cw) rows."""
    rows = [int(v) for row in table for v in row]
    arr = (ctypes.c_int64 * max(1, len(rows)))(*rows)
    out = (ctypes.c_int64 * 3)()
    _check(load().svdq_cube_schedule(ctypes.cast(arr, _c_p), len(rows) // 4, int(step),
                                     ctypes.cast(out, _c_p)))
    return tuple(out)


def svdq_cube_groups(cube_ptr):
    """Host: work groups of the DeltaQuant activation kernel for a host CSR cube_ptr (numpy
    int32 [n_cubes + 1]); returns group_ptr (numpy int32 [n_groups + 1])."""
    import numpy as np
    cp = np.ascontiguousarray(cube_ptr, dtype=np.int32)
    nc = len(cp) - 1
    n = ctypes.c_int64(0)
    gp = np.zeros(nc + 1, np.int32)
    _check(load().svdq_cube_groups(cp.ctypes.data, nc, gp.ctypes.data,
                                   ctypes.cast(ctypes.pointer(n), _c_p)))
    return gp[:n.value + 1].copy()


def svdq_delta_workspace_bytes(n_cubes, K):
    return int(load().svdq_delta_workspace_bytes(int(n_cubes), int(K)))


def svdq_delta_quant_act(X, lam, act_amax, cube_ptr, cube_rows, n_cubes, group_ptr, lora_down,
                         r, core_codes, core_scale, delta_codes, delta_scales, g_delta, D,
                         sat_count, workspace, stream=None):
    """DeltaQuant activations: FP8 cube-mean core + NVFP4 delta + D; group_ptr from
    svdq_cube_groups (device int32), workspace uint8 (svdq_delta_workspace_bytes)."""
    torch = _torch()
    M, K = X.shape
    _check(load().svdq_delta_quant_act(
        _ptr(X, _bf16(), "X", rows=True), M, K, _ld(X), _ptr(lam, torch.float32, "lambda", K),
        _ptr(act_amax, torch.float32, "act_amax", 1), _ptr(cube_ptr, torch.int32, "cube_ptr"),
        _ptr(cube_rows, torch.int32, "cube_rows", M), int(n_cubes),
        _ptr(group_ptr, torch.int32, "group_ptr"), group_ptr.numel() - 1,
        _ptr(lora_down if r else None, _bf16(), "lora_down", r * K), int(r),
        _ptr(core_codes, torch.uint8, "core_codes", n_cubes * K),
        _ptr(core_scale, torch.float32, "core_scale", n_cubes),
        _ptr(delta_codes, torch.uint8, "delta_codes", M * K // 2),
        _ptr(delta_scales, torch.uint8, "delta_scales", M * K // 16),
        _ptr(g_delta, torch.float32, "g_delta", 1), _ptr(D if r else None, torch.float32, "D", M * r),
        _ptr(sat_count, (torch.int32,), "sat_count", 1),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def svdq_delta_quant_act_noalloc(X, lam, act_amax, cube_ptr, cube_rows, n_cubes, group_ptr,
                                 lora_down, r, core_codes, core_scale, delta_codes, delta_scales,
                                 g_delta, D, sat_count=None, stream=None):
    """svdq_delta_quant_act through the library's static scratch (no workspace argument)."""
    torch = _torch()
    M, K = X.shape
    _check(load().svdq_delta_quant_act_noalloc(
        _ptr(X, _bf16(), "X", rows=True), M, K, _ld(X), _ptr(lam, torch.float32, "lambda", K),
        _ptr(act_amax, torch.float32, "act_amax", 1), _ptr(cube_ptr, torch.int32, "cube_ptr"),
        _ptr(cube_rows, torch.int32, "cube_rows", M), int(n_cubes),
        _ptr(group_ptr, torch.int32, "group_ptr"), group_ptr.numel() - 1,
        _ptr(lora_down if r else None, _bf16(), "lora_down", r * K), int(r),
        _ptr(core_codes, torch.uint8, "core_codes", n_cubes * K),
        _ptr(core_scale, torch.float32, "core_scale", n_cubes),
        _ptr(delta_codes, torch.uint8, "delta_codes", M * K // 2),
        _ptr(delta_scales, torch.uint8, "delta_scales", M * K // 16),
        _ptr(g_delta, torch.float32, "g_delta", 1), _ptr(D if r else None, torch.float32, "D", M * r),
        _ptr(sat_count, (torch.int32,), "sat_count", 1), _stream(stream)))


def svdq_gemm_core(n_cubes, N, K, core_codes, core_scale, w_codes, w_scales, g_w, core_out,
                   stream=None):
    """core_out [n_cubes, N] fp32."""
    torch = _torch()
    _check(load().svdq_gemm_core(
        int(n_cubes), N, K, _ptr(core_codes, torch.uint8, "core_codes", n_cubes * K),
        _ptr(core_scale, torch.float32, "core_scale", n_cubes),
        _ptr(w_codes, torch.uint8, "w_codes", N * K // 2),
        _ptr(w_scales, torch.uint8, "w_scales", N * K // 16), _ptr(g_w, torch.float32, "g_w", 1),
        _ptr(core_out, torch.float32, "core_out", n_cubes * N), _stream(stream)))


def svdq_score_reference_rows(X, W, rows, Yref, stream=None):
    """Yref [n_rows, N] bf16 = bf16(X[rows] · Wᵀ) (written)."""
    torch = _torch()
    M, K = X.shape
    N = W.shape[0]
    n = rows.numel()
    _check(load().svdq_score_reference_rows(
        _ptr(X, _bf16(), "X", rows=True), _ld(X), _ptr(W, _bf16(), "W", rows=True), _ld(W), M, N,
        K, _ptr(rows, torch.int32, "rows"), n, _ptr(Yref, _bf16(), "Yref", n * N, rows=True),
        _ld(Yref), _stream(stream)))


def svdq_score_modal_rel_l2_ref(Y, Yref, rows, row_group, sums, stream=None):
    """Adds per-group (Σ(Y[rows]−Yref)², ΣYref²) into sums (fp64 [4, 2])."""
    torch = _torch()
    M, N = Y.shape
    n = rows.numel()
    _check(load().svdq_score_modal_rel_l2_ref(
        _ptr(Y, _bf16(), "Y", M * N, rows=True), _ld(Y),
        _ptr(Yref, _bf16(), "Yref", n * N, rows=True), _ld(Yref), M, N,
        _ptr(rows, torch.int32, "rows"), _ptr(row_group, torch.int8, "row_group"), n,
        _ptr(sums, torch.float64, "sums", 8), _stream(stream)))


def svdq_score_modal_rel_l2(Y, X, W, rows, row_group, sums, stream=None):
    """Adds per-group (Σ(Y−Y_ref)², ΣY_ref²) into sums (fp64 [4, 2])."""
    torch = _torch()
    M, K = X.shape
    N = W.shape[0]
    _check(load().svdq_score_modal_rel_l2(
        _ptr(Y, _bf16(), "Y", M * N, rows=True), _ld(Y), _ptr(X, _bf16(), "X", rows=True), _ld(X),
        _ptr(W, _bf16(), "W", rows=True), _ld(W), M, N, K, _ptr(rows, torch.int32, "rows"),
        _ptr(row_group, torch.int8, "row_group"), rows.numel(),
        _ptr(sums, torch.float64, "sums", 8), _stream(stream)))
