"""Low-rank down-projection and the W4A4 linear, in float64 from exactly dequantised operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph) is
    Y = X̂·L1·L2 + Q(X̂)·Q(R)
Readings:
  * the low-rank branch is 16-bit: its input is the bf16-rounded X̂ and its factors L1, L2 are
    bf16; the intermediate D = bf16(X̂) @ L1 is NOT rounded again (it is kept at the
    accumulator's precision between the two products): D = float64(bf16(X̂)) @ float64(L1);
  * no bias;
  * Y64 = A_deq @ W_deqᵀ + D @ L2 in float64, where A_deq / W_deq are the exact dequantised
    NVFP4 (code · scale · tensor scale) or int4 (code · scale) operands; Y = bf16(Y64).
"""
import numpy as np

from .formats import bf16_bits_to_f32, bf16_rne, bf16_round_f32
from .quant import nvfp4_dequantize, int4_dequantize
from .mx import mx_dequantize


def lowrank_down(xhat32, lora_down_bits):
    """D = bf16(X̂) @ L1 in float64 with L1 = lora_downᵀ; [M, r] float64."""
    xb = bf16_round_f32(xhat32).astype(np.float64)                   # [M, K]
    L1 = bf16_bits_to_f32(lora_down_bits).astype(np.float64).T        # [K, r]
    if L1.shape[1] == 0:
        return np.zeros((xb.shape[0], 0))
    return xb @ L1


def lowrank_up(D, lora_up_bits):
    """D @ L2 in float64, [M, N] (L2 = lora_upᵀ); D float64 [M, r]."""
    D = np.asarray(D, dtype=np.float64)                               # [M, r]
    up = bf16_bits_to_f32(lora_up_bits).astype(np.float64)            # [N, r]
    if up.shape[1] == 0:
        return np.zeros((D.shape[0], up.shape[0]))
    return D @ up.T


def linear_f64(A_deq, W_deq, D, lora_up_bits):
    """Y64 = A_deq @ W_deqᵀ + D @ L2."""
    return A_deq @ np.asarray(W_deq, dtype=np.float64).T + lowrank_up(D, lora_up_bits)


def linear_nvfp4(a_codes, a_scales, g_a, w_codes, w_scales, g_w, D, lora_up_bits):
    """NVFP4 W4A4 layer output: (Y64 float64 [M, N], Y bf16 bits [M, N])."""
    A = nvfp4_dequantize(a_codes, a_scales, g_a)
    W = nvfp4_dequantize(w_codes, w_scales, g_w)
    y64 = linear_f64(A, W, D, lora_up_bits)
    return y64, bf16_rne(y64)


def linear_int4(a_codes, a_scales16, w_codes, w_scales16, D, lora_up_bits):
    """int4-g64 W4A4 layer output: (Y64, Y bf16 bits)."""
    A = int4_dequantize(a_codes, a_scales16)
    W = int4_dequantize(w_codes, w_scales16)
    y64 = linear_f64(A, W, D, lora_up_bits)
    return y64, bf16_rne(y64)


def linear_mx(a_codes, a_scales, w_codes, w_scales, D, lora_up_bits, elem):
    """MX (MXFP4 W4A4 or MXFP8 W8A8) layer output: (Y64, Y bf16 bits)."""
    A = mx_dequantize(a_codes, a_scales, elem)
    W = mx_dequantize(w_codes, w_scales, elem)
    y64 = linear_f64(A, W, D, lora_up_bits)
    return y64, bf16_rne(y64)


def reference_bf16_linear(X_bits, W_bits):
    """Unquantised reference Y_ref = bf16(X @ Wᵀ) from the bf16 X and W, product in float64."""
    X = bf16_bits_to_f32(X_bits).astype(np.float64)
    W = bf16_bits_to_f32(W_bits).astype(np.float64)
    return bf16_rne(X @ W.T)
