"""MX (OCP microscaling) quantisers: one E8M0 power-of-two scale per 32 elements along K, with
E2M1 (MXFP4) or E4M3 (MXFP8) elements, and their exact dequantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"MiniMax-H3 — MXFP8 (weight-quantized, vLLM-Omni native layout)", section "Quant format": the
format is mx_fp with 8-bit elements (F8_E4M3), group size 32, symmetric, round-to-nearest (no
tuning iterations), per-32 E8M0 block scales, and dynamically quantised activations with the same
group size.  The page does not spell out how the block exponent is chosen; the reading used here
is the OCP microscaling rule, with the element step pinned in float32:

    emax = exponent of the element format's largest normal (E4M3: 448 = 1.75·2^8 -> 8;
           E2M1: 6 = 1.5·2^2 -> 2)
    per block of 32 along K:
        a = max |x|
        e = floor(log2 a) - emax        (a == 0 -> e = -127), clamped to [-127, 127]
        scale code = e + 127            (E8M0: value 2^(code - 127))
        q = x · 2^-e                    (a power-of-two scaling, exact in float32 wherever it
                                         can change a code)
        code = element(q)               nearest even, saturating at the largest finite value;
                                         the sign bit is the sign of x, also when q rounds to 0
MXFP4 codes are packed two per byte, element 2j in the low nibble of byte j; MXFP8 codes are one
byte per element.  The W4A4 (MXFP4) and W8A8 (MXFP8) variants of the layer use the same
quantiser for the weight residual and for the smoothed activations.
"""
import numpy as np

from .formats import (e2m1_decode, e2m1_encode_mag, e4m3_decode, e4m3_encode_signed,
                      pack_nibbles, unpack_nibbles)

F32 = np.float32
BLOCK = 32
EMAX = {"e2m1": 2, "e4m3": 8}


def mx_exponent(a, elem):
    """Block exponents e for non-negative float32 block maxima a (any shape)."""
    a = np.asarray(a, dtype=F32).astype(np.float64)
    _, ex = np.frexp(a)                       # a = m · 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1
    e = ex.astype(np.int64) - 1 - EMAX[elem]
    e = np.where(a == 0, -127, e)
    return np.clip(e, -127, 127)


def mx_quantize(x32, elem):
    """Quantise float32 rows [R, K] (K % 32 == 0): (codes, scales E8M0 uint8 [R, K/32]).

    codes: MXFP4 packed nibbles [R, K/2]; MXFP8 bytes [R, K]."""
    x32 = np.asarray(x32, dtype=F32)
    R, K = x32.shape
    xb = x32.reshape(R, K // BLOCK, BLOCK)
    a = np.abs(xb).max(axis=2)
    e = mx_exponent(a, elem)                                  # [R, K/32]
    el = mx_element_codes(xb, np.broadcast_to(e[:, :, None], xb.shape), elem).reshape(R, K)
    codes = pack_nibbles(el) if elem == "e2m1" else el
    scales = (e + 127).astype(np.uint8)
    return codes, scales


def mx_element_codes(x32, e, elem):
    """Element codes (E2M1 nibble with the sign in bit 3, or E4M3 byte) of float32 x in blocks
    of exponent e (same shape)."""
    x32 = np.asarray(x32, dtype=F32)
    q = np.ldexp(x32, (-np.asarray(e)).astype(np.int32)).astype(F32)
    if elem == "e2m1":
        mag = e2m1_encode_mag(np.abs(q))
        return (mag | (np.signbit(x32).astype(np.uint8) << 3)).astype(np.uint8)
    return e4m3_encode_signed(q)


def mx_dequantize(codes, scales, elem):
    """Exact float64 values code · 2^(scale - 127) of an MX tensor [R, K]."""
    scales = np.asarray(scales, dtype=np.int64)
    if elem == "e2m1":
        vals = e2m1_decode(unpack_nibbles(codes))
    else:
        vals = e4m3_decode(codes)
    R, K = vals.shape
    mult = np.ldexp(1.0, scales - 127)                        # [R, K/32]
    return (vals.reshape(R, K // BLOCK, BLOCK) * mult[:, :, None]).reshape(R, K)
