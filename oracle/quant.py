"""NVFP4 and int4-g64 quantisers (round to nearest even), and their exact dequantisation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

NVFP4 (source: "MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on", section
"Why"; the format: an E4M3 byte scales each block of 16 channels along K, derived from that
block's maximum, under one fp32 scale for the whole tensor).  The pages give the structure but not the arithmetic; the reading used here,
with its float32 operation order pinned so that codes are reproducible bit for bit:

    g   = amax_t / 2688            (2688 = 6 * 448; g = 1 when amax_t == 0)
    d6  = 6 * g
    per block of 16 along K:
        a = max |x|
        q = a / d6
        s = E4M3(q)                nearest-even, satfinite at 448
        S = value(s) * g
        S == 0  ->  every code is a signed zero
        else    ->  inv = 1 / S ;  code = sign(x) | E2M1(|x| * inv)
    a block is "saturated" when its absmax exceeds the tensor amax the tensor scale came from,
    a > amax_t (then its required scale would exceed the largest E4M3 value, 448).  The
    comparison is made on the exact values, so rounding in q cannot flag the block that holds
    the tensor amax itself.  Saturated groups are counted as the DeltaQuant page counts them at
    run time (section "The activation scale bound held").

The division-free "x * (1/S)" form (a reciprocal per block, a multiply per element) is the
reading chosen for the element step; the sign bit of a code is the sign bit of x, so a negative
value that rounds to zero gives code 0x8.

int4 per group of 64 ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph:
int4 activations quantised per token at run time; group size 64 and fp16 scales as in the int4
workload):

    per group of 64 along K:
        a = max |x|
        s = fp16(a / 7)            round to nearest even
        s == 0 -> codes 0
        else   -> inv = 1 / float(s) ;  code = clamp(rint(x * inv), -8, 7)   (rint: half to even)
    codes are two's-complement nibbles, element 2j in the low nibble of byte j.
"""
import numpy as np

from .formats import (e4m3_encode, e4m3_decode, e2m1_encode_mag, e2m1_decode, fp16_rne,
                      pack_nibbles, unpack_nibbles)

NVFP4_BLOCK = 16
INT4_GROUP = 64
F32 = np.float32


def nvfp4_tensor_scale(amax_t):
    """g = amax_t / 2688 in float32 (1 when amax_t is 0)."""
    amax_t = F32(amax_t)
    if amax_t == 0:
        return F32(1.0)
    return F32(amax_t / F32(2688.0))


def nvfp4_block_scales(a, g):
    """E4M3 codes s and float32 values S = value(s)·g of the block scales for block maxima a."""
    d6 = F32(F32(6.0) * F32(g))
    q = (np.asarray(a, dtype=F32) / d6).astype(F32)
    s = e4m3_encode(q)
    S = (e4m3_decode(s).astype(F32) * F32(g)).astype(F32)
    return s, S


def nvfp4_nibbles(x32, S):
    """E2M1 nibbles (sign in bit 3) of float32 x under block scale values S (same shape)."""
    x32 = np.asarray(x32, dtype=F32)
    S = np.asarray(S, dtype=F32)
    nz = S != 0
    inv = np.zeros_like(S)
    inv[nz] = (F32(1.0) / S[nz]).astype(F32)
    y = (np.abs(x32) * inv).astype(F32)
    mag = e2m1_encode_mag(y)
    mag[~nz] = 0
    return (mag | (np.signbit(x32).astype(np.uint8) << np.uint8(3))).astype(np.uint8)


def nvfp4_quantize(x32, amax_t):
    """Quantise float32 rows [R, K] to NVFP4 with tensor amax `amax_t`.

    Returns (codes uint8 [R, K/2], scales uint8 [R, K/16] (E4M3), g float32, n_saturated int).
    """
    x32 = np.asarray(x32, dtype=F32)
    R, K = x32.shape
    if K % NVFP4_BLOCK:
        raise ValueError("K must be a multiple of 16")
    g = nvfp4_tensor_scale(amax_t)
    xb = x32.reshape(R, K // NVFP4_BLOCK, NVFP4_BLOCK)
    a = np.abs(xb).max(axis=2)                              # exact
    n_sat = int(np.count_nonzero(a > F32(amax_t)))
    s, S = nvfp4_block_scales(a, g)                         # [R, K/16]
    nib = nvfp4_nibbles(xb, np.broadcast_to(S[:, :, None], xb.shape))
    codes = pack_nibbles(nib.reshape(R, K))
    return codes, s.astype(np.uint8), g, n_sat


def nvfp4_dequantize(codes, scales, g):
    """Exact float64 values code * scale * g of an NVFP4 tensor [R, K]."""
    nib = unpack_nibbles(codes)
    R, K = nib.shape
    v = e2m1_decode(nib).reshape(R, K // NVFP4_BLOCK, NVFP4_BLOCK)
    s = e4m3_decode(scales)[:, :, None]
    return (v * s * np.float64(F32(g))).reshape(R, K)


def int4_quantize(x32):
    """Quantise float32 rows [R, K] to int4 with one fp16 scale per 64 along K.

    Returns (codes uint8 [R, K/2], scales float16 [R, K/64]).
    """
    x32 = np.asarray(x32, dtype=F32)
    R, K = x32.shape
    if K % INT4_GROUP:
        raise ValueError("K must be a multiple of 64")
    xg = x32.reshape(R, K // INT4_GROUP, INT4_GROUP)
    s16 = int4_scale(np.abs(xg).max(axis=2))
    c = int4_codes(xg, np.broadcast_to(s16[:, :, None], xg.shape))
    nib = (c.astype(np.uint8) & np.uint8(0xF)).reshape(R, K)
    return pack_nibbles(nib), s16


def int4_scale(a):
    """fp16 scales fp16(a / 7) of groups with float32 absmax a."""
    return fp16_rne((np.asarray(a, dtype=F32) / F32(7.0)).astype(F32))


def int4_codes(x32, s16):
    """int8 codes clamp(rint(x · fl32(1/s)), −8, 7) of float32 x under fp16 scales s16 of the
    same shape (0 where s == 0)."""
    x32 = np.asarray(x32, dtype=F32)
    sf = np.asarray(s16, dtype=np.float16).astype(F32)
    nz = sf != 0
    inv = np.zeros_like(sf)
    inv[nz] = (F32(1.0) / sf[nz]).astype(F32)
    v = (x32 * inv).astype(F32)
    c = np.clip(np.rint(v), -8, 7).astype(np.int8)
    c[~nz] = 0
    return c


def int4_dequantize(codes, scales16):
    """Exact float64 values code * scale of an int4-g64 tensor [R, K]."""
    nib = unpack_nibbles(codes).astype(np.int16)
    c = np.where(nib >= 8, nib - 16, nib).astype(np.float64)
    R, K = c.shape
    s = np.asarray(scales16, dtype=np.float16).astype(np.float64)[:, :, None]
    return (c.reshape(R, K // INT4_GROUP, INT4_GROUP) * s).reshape(R, K)


def int4_codes_signed(codes):
    """Packed int4 bytes -> int8 codes [R, K]."""
    nib = unpack_nibbles(codes).astype(np.int16)
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)
