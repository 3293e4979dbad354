"""Number formats used by the W4A4 layer, written out from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bf16: 1 sign, 8 exponent, 7 mantissa bits; round to nearest, ties to even.
* fp16 (IEEE binary16): numpy's float32 -> float16 cast, which rounds to nearest even.
* E4M3 ("FP8", the NVFP4 block-scale format and the DeltaQuant core format): 1 sign,
  4 exponent (bias 7), 3 mantissa bits, no infinities; the largest finite value is 448 and the
  smallest subnormal 2^-9.  Encoding here is "satfinite": magnitudes above 448 become 448.
* E2M1 ("FP4", the NVFP4 element format): magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign bit 3.
  Encoding saturates at 6.

The NVFP4 structure (16 consecutive K-elements share one FP8 scale set by the group absmax, plus
an fp32 tensor scale) is stated in "MiniMax-H3 NVFP4 — what the smoothing scale should be
calibrated on", section "Why".  The value sets above are the formats' own definitions.

Every encoder picks the nearest representable value and breaks an exact tie toward the even code
(the code whose least significant bit is 0), which is round-to-nearest-even for these formats
because their codes are ordered like their values.
"""
import numpy as np

# --------------------------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------------------------

def bf16_bits_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_rne(x):
    """Round float32 / float64 values to bf16 (nearest, ties to even); returns uint16 bits.

    Done in float64 arithmetic, which is exact here: the rounding quantum q is a power of two,
    x / q is exact and has fewer than 53 significant bits, np.rint rounds half to even, and the
    product by q is exact.  Values whose magnitude rounds past the largest finite bf16 become
    infinities; NaN is not expected.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                        # ax = m * 2**e with m in [0.5, 1)
    # bf16 keeps 8 significant bits: quantum 2**(e-8); subnormal quantum 2**-133.
    qexp = np.maximum(e - 8, -133)
    q = np.ldexp(1.0, qexp)
    r = np.rint(ax / q) * q
    r = np.where(ax == 0, 0.0, r)
    r = np.copysign(r, x)
    big = np.abs(r) > 3.3895313892515355e38    # (2 - 2**-7) * 2**127
    r32 = r.astype(np.float32)                 # exact: r is representable in bf16 ⊂ float32
    r32 = np.where(big, np.copysign(np.float32(np.inf), r32), r32).astype(np.float32)
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_round_f32(x):
    """float values rounded to bf16 and returned as float32."""
    return bf16_bits_to_f32(bf16_rne(x))


# --------------------------------------------------------------------------------------------
# fp16
# --------------------------------------------------------------------------------------------

def fp16_rne(x32):
    """float32 -> float16, round to nearest even (numpy's IEEE cast)."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------------------------
# E4M3
# --------------------------------------------------------------------------------------------

def _e4m3_table():
    """Values of the 127 non-negative finite E4M3 codes 0x00..0x7E, in code order."""
    vals = []
    for code in range(0x7F):
        e = code >> 3
        m = code & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)                 # subnormal: m/8 * 2^(1-7)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3_VALUES = _e4m3_table()          # index = code, strictly increasing
E4M3_MAX = 448.0


def _nearest_even(table, v):
    """Index of the entry of the increasing `table` nearest to v (v within the table's range),
    ties toward the even index."""
    v = np.asarray(v, dtype=np.float64)
    hi = np.searchsorted(table, v, side="left")          # first entry >= v
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    dlo = np.abs(v - table[lo])
    dhi = np.abs(table[hi] - v)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def e4m3_encode(v):
    """Non-negative float32 values -> E4M3 codes (uint8), nearest-even, satfinite at 448."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode expects non-negative, non-NaN magnitudes")
    v = np.minimum(v, E4M3_MAX)
    return _nearest_even(E4M3_VALUES, v).astype(np.uint8)


def e4m3_encode_signed(v):
    """float32 values -> E4M3 codes with the sign in bit 7 (sign of the input, also for zero)."""
    v = np.asarray(v, dtype=np.float32)
    mag = e4m3_encode(np.abs(v))
    return (mag | (np.signbit(v).astype(np.uint8) << np.uint8(7))).astype(np.uint8)


def e4m3_decode(codes):
    """E4M3 codes (sign in bit 7) -> float64 values (exact).  0x7F / 0xFF (NaN) rejected."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = c & np.uint8(0x7F)
    if np.any(mag == 0x7F):
        raise ValueError("E4M3 NaN code")
    val = E4M3_VALUES[mag]
    return np.where(c & np.uint8(0x80), -val, val)


# --------------------------------------------------------------------------------------------
# E2M1
# --------------------------------------------------------------------------------------------

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0


def e2m1_encode_mag(y):
    """Non-negative float32 magnitudes -> 3-bit E2M1 magnitude codes, nearest-even, saturating."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    y = np.minimum(y, E2M1_MAX)
    return _nearest_even(E2M1_VALUES, y).astype(np.uint8)


def e2m1_decode(nibbles):
    """4-bit E2M1 codes (sign in bit 3) -> float64 values."""
    n = np.asarray(nibbles, dtype=np.uint8)
    val = E2M1_VALUES[n & np.uint8(7)]
    return np.where(n & np.uint8(8), -val, val)


# --------------------------------------------------------------------------------------------
# nibble packing (reading: low nibble holds the even K index)
# --------------------------------------------------------------------------------------------

def pack_nibbles(nib):
    """[..., K] 4-bit values -> [..., K/2] bytes; element 2j in the low nibble of byte j."""
    nib = np.asarray(nib, dtype=np.uint8)
    if nib.shape[-1] % 2:
        raise ValueError("K must be even")
    lo = nib[..., 0::2] & np.uint8(0xF)
    hi = nib[..., 1::2] & np.uint8(0xF)
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed):
    """[..., K/2] bytes -> [..., K] 4-bit values (inverse of pack_nibbles)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0xF)
    out[..., 1::2] = p >> np.uint8(4)
    return out
