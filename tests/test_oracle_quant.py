"""Pins of the oracle's NVFP4 and int4 quantisers: exact on-grid cases, idempotence, the block
maximum landing on the top code, error bounds, saturation, and signed zeros."""
import numpy as np

from oracle import quant as Q
from oracle import formats as F

F32 = np.float32


def _on_grid_nvfp4_block(rng, j):
    """16 values v * 2^j, v from the E2M1 set, with a ±6 among them (block absmax 6 * 2^j)."""
    v = rng.choice(F.E2M1_VALUES, 16) * rng.choice([-1.0, 1.0], 16)
    v[rng.integers(0, 16)] = 6.0 * rng.choice([-1.0, 1.0])
    return v * 2.0 ** j


def test_nvfp4_exact_on_grid_with_power_of_two_tensor_scale():
    rng = np.random.default_rng(0)
    p = 2
    rows = []
    for _ in range(6):
        rows.append(np.concatenate([_on_grid_nvfp4_block(rng, j) for j in rng.integers(-6, 3, 4)]))
    x = np.array(rows, dtype=F32)
    codes, scales, g, sat = Q.nvfp4_quantize(x, F32(2688.0 * 2 ** p))
    assert g == F32(2.0 ** p) and sat == 0
    assert np.array_equal(Q.nvfp4_dequantize(codes, scales, g), x.astype(np.float64))


def test_nvfp4_unit_scale_block_is_plain_e2m1_rounding():
    # amax_t = 2688 -> g = 1; a block whose absmax is 6 gets q = 1 -> s = 1.0 -> S = 1, so every
    # code is the plain E2M1 rounding of the element.
    rng = np.random.default_rng(1)
    x = rng.uniform(-6, 6, (50, 16)).astype(F32)
    x[:, 3] = 6.0
    codes, scales, g, _ = Q.nvfp4_quantize(x, F32(2688.0))
    assert np.all(scales == 0x38)
    nib = F.unpack_nibbles(codes)
    assert np.array_equal(nib & 7, F.e2m1_encode_mag(np.abs(x)))
    assert np.array_equal(nib >> 3, np.signbit(x).astype(np.uint8))


def test_nvfp4_roundtrip_idempotent_and_block_max_on_top_code():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal(256))).astype(F32)
    amax = F32(np.abs(x).max())
    codes, scales, g, sat = Q.nvfp4_quantize(x, amax)
    normal = F.e4m3_decode(scales) >= 2.0 ** -6
    assert normal.mean() > 0.9
    xd = Q.nvfp4_dequantize(codes, scales, g).astype(F32)
    codes2, scales2, g2, _ = Q.nvfp4_quantize(xd, amax)
    assert g2 == g
    nb = normal.repeat(8, axis=1)      # 8 bytes per 16-block
    assert np.array_equal(scales2[normal], scales[normal])
    assert np.array_equal(codes2[nb], codes[nb])
    nib = F.unpack_nibbles(codes).reshape(64, 16, 16)
    top = (nib & 7).max(axis=2)
    assert np.all(top[normal] == 7)   # every normal-scale block holds a ±6


def test_nvfp4_error_bound_and_saturation_count():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((32, 128)).astype(F32)
    amax = F32(np.abs(x).max())
    codes, scales, g, sat = Q.nvfp4_quantize(x, amax)
    S = (F.e4m3_decode(scales) * np.float64(g)).repeat(16, axis=1)
    err = np.abs(Q.nvfp4_dequantize(codes, scales, g) - x)
    assert np.all(err <= S * 1.0 + 1e-12)          # largest E2M1 half-gap is 1 (between 4 and 6)
    assert sat == 0
    # a tensor amax smaller than a block absmax saturates that block (q > 448)
    _, s2, _, sat2 = Q.nvfp4_quantize(x, amax / F32(4.0))
    assert sat2 > 0 and np.any(s2 == 0x7E)


def test_nvfp4_signed_zero_and_zero_block():
    x = np.zeros((2, 16), dtype=F32)
    x[0, 0] = 6.0
    x[0, 1] = -1e-6          # rounds to zero, keeps its sign
    x[1, 2] = -0.0
    codes, scales, _, _ = Q.nvfp4_quantize(x, F32(6.0))
    nib = F.unpack_nibbles(codes)
    assert nib[0, 1] == 0x8 and nib[0, 0] == 0x7 and nib[0, 2] == 0x0
    assert scales[1, 0] == 0 and nib[1, 2] == 0x8 and np.all(np.delete(nib[1], 2) == 0)


def test_int4_exact_on_grid_and_top_code():
    rng = np.random.default_rng(4)
    s = F.fp16_rne(rng.uniform(0.01, 3, (8, 4)).astype(F32)).astype(np.float64)
    c = rng.integers(-7, 8, (8, 4, 64))
    c[:, :, 5] = 7 * rng.choice([-1, 1], (8, 4))
    x = (c * s[:, :, None]).reshape(8, 256).astype(F32)
    assert np.array_equal(x.astype(np.float64), (c * s[:, :, None]).reshape(8, 256))
    codes, s16 = Q.int4_quantize(x)
    assert np.array_equal(s16.astype(np.float64), s)
    assert np.array_equal(Q.int4_codes_signed(codes).reshape(8, 4, 64), c)
    assert np.array_equal(Q.int4_dequantize(codes, s16), x.astype(np.float64))


def test_int4_range_error_bound_and_no_minus_eight_from_rtn():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 512)) * 3).astype(F32)
    codes, s16 = Q.int4_quantize(x)
    c = Q.int4_codes_signed(codes)
    assert c.min() >= -7 and c.max() <= 7
    assert np.all(np.abs(c.reshape(40, 8, 64)).max(axis=2) == 7)
    err = np.abs(Q.int4_dequantize(codes, s16) - x)
    S = s16.astype(np.float64).repeat(64, axis=1)
    assert np.all(err <= S * 0.5 + S * 2.0 ** -10 + 1e-12)
    assert np.allclose(s16.astype(np.float64),
                       np.abs(x).reshape(40, 8, 64).max(axis=2) / 7, rtol=2 ** -10)


def test_int4_two_complement_nibbles_and_zero_group():
    x = np.zeros((1, 64), dtype=F32)
    x[0, 0], x[0, 1] = 7.0, -7.0
    codes, s16 = Q.int4_quantize(x)
    assert s16[0, 0] == 1.0
    assert codes[0, 0] == (0x7 | (0x9 << 4))     # 7 in the low nibble, -7 = 0x9 in the high one
    z, sz = Q.int4_quantize(np.zeros((1, 64), dtype=F32))
    assert sz[0, 0] == 0 and np.all(z == 0)
