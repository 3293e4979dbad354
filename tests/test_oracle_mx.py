"""Pins of the oracle's MX quantiser (E8M0 scale per 32, E2M1 / E4M3 elements) against facts that
do not depend on its code: the exponent rule as an inequality, worked blocks computed by hand,
an exhaustive nearest-even search, idempotence, and the exact dequantised product.

"MiniMax-H3 — MXFP8 (weight-quantized, vLLM-Omni native layout)", section "Quant format" (mx_fp,
group size 32, E8M0 block scales, round to nearest); block exponent by the OCP microscaling rule
(the reading stated in oracle/mx.py)."""
import numpy as np
import pytest

from oracle import mx
from oracle.formats import E2M1_VALUES, E4M3_VALUES, unpack_nibbles

F32 = np.float32


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_exponent_rule_brackets_the_block_max(elem):
    rng = np.random.default_rng(0)
    a = np.concatenate([
        (rng.standard_normal(4000) * 10.0 ** rng.uniform(-30, 30, 4000)).astype(F32),
        np.ldexp(F32(1), np.arange(-140, 127)).astype(F32),          # powers of two
        np.nextafter(np.ldexp(F32(1), np.arange(-120, 120)).astype(F32), F32(0)),  # just below
    ])
    a = np.abs(a[np.isfinite(a) & (a != 0)])
    e = mx.mx_exponent(a, elem)
    emax = {"e2m1": 2, "e4m3": 8}[elem]
    lo = np.ldexp(1.0, e + emax)
    inside = e > -127
    # 2^(e + emax) <= a < 2^(e + emax + 1), exactly, unless the exponent was clamped at -127
    assert np.all(lo[inside] <= a[inside].astype(np.float64))
    assert np.all(a.astype(np.float64) < 2 * lo)
    assert np.all(a[~inside].astype(np.float64) < np.ldexp(1.0, -127 + emax + 1))


def test_zero_block_has_the_smallest_scale_and_zero_codes():
    for elem in ("e2m1", "e4m3"):
        codes, scales = mx.mx_quantize(np.zeros((2, 64), F32), elem)
        assert np.all(scales == 0)
        assert np.all(mx.mx_dequantize(codes, scales, elem) == 0)


def test_worked_mxfp4_block():
    # block max 6.5: floor(log2 6.5) = 2, e = 0, q = x; 6.5 saturates to 6 (code 7);
    # -0.3 is nearer 0.5 than 0 (code 0x9); 2.5 ties between 2 and 3 -> even code 4 (value 2)
    x = np.zeros((1, 32), F32)
    x[0, :4] = [6.5, -0.3, 2.5, 0.0]
    codes, scales = mx.mx_quantize(x, "e2m1")
    nib = unpack_nibbles(codes)[0]
    assert scales[0, 0] == 127
    assert list(nib[:4]) == [7, 0x9, 4, 0]
    # block max 0.75: floor(log2 0.75) = -1, e = -3, q = 8x: 0.75 -> 6 (code 7), 0.1 -> 0.8 -> 1
    x = np.zeros((1, 32), F32)
    x[0, :2] = [0.75, 0.1]
    codes, scales = mx.mx_quantize(x, "e2m1")
    assert scales[0, 0] == 124
    assert list(unpack_nibbles(codes)[0, :2]) == [7, 2]


def test_worked_mxfp8_block():
    # block max 1000: floor(log2 1000) = 9, e = 1, q = x/2: 500 saturates to 448 (0x7E);
    # 3 -> 1.5 = 1.100b · 2^0: exponent field 7, mantissa 4 -> 0x3C; -3 -> 0xBC
    x = np.zeros((1, 32), F32)
    x[0, :3] = [1000.0, 3.0, -3.0]
    codes, scales = mx.mx_quantize(x, "e4m3")
    assert scales[0, 0] == 128
    assert list(codes[0, :3]) == [0x7E, 0x3C, 0xBC]


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_codes_are_nearest_even_by_exhaustive_search(elem):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 32)) * np.exp(rng.standard_normal((64, 1)) * 3)).astype(F32)
    x[::7, 5] = 0.0
    codes, scales = mx.mx_quantize(x, elem)
    table = E2M1_VALUES if elem == "e2m1" else E4M3_VALUES
    top = table.max()
    got = mx.mx_dequantize(codes, scales, elem)
    for i in range(x.shape[0]):
        e = int(scales[i, 0]) - 127
        q = np.abs(x[i].astype(np.float64)) * 2.0 ** (-e)
        for k in range(32):
            v = min(q[k], top)
            d = np.abs(table - v)
            best = np.flatnonzero(d == d.min())
            pick = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            want = table[pick] * 2.0 ** e * (-1 if np.signbit(x[i, k]) else 1)
            assert got[i, k] == want


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_requantising_dequantised_values_is_the_identity(elem):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((16, 128)) * 5).astype(F32)
    codes, scales = mx.mx_quantize(x, elem)
    deq = mx.mx_dequantize(codes, scales, elem).astype(F32)
    codes2, scales2 = mx.mx_quantize(deq, elem)
    assert np.array_equal(scales, scales2)
    # negative zeros may come back as +0 codes only where the value is zero
    v1, v2 = mx.mx_dequantize(codes, scales, elem), mx.mx_dequantize(codes2, scales2, elem)
    assert np.array_equal(v1, v2)


def test_layer_output_is_the_exact_product_of_dequantised_operands():
    from oracle import gemm
    rng = np.random.default_rng(3)
    a = (rng.standard_normal((4, 64))).astype(F32)
    w = (rng.standard_normal((8, 64))).astype(F32)
    ac, as_ = mx.mx_quantize(a, "e2m1")
    wc, ws = mx.mx_quantize(w, "e2m1")
    up = np.zeros((8, 0), np.uint16)
    y64, _ = gemm.linear_mx(ac, as_, wc, ws, np.zeros((4, 0)), up, "e2m1")
    # brute force: sum over k of code values times block scales
    A = mx.mx_dequantize(ac, as_, "e2m1")
    W = mx.mx_dequantize(wc, ws, "e2m1")
    ref = np.array([[sum(A[i, k] * W[j, k] for k in range(64)) for j in range(8)] for i in range(4)])
    assert np.array_equal(y64, ref)
