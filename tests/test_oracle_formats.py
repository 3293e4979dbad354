"""Pins of the oracle's number formats: closed-form value sets, tie rules, library casts."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ------------------------------------------------------------------------------ E2M1

def test_e2m1_value_set_matches_golden():
    for row in _read_golden("e2m1_format.txt"):
        if row[0].isdigit():
            code, val = int(row[0]), float(row[1])
            got = F.e2m1_decode(np.array([code], dtype=np.uint8))[0]
            assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e2m1_ties_and_saturation_match_golden():
    for row in _read_golden("e2m1_format.txt"):
        if row[0] in ("tie", "sat"):
            y, code = np.float32(float(row[1])), int(row[2])
            assert F.e2m1_encode_mag(np.array([y]))[0] == code, row


def _brute_nearest_even(values, y):
    """argmin over all table entries, exact ties resolved to the even index."""
    d = np.abs(values[None, :] - y[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.argmax(cand, axis=1)
    two = cand.sum(axis=1) == 2
    second = len(values) - 1 - np.argmax(cand[:, ::-1], axis=1)
    return np.where(two & (idx % 2 == 1), second, idx)


def test_e2m1_encoder_equals_brute_force_on_midpoints_and_dense_grid():
    mids = (F.E2M1_VALUES[1:] + F.E2M1_VALUES[:-1]) / 2
    pts = list(F.E2M1_VALUES) + list(mids)
    ys = []
    for p in pts:
        p32 = np.float32(p)
        ys += [p32, np.nextafter(p32, np.float32(0)), np.nextafter(p32, np.float32(np.inf))]
    ys += list(np.linspace(0, 6, 6001, dtype=np.float32))
    ys = np.array(ys, dtype=np.float32)
    ys = ys[ys >= 0]
    got = F.e2m1_encode_mag(ys)
    want = _brute_nearest_even(F.E2M1_VALUES, ys.astype(np.float64))
    assert np.array_equal(got, want)


# ------------------------------------------------------------------------------ E4M3

def test_e4m3_value_set_closed_form():
    v = F.E4M3_VALUES
    assert len(v) == 127 and np.all(np.diff(v) > 0)
    g = {r[0]: r[1:] for r in _read_golden("e4m3_format.txt") if r[0] != "code"}
    assert v[-1] == float(g["max_finite"][0]) and int(g["max_finite_code"][0], 16) == 0x7E
    assert v[1] == float(g["min_subnormal"][0]) and v[8] == float(g["min_normal"][0])
    assert np.count_nonzero(v > 0) == int(g["positive_finite_nonzero_count"][0])
    for r in _read_golden("e4m3_format.txt"):
        if r[0] == "code":
            got = F.e4m3_decode(np.array([int(r[1], 16)], dtype=np.uint8))[0]
            assert got == float(r[2]) and np.signbit(got) == np.signbit(float(r[2]))


def test_e4m3_decode_equals_torch_float8():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(F.e4m3_decode(codes), t)


def test_e4m3_encode_equals_torch_float8_in_finite_range():
    rng = np.random.default_rng(1)
    v = F.E4M3_VALUES
    mids = (v[1:] + v[:-1]) / 2
    xs = [np.float32(m) for m in mids]
    xs += [np.nextafter(np.float32(m), np.float32(0)) for m in mids]
    xs += [np.nextafter(np.float32(m), np.float32(1e9)) for m in mids]
    xs += list(rng.uniform(0, 448, 20000).astype(np.float32))
    xs += list((2.0 ** rng.uniform(-12, 8.8, 20000)).astype(np.float32))
    x = np.array(xs, dtype=np.float32)
    x = x[x <= 448]
    got = F.e4m3_encode(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_satfinite():
    x = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 1e30], dtype=np.float32)
    assert np.all(F.e4m3_encode(x) == 0x7E)
    assert F.e4m3_encode_signed(np.array([-1000.0, -0.0], dtype=np.float32)).tolist() == [0xFE, 0x80]


# ------------------------------------------------------------------------------ bf16 / fp16

def test_bf16_from_float32_equals_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(37.0)
    u = x.view(np.uint32).copy()
    u[:1000] = (u[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties
    x = u.view(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_rne(x), want)
    assert np.array_equal(synth.to_bf16_bits(x), want)


def test_bf16_from_float64_brute_force():
    rng = np.random.default_rng(3)
    for e in (-3, 0, 5, 20):
        x = rng.uniform(1, 2, 4000) * 2.0 ** e
        x[:50] = (1 + (2 * rng.integers(0, 128, 50) + 1) / 256.0) * 2.0 ** e   # exact ties
        grid = (1 + np.arange(129) / 128.0) * 2.0 ** e
        j = _brute_nearest_even(grid, x)
        want = grid[j]
        got = F.bf16_round_f32(x).astype(np.float64)
        assert np.array_equal(got, want)
        assert np.array_equal(F.bf16_round_f32(-x).astype(np.float64), -want)


def test_fp16_equals_torch_half():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-6, 4, 50000)).astype(np.float32)
    want = torch.from_numpy(x).half().numpy()
    assert np.array_equal(F.fp16_rne(x).view(np.uint16), want.view(np.uint16))


# ------------------------------------------------------------------------------ packing

def test_nibble_order_low_nibble_is_even_index():
    assert F.pack_nibbles(np.array([[1, 2, 3, 4]], dtype=np.uint8)).tolist() == [[0x21, 0x43]]
    rng = np.random.default_rng(5)
    n = rng.integers(0, 16, (7, 64)).astype(np.uint8)
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(n)), n)
