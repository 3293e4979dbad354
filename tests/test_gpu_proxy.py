"""GPU parity of the bits-lost proxy ("MiniMax-H3 NVFP4 — what the smoothing scale should be
calibrated on", section "Why") against the oracle, on the GPU calibration statistics of seeded
synthetic batches: λ from all rows, video only, text only and none, in the three group sizes.
The proxy is a mean of float64 logarithms; the sums run in a different order on the two sides,
so the bar is a relative 1e-12 (the exact values are not defined beyond rounding order)."""
import numpy as np
import pytest

import synth
from oracle import proxy as OP
from tests.gpu_common import dev_bf16, dev, torch_mod

pytestmark = pytest.mark.gpu
REL = 1e-12


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _check(got, ref):
    got = got.cpu().numpy()
    assert np.all(np.abs(got - ref) <= REL * np.maximum(np.abs(ref), 1.0)), (got, ref)


@pytest.mark.parametrize("idx", [0, 1])
@pytest.mark.parametrize("mask", [7, 2, 1, 0])
def test_proxy_on_calibration_statistics(L, idx, mask):
    cfg = synth.config(idx)
    X, W = synth.x_bits(cfg), synth.weight_bits(cfg["N"], cfg["K"])
    cal = L.calibrate(dev_bf16(X), cfg["seg"], dev_bf16(W), mask)
    ax, lam = cal["ax"].cpu().numpy(), cal["lambda"].cpu().numpy()
    for block in (16, 32, 64):
        _check(L.bits_lost(cal["ax"], cal["lambda"], block), OP.bits_lost(ax, lam, block))
    _check(L.bits_lost(cal["ax"], None, 16), OP.bits_lost(ax, None, 16))
    print(f"[proxy] {cfg['name']} mask {mask}: {OP.bits_lost(ax, lam, 16)}", flush=True)


def test_proxy_degenerate_inputs(L):
    torch = torch_mod()
    K = 320
    ax = np.zeros((3, K), np.float32)
    ax[1, 5] = 3.0                                  # one live channel
    ax[2, :] = np.ldexp(np.float32(1), -(np.arange(K) % 16))   # halving ladders: 7.5 bits
    lam = np.ones(K, np.float32)
    lam[16:32] = 0.25                               # power-of-two λ on one group: no change
    got = L.bits_lost(dev(ax), dev(lam), 16)
    _check(got, OP.bits_lost(ax, lam, 16))
    assert got.cpu().numpy()[0] == 0.0
