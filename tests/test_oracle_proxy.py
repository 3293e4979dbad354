"""Pins of the oracle's bits-lost proxy ("MiniMax-H3 NVFP4 — what the smoothing scale should be
calibrated on", section "Why") against facts the definition fixes: closed forms, the channels
it leaves out, the invariances of a ratio inside a group, and the page's own qualitative claim
that dividing by a profile unrelated to a modality's own sharpens it."""
import numpy as np
import pytest

from oracle import proxy
from oracle import calib as OC

F32 = np.float32


def test_flat_groups_lose_nothing():
    ax = np.tile(np.repeat(np.array([0.5, 3.0, 7.25, 1e-3], F32), 16), (3, 1))
    assert np.array_equal(proxy.bits_lost(ax, None, 16), np.zeros(3))


def test_halving_ladder_has_the_closed_form_mean():
    # one group of 16 channels 2^0 .. 2^-15: channel j loses exactly j bits, mean 7.5
    g = np.ldexp(F32(1), -np.arange(16)).astype(F32)
    ax = np.stack([g, g[::-1], np.roll(g, 5)])
    assert np.array_equal(proxy.bits_lost(ax, None, 16), np.full(3, 7.5))
    # in blocks of 32 the second ladder half sits 16 bits under the first: mean 15.5
    ax2 = np.concatenate([g, np.ldexp(g, -16)]).astype(F32)[None, :].repeat(3, 0)
    assert np.array_equal(proxy.bits_lost(ax2, None, 32), np.full(3, 15.5))


def test_silent_channels_are_left_out():
    ax = np.zeros((3, 32), F32)
    ax[0, 3] = 2.0                       # a lone live channel: its own group max, 0 bits
    ax[1, 0], ax[1, 1] = 4.0, 1.0        # two live channels: 0 and 2 bits, mean 1
    out = proxy.bits_lost(ax, None, 16)
    assert out[0] == 0.0 and out[1] == 1.0 and out[2] == 0.0   # modality 2: no live channel


def test_power_of_two_scaling_of_a_group_changes_nothing():
    rng = np.random.default_rng(0)
    ax = np.exp(rng.normal(0, 1, (3, 128))).astype(F32)
    lam = np.repeat(np.ldexp(F32(1), rng.integers(-6, 7, 8)), 16).astype(F32)
    assert np.array_equal(proxy.bits_lost(ax, lam, 16), proxy.bits_lost(ax, None, 16))


def test_lambda_equal_to_a_profile_flattens_that_modality():
    rng = np.random.default_rng(1)
    ax = np.exp(rng.normal(0, 1, (3, 512))).astype(F32)
    out = proxy.bits_lost(ax, ax[1], 16)
    assert out[1] < 1e-6                  # c_k = fl(ax·fl(1/ax)) is 1 within an ulp or two
    assert out[0] > 0.5 and out[2] > 0.5


def test_uncorrelated_lambda_sharpens_the_other_modalities():
    # page 1 "Why": smoothing by a λ unrelated to a modality's own channel profile
    # sharpens it, while λ built from a modality's own statistics flattens that modality
    rng = np.random.default_rng(2)
    K = 4096
    ax = np.exp(0.75 * rng.normal(0, 1, (3, K))).astype(F32)
    aw = np.exp(0.1 * rng.normal(0, 1, K)).astype(F32)
    none = proxy.bits_lost(ax, None, 16)
    lam_video = OC.lambda_from_stats(ax, aw, 0b010, 0.5)
    under_video = proxy.bits_lost(ax, lam_video, 16)
    assert under_video[1] < none[1]                        # video flattened
    assert under_video[0] > none[0] and under_video[2] > none[2]   # text, audio sharpened


@pytest.mark.parametrize("block", [16, 32, 64])
def test_block_must_divide_k(block):
    with pytest.raises(ValueError):
        proxy.bits_lost(np.ones((3, block + 8), F32), None, block)
