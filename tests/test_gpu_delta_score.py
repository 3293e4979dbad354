"""GPU parity of the per-modality scoring kernel against the oracle, including the λ sweep of
the MLP down-projection at full size."""
import numpy as np
import pytest

import synth
from oracle import calib as OC, svd as OS, layer as OL, delta as DQ, score as SC, gemm as OG
from oracle.formats import bf16_bits_to_f32
from tests.gpu_common import dev_bf16, host_bits, dev, check_y, check_d, torch_mod

pytestmark = pytest.mark.gpu
SCORE_ABS = 1e-4
CORE_OUT_REL_L2 = 1e-5


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _gpu_layer(L, Xd, seg, Wd, mask, down, up, fmt=0):
    cal = L.calibrate(Xd, seg, Wd, mask)
    r = down.shape[0]
    pw = L.prepare_weight(Wd, cal["lambda"], dev_bf16(down) if r else None,
                          dev_bf16(up) if r else None, fmt)
    codes, scales, g, D = L.quantize_activation(Xd, cal["lambda"], cal["act_amax"],
                                                dev_bf16(down) if r else None, fmt)
    Y = L.gemm(codes, scales, g, D, pw, Xd.shape[0])
    return cal, pw, codes, scales, g, D, Y


def _gpu_scores(Y, Xd, Wd, rows, grp):
    torch = torch_mod()
    from w4a4_quantized_dit_amd import _lib
    sums = torch.zeros(8, dtype=torch.float64, device="cuda")
    _lib.svdq_score_modal_rel_l2(Y, Xd, Wd, dev(rows), dev(grp), sums)
    return sums.cpu().numpy().reshape(4, 2)


def test_score_kernel_on_oracle_output(L):
    """The scoring kernel fed the oracle's own layer output reproduces the oracle's sums."""
    torch = torch_mod()
    M, K, N = 700, 512, 512
    cfg = dict(M=M, K=K, N=N, seg=synth.segments(M, 40, 30), gen="outlier")
    X, W = synth.x_bits(cfg, 11), synth.weight_bits(N, K, 11)
    ax, aw, lam, amax = OC.calibrate(X, cfg["seg"], W, 7)
    down, up = OS.lowrank_factors(W, lam, 16)
    act = OL.prepare_activation(X, lam, amax, down, "nvfp4")
    wt = OL.prepare_weight(W, lam, down, up, "nvfp4")
    _, y = OL.forward(act, wt, up, "nvfp4")
    rows, grp = synth.sample_rows(cfg["seg"], n_per=100, seed=3)
    want = SC.modal_sums(y[rows], SC.reference_rows(X, W, rows), grp)
    Yd = torch.from_numpy(y.view(np.int16)).cuda().view(torch.bfloat16)
    got = _gpu_scores(Yd, dev_bf16(X), dev_bf16(W), rows, grp)
    assert np.allclose(got, want, rtol=2e-3, atol=0)
    assert np.all(np.abs(SC.rel_l2(got) - SC.rel_l2(want)) <= SCORE_ABS)


def test_two_part_scoring_matches_fused_and_oracle(L):
    """Reference rows stored once, then sums against them (what a multi-λ sweep runs): the
    stored rows are the oracle's bf16(X·Wᵀ) rows to within one bf16 rounding, the sums equal the
    fused kernel's (same per-element terms, fp64 in another order), and the rel-L2 scores equal
    the oracle's.  Y, X, W and the reference rows are row-strided views."""
    torch = torch_mod()
    from w4a4_quantized_dit_amd import _lib
    M, K, N = 700, 768, 512
    cfg = dict(M=M, K=K, N=N, seg=synth.segments(M, 40, 30), gen="outlier")
    X, W = synth.x_bits(cfg, 13), synth.weight_bits(N, K, 13)
    ax, aw, lam, amax = OC.calibrate(X, cfg["seg"], W, 7)
    down, up = OS.lowrank_factors(W, lam, 16)
    act = OL.prepare_activation(X, lam, amax, down, "nvfp4")
    wt = OL.prepare_weight(W, lam, down, up, "nvfp4")
    _, y = OL.forward(act, wt, up, "nvfp4")
    rows, grp = synth.sample_rows(cfg["seg"], n_per=100, seed=5)
    ref_want = SC.reference_rows(X, W, rows)

    def padded(bits, pad=64):
        buf = np.zeros((bits.shape[0], bits.shape[1] + pad), np.uint16)
        buf[:, :bits.shape[1]] = bits
        return dev_bf16(buf)[:, :bits.shape[1]]

    Xd, Wd, Yd = padded(X), padded(W), padded(y)
    Yref = torch.zeros(len(rows), N + 128, dtype=torch.bfloat16, device="cuda")[:, :N]
    _lib.svdq_score_reference_rows(Xd, Wd, dev(rows), Yref)
    got_ref = bf16_bits_to_f32(host_bits(Yref)).astype(np.float64)
    want_ref = bf16_bits_to_f32(ref_want).astype(np.float64)
    rms = np.sqrt(np.mean(want_ref ** 2))
    assert np.all(np.abs(got_ref - want_ref) <= 2.0 ** -7 * np.abs(want_ref) + 1e-6 * rms)
    assert np.mean(got_ref == want_ref) > 0.99

    sums = torch.zeros(8, dtype=torch.float64, device="cuda")
    _lib.svdq_score_modal_rel_l2_ref(Yd, Yref, dev(rows), dev(grp), sums)
    two_part = sums.cpu().numpy().reshape(4, 2)
    fused = _gpu_scores(Yd, Xd, Wd, rows, grp)
    assert np.allclose(two_part, fused, rtol=1e-9, atol=0)
    want = SC.modal_sums(y[rows], ref_want, grp)
    assert np.allclose(two_part, want, rtol=2e-3, atol=0)
    assert np.all(np.abs(SC.rel_l2(two_part) - SC.rel_l2(want)) <= SCORE_ABS)


def test_score_end_to_end_small(L):
    M, K, N = 900, 768, 512
    cfg = dict(M=M, K=K, N=N, seg=synth.segments(M, 30, 20), gen="outlier")
    X, W = synth.x_bits(cfg, 12), synth.weight_bits(N, K, 12)
    rows, grp = synth.sample_rows(cfg["seg"], n_per=200, seed=4)
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    for mask in (0, 7, 2, 1):
        ax, aw, lam, amax = OC.calibrate(X, cfg["seg"], W, mask)
        down, up = OS.lowrank_factors(W, lam, 16)
        wt = OL.prepare_weight(W, lam, down, up, "nvfp4")
        act = OL.prepare_activation(X[rows], lam, amax, down, "nvfp4")
        _, y = OL.forward(act, wt, up, "nvfp4")
        want = SC.rel_l2(SC.modal_sums(y, SC.reference_rows(X, W, rows), grp))
        *_, Y = _gpu_layer(L, Xd, cfg["seg"], Wd, mask, down, up)
        got = SC.rel_l2(_gpu_scores(Y, Xd, Wd, rows, grp))
        assert np.all(np.abs(got - want) <= SCORE_ABS), (mask, got, want)


@pytest.fixture(scope="module")
def sweep_inputs():
    cfg = synth.config(3)
    print(f"[sweep] generating {cfg['name']}", flush=True)
    X = synth.x_bits(cfg)
    W = synth.weight_bits(cfg["N"], cfg["K"])
    ax = OC.channel_absmax_per_modality(X, cfg["seg"])
    aw = OC.weight_absmax(W)
    rows, grp = synth.sample_rows(cfg["seg"], n_per=4096, seed=0)
    return dict(cfg=cfg, X=X, W=W, ax=ax, aw=aw, rows=rows, grp=grp, results={})


@pytest.mark.parametrize("mask", [0, 7, 2, 1], ids=["lambda1", "all", "video", "text"])
def test_lambda_sweep_full_size(L, sweep_inputs, mask):
    """The lambda calibration sweep at full size (M=65536, K=13824, N=5120, rank 32, NVFP4):
    calibration bit-exact, codes bit-exact on the sampled rows, Y within tolerance, and the
    per-modality scores of the GPU path within 1e-4 of the oracle's."""
    s = sweep_inputs
    cfg, X, W, rows, grp = s["cfg"], s["X"], s["W"], s["rows"], s["grp"]
    lam = OC.lambda_from_stats(s["ax"], s["aw"], mask)
    amax = OC.act_amax_from_stats(s["ax"], lam)
    down, up = OS.lowrank_factors(W, lam, cfg["r"])
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    cal, pw, codes, scales, g, D, Y = _gpu_layer(L, Xd, cfg["seg"], Wd, mask, down, up)
    assert np.array_equal(cal["lambda"].cpu().numpy(), lam)
    assert cal["act_amax"].cpu().numpy()[0] == amax
    wt = OL.prepare_weight(W, lam, down, up, "nvfp4")
    assert np.array_equal(pw.codes.cpu().numpy(), wt["codes"])
    act = OL.prepare_activation(X[rows], lam, amax, down, "nvfp4")
    assert np.array_equal(codes.cpu().numpy()[rows], act["codes"])
    assert np.array_equal(scales.cpu().numpy()[rows], act["scales"])
    check_d(D.cpu().numpy()[rows], act["D"])
    _, y = OL.forward(act, wt, up, "nvfp4")
    check_y(host_bits(Y)[rows], y)
    want = SC.rel_l2(SC.modal_sums(y, SC.reference_rows(X, W, rows), grp))
    got = SC.rel_l2(_gpu_scores(Y, Xd, Wd, rows, grp))
    s["results"][mask] = got
    print(f"[sweep] mask={mask} rel-L2 text/video/audio/uniform = "
          + " ".join(f"{v:.4f}" for v in got), flush=True)
    assert np.all(np.abs(got - want) <= SCORE_ABS), (got, want)
