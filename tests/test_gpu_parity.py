"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on seeded inputs.

Bit-exact: calibration maxima, λ, act_amax, every code and scale, the tensor scales, the
saturation counts.  Within tolerance: D and Y (see gpu_common)."""
import numpy as np
import pytest

import synth
from oracle import quant as OQ, calib as OC
from oracle.formats import bf16_bits_to_f32, pack_nibbles
from tests.gpu_common import (dev_bf16, host_bits, dev, check_y, check_d, oracle_case,
                              torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _outlier_inputs(M, K, N, seg=None, seed=0):
    cfg = dict(M=M, K=K, N=N, seg=seg or synth.segments(M), gen="outlier")
    return synth.x_bits(cfg, seed), synth.weight_bits(N, K, seed), cfg["seg"]


def _run_gpu(L, X, seg, W, mask, fmt, down, up, alpha=0.5, static=True):
    torch = torch_mod()
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    cal = L.calibrate(Xd, seg, Wd, mask, alpha)
    r = down.shape[0]
    downd = dev_bf16(down) if r else None
    upd = dev_bf16(up) if r else None
    pw = L.prepare_weight(Wd, cal["lambda"], downd, upd, fmt)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    codes, scales, g, D = L.quantize_activation(Xd, cal["lambda"], cal["act_amax"] if static else None,
                                                downd, fmt, sat_count=sat)
    Y = L.gemm(codes, scales, g, D, pw, X.shape[0])
    torch.cuda.synchronize()
    return dict(cal=cal, pw=pw, codes=codes, scales=scales, g=g, D=D, Y=Y, sat=sat)


def _compare(o, gpu, fmt):
    c = gpu["cal"]
    assert np.array_equal(c["ax"].cpu().numpy(), o["ax"])
    assert np.array_equal(c["aw"].cpu().numpy(), o["aw"])
    assert np.array_equal(c["lambda"].cpu().numpy(), o["lam"])
    assert c["act_amax"].cpu().numpy()[0] == o["amax"]
    pw = gpu["pw"]
    assert np.array_equal(pw.codes.cpu().numpy(), o["wt"]["codes"])
    if fmt == 0:
        assert np.array_equal(pw.scales.cpu().numpy(), o["wt"]["scales"])
        assert pw.g.cpu().numpy()[0] == o["wt"]["g"]
        assert gpu["g"].cpu().numpy()[0] == o["act"]["g"]
        assert int(gpu["sat"].cpu().numpy()[0]) == o["act"]["n_sat"]
    else:
        assert np.array_equal(pw.scales.cpu().numpy().view(np.uint16),
                              o["wt"]["scales"].view(np.uint16))
    assert np.array_equal(gpu["codes"].cpu().numpy(), o["act"]["codes"])
    if fmt == 0:
        assert np.array_equal(gpu["scales"].cpu().numpy(), o["act"]["scales"])
    else:
        assert np.array_equal(gpu["scales"].cpu().numpy().view(np.uint16),
                              o["act"]["scales"].view(np.uint16))
    if gpu["D"] is not None:
        check_d(gpu["D"].cpu().numpy(), o["act"]["D"])
    return check_y(host_bits(gpu["Y"]), o["y"])


@pytest.mark.parametrize("fmt", [0, 1])
def test_tiny_workload_end_to_end(L, fmt):
    cfg = synth.config(0)
    X, W = synth.x_bits(cfg), synth.weight_bits(cfg["N"], cfg["K"])
    o = oracle_case(X, cfg["seg"], W, 7, cfg["r"], "nvfp4" if fmt == 0 else "int4")
    gpu = _run_gpu(L, X, cfg["seg"], W, 7, fmt, o["down"], o["up"])
    print(f"tiny fmt={fmt} rel-L2 {_compare(o, gpu, fmt):.2e}")


@pytest.mark.parametrize("fmt,M,K,N,r,mask", [
    (0, 333, 512, 512, 16, 7),      # ragged M over several tiles
    (1, 333, 512, 512, 16, 7),
    (0, 1, 256, 256, 8, 2),         # a single row (video only)
    (0, 517, 768, 256, 0, 0),       # plain W4A4: no low-rank branch, λ = 1
    (1, 260, 256, 768, 128, 1),     # rank 128, text-only λ
    (0, 700, 1024, 512, 40, 4),     # rank not a multiple of 16, audio-only λ
])
def test_shapes_ranks_masks(L, fmt, M, K, N, r, mask):
    X, W, seg = _outlier_inputs(M, K, N, seed=M + K)
    o = oracle_case(X, seg, W, mask, r, "nvfp4" if fmt == 0 else "int4")
    gpu = _run_gpu(L, X, seg, W, mask, fmt, o["down"], o["up"])
    _compare(o, gpu, fmt)


def test_dynamic_amax_equals_static_on_calibration_rows(L):
    X, W, seg = _outlier_inputs(300, 512, 256, seed=3)
    o = oracle_case(X, seg, W, 7, 16, "nvfp4")
    st = _run_gpu(L, X, seg, W, 7, 0, o["down"], o["up"], static=True)
    dy = _run_gpu(L, X, seg, W, 7, 0, o["down"], o["up"], static=False)
    assert np.array_equal(st["codes"].cpu().numpy(), dy["codes"].cpu().numpy())
    assert np.array_equal(st["scales"].cpu().numpy(), dy["scales"].cpu().numpy())
    assert st["g"].cpu().numpy()[0] == dy["g"].cpu().numpy()[0]


def test_saturation_count_with_small_static_amax(L):
    torch = torch_mod()
    X, W, seg = _outlier_inputs(128, 256, 256, seed=4)
    lam = np.ones(256, np.float32)
    amax = np.float32(np.abs(bf16_bits_to_f32(X)).max() / 8)
    xhat = OC.smooth(X, lam)
    codes, scales, g, n_sat = OQ.nvfp4_quantize(xhat, amax)
    assert n_sat > 0
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    c, s, gg, _ = L.quantize_activation(dev_bf16(X), dev(lam), dev(np.array([amax], np.float32)),
                                        None, 0, sat_count=sat)
    assert np.array_equal(c.cpu().numpy(), codes) and np.array_equal(s.cpu().numpy(), scales)
    assert int(sat.cpu()[0]) == n_sat


def test_calibration_accumulates_over_batches(L):
    X, W, seg = _outlier_inputs(400, 512, 256, seed=5)
    a, b = X[:150], X[150:]
    sa = (0, 4, 150, 150)
    sb = (0, 0, 398 - 150, 250)
    Xd = dev_bf16(X)
    st = L.calibrate(dev_bf16(a), sa, dev_bf16(W), 7)
    st = L.calibrate(dev_bf16(b), sb, dev_bf16(W), 7, state=st)
    ax = np.maximum(OC.channel_absmax_per_modality(a, sa), OC.channel_absmax_per_modality(b, sb))
    aw = OC.weight_absmax(W)
    lam = OC.lambda_from_stats(ax, aw, 7)
    assert np.array_equal(st["ax"].cpu().numpy(), ax)
    assert np.array_equal(st["lambda"].cpu().numpy(), lam)
    assert st["act_amax"].cpu().numpy()[0] == OC.act_amax_from_stats(ax, lam)
    del Xd


def test_general_alpha_within_one_ulp(L):
    X, W, seg = _outlier_inputs(200, 256, 256, seed=6)
    cal = L.calibrate(dev_bf16(X), seg, dev_bf16(W), 7, alpha=0.3)
    _, _, lam, _ = OC.calibrate(X, seg, W, 7, alpha=0.3)
    got = cal["lambda"].cpu().numpy()
    ulp = np.abs(got.view(np.int32).astype(np.int64) - lam.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1


def test_calibration_without_weight_gives_unit_aw(L):
    X, W, seg = _outlier_inputs(100, 256, 256, seed=7)
    cal = L.calibrate(dev_bf16(X), seg, None, 7)
    ax, aw, lam, amax = OC.calibrate(X, seg, None, 7)
    assert np.all(cal["aw"].cpu().numpy() == 1.0)
    assert np.array_equal(cal["lambda"].cpu().numpy(), lam)


def test_integer_exact_gemm_is_bit_exact(L):
    torch = torch_mod()
    from w4a4_quantized_dit_amd import _lib
    from oracle import gemm as OG
    rng = np.random.default_rng(8)
    M, N, K = 300, 512, 1024
    an = rng.integers(0, 16, (M, K)).astype(np.uint8)
    wn = rng.integers(0, 16, (N, K)).astype(np.uint8)
    ac, wc = pack_nibbles(an), pack_nibbles(wn)
    a_s = np.full((M, K // 16), 0x38, np.uint8)
    w_s = np.full((N, K // 16), 0x38, np.uint8)
    one = np.ones(1, np.float32)
    y64, y = OG.linear_nvfp4(ac, a_s, np.float32(1), wc, w_s, np.float32(1),
                             np.zeros((M, 0), np.uint16), np.zeros((N, 0), np.uint16))
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    _lib.svdq_w4a4_gemm(0, M, N, K, dev(ac), dev(a_s), dev(one), dev(wc), dev(w_s), dev(one),
                        None, None, 0, Y)
    assert np.array_equal(host_bits(Y), y)


def test_repeat_runs_are_bitwise_identical(L):
    X, W, seg = _outlier_inputs(333, 512, 512, seed=9)
    o = oracle_case(X, seg, W, 7, 16, "nvfp4")
    g1 = _run_gpu(L, X, seg, W, 7, 0, o["down"], o["up"])
    g2 = _run_gpu(L, X, seg, W, 7, 0, o["down"], o["up"])
    assert np.array_equal(host_bits(g1["Y"]), host_bits(g2["Y"]))
    assert np.array_equal(g1["D"].cpu().numpy(), g2["D"].cpu().numpy())


def test_mispermuted_lambda_fails_parity(L):
    """A λ written in another channel order must break code parity (the pages' pitfall of a
    smoothing factor addressed in a different channel order)."""
    torch = torch_mod()
    X, W, seg = _outlier_inputs(128, 512, 256, seed=10)
    o = oracle_case(X, seg, W, 7, 16, "nvfp4")
    perm = np.arange(512).reshape(-1, 16)[:, [0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15]]
    lam_bad = o["lam"][perm.reshape(-1)]
    c, s, g, D = L.quantize_activation(dev_bf16(X), dev(lam_bad), dev(np.array([o["amax"]])),
                                       dev_bf16(o["down"]), 0)
    assert not np.array_equal(c.cpu().numpy(), o["act"]["codes"])


@pytest.mark.parametrize("fmt,N,K,r", [(0, 768, 1024, 32), (0, 300, 512, 0), (0, 256, 256, 8),
                                       (1, 300, 512, 16), (3, 256, 512, 8)])
def test_quantize_weight_with_workspace_matches(L, fmt, N, K, r):
    """svdq_quantize_weight_ws (the NVFP4 residual formed once, kept in the workspace and read
    back by the quantising pass) gives the codes, scales and tensor scale of
    svdq_quantize_weight bit for bit, and the oracle's; twice in a row, the second on a smaller
    weight through the same workspace."""
    from oracle import layer as OL
    names = {0: "nvfp4", 1: "int4", 2: "mxfp4", 3: "mxfp8"}
    ws = L.quantize_weight_workspace(N, K, fmt)
    for n in (N, N // 2):
        rng = np.random.default_rng(n)
        W = synth.weight_bits(n, K, 11)
        lam = (rng.random(K).astype(np.float32) + 0.5)
        down = synth.weight_bits(r, K, 12) if r else np.zeros((0, K), np.uint16)
        up = synth.weight_bits(n, r, 13) if r else np.zeros((n, 0), np.uint16)
        args = (dev_bf16(W), dev(lam), dev_bf16(down) if r else None, dev_bf16(up) if r else None)
        a = L.prepare_weight(*args, fmt)
        b = L.prepare_weight(*args, fmt, workspace=ws)
        ref = OL.prepare_weight(W, lam, down, up, names[fmt])
        for pw in (a, b):
            assert np.array_equal(pw.codes.cpu().numpy(), ref["codes"])
            assert np.array_equal(pw.scales.cpu().numpy().view(np.uint8),
                                  np.asarray(ref["scales"]).view(np.uint8))
            if fmt == 0:
                assert pw.g.cpu().numpy()[0] == ref["g"]
