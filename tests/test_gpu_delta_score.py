"""GPU parity of the per-modality scoring kernel and of the DeltaQuant path (cube geometry, FP8
cube-mean core, NVFP4 delta, core GEMM, delta GEMM with the core term) against the oracle,
including the lambda sweep and the DeltaQuant workload at full size."""
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


def _delta_case(cfg, seed=0, factors=None):
    """Oracle side of the DeltaQuant layer for a cube-field workload."""
    T, H, Wd = cfg["grid"]
    X = synth.x_bits(cfg, seed)
    W = synth.weight_bits(cfg["N"], cfg["K"], seed)
    ax, aw, lam, amax = OC.calibrate(X, cfg["seg"], W, 7)
    down, up = factors if factors is not None else OS.lowrank_factors(W, lam, cfg["r"])
    r2c, ptr, crow = DQ.cube_geometry(T, H, Wd, 2, 2, 2, cfg["n_text"], cfg["n_audio"], 4)
    xhat = OC.smooth(X, lam)
    core = DQ.cube_core(xhat, ptr, crow)
    cc, cs = DQ.core_fp8(core)
    d = DQ.delta_rows(xhat, core, r2c)
    dc, dsc, gd, sat = DQ.delta_quantize(d, amax)
    wt = OL.prepare_weight(W, lam, down, up, "nvfp4")
    co = DQ.core_out_f64(cc, cs, wt["codes"], wt["scales"], wt["g"])
    return dict(X=X, W=W, lam=lam, amax=amax, down=down, up=up, r2c=r2c, ptr=ptr, crow=crow,
                xhat=xhat, cc=cc, cs=cs, dc=dc, dsc=dsc, gd=gd, sat=sat, wt=wt, co=co)


def _gpu_delta(L, o, cfg):
    torch = torch_mod()
    from w4a4_quantized_dit_amd import _lib
    T, H, Wg = cfg["grid"]
    r2c, ptr, crow = _lib.svdq_cube_geometry(T, H, Wg, 2, 2, 2, cfg["n_text"], cfg["n_audio"], 4)
    M, K, N, r = cfg["M"], cfg["K"], cfg["N"], cfg["r"]
    nc = len(ptr) - 1
    Xd, Wd = dev_bf16(o["X"]), dev_bf16(o["W"])
    cal = L.calibrate(Xd, cfg["seg"], Wd, 7)
    pw = L.prepare_weight(Wd, cal["lambda"], dev_bf16(o["down"]), dev_bf16(o["up"]), 0)
    u8 = torch.uint8
    cc = torch.empty(nc, K, dtype=u8, device="cuda")
    cs = torch.empty(nc, device="cuda")
    dc = torch.empty(M, K // 2, dtype=u8, device="cuda")
    dsc = torch.empty(M, K // 16, dtype=u8, device="cuda")
    gd = torch.empty(1, device="cuda")
    D = torch.empty(M, r, device="cuda")
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    _lib.svdq_delta_quant_act(Xd, cal["lambda"], cal["act_amax"], dev(ptr), dev(crow), nc,
                              dev_bf16(o["down"]), r, cc, cs, dc, dsc, gd, D, sat)
    co = torch.empty(nc, N, device="cuda")
    _lib.svdq_gemm_core(nc, N, K, cc, cs, pw.codes, pw.scales, pw.g, co)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    _lib.svdq_w4a4_gemm(0, M, N, K, dc, dsc, gd, pw.codes, pw.scales, pw.g, D, pw.lora_up, r, Y,
                        core_out=co, row_to_cube=dev(r2c))
    torch.cuda.synchronize()
    return dict(geo=(r2c, ptr, crow), cal=cal, cc=cc, cs=cs, dc=dc, dsc=dsc, gd=gd, D=D, sat=sat,
                co=co, Y=Y)


def _compare_delta(o, g, rows):
    for a, b in zip(g["geo"], (o["r2c"], o["ptr"], o["crow"])):
        assert np.array_equal(a, b)
    assert np.array_equal(g["cal"]["lambda"].cpu().numpy(), o["lam"])
    assert np.array_equal(g["cs"].cpu().numpy(), o["cs"])
    assert np.array_equal(g["cc"].cpu().numpy(), o["cc"])
    assert g["gd"].cpu().numpy()[0] == o["gd"]
    assert int(g["sat"].cpu()[0]) == o["sat"] == 0
    assert np.array_equal(g["dc"].cpu().numpy(), o["dc"])
    assert np.array_equal(g["dsc"].cpu().numpy(), o["dsc"])
    co = g["co"].cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(co - o["co"]) / np.linalg.norm(o["co"])
    assert rel <= CORE_OUT_REL_L2, rel
    D_rows = OG.lowrank_down(o["xhat"][rows], o["down"])
    check_d(g["D"].cpu().numpy()[rows], D_rows)
    D_full = np.zeros((o["xhat"].shape[0], o["down"].shape[0]))
    D_full[rows] = D_rows          # only the sampled rows are read below
    _, y = DQ.delta_linear(o["co"], o["r2c"], o["dc"], o["dsc"], o["gd"], o["wt"]["codes"],
                           o["wt"]["scales"], o["wt"]["g"], D_full, o["up"], rows=rows)
    return check_y(host_bits(g["Y"])[rows], y)


def test_deltaquant_small_grid(L):
    cfg = dict(synth.config(4))
    cfg.update(grid=(5, 6, 7), n_text=13, n_audio=9, K=512, N=256, r=32)
    cfg["M"] = 13 + 5 * 6 * 7 + 9
    cfg["seg"] = (0, 13, 13 + 210, cfg["M"])
    o = _delta_case(cfg)
    g = _gpu_delta(L, o, cfg)
    rows = np.arange(cfg["M"])
    print(f"deltaquant small rel-L2 {_compare_delta(o, g, rows):.2e}")


def test_deltaquant_full_size(L):
    """The DeltaQuant workload: 31x24x42 video grid (prime T, ragged edge cubes), 312 text and
    128 audio rows in 1-D cubes, K = N = 5120, rank 128."""
    cfg = synth.config(4)
    print(f"[delta] {cfg['name']}", flush=True)
    o = _delta_case(cfg)
    g = _gpu_delta(L, o, cfg)
    M = cfg["M"]
    rows = np.array(sorted(set(range(0, M, 97)) | set(range(0, 312)) | set(range(M - 128, M))
                           | set(range(312 + 30 * 24 * 42, 312 + 30 * 24 * 42 + 50))))
    print(f"[delta] {len(rows)} sampled rows rel-L2 {_compare_delta(o, g, rows):.2e}", flush=True)
