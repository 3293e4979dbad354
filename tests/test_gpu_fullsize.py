"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Whole tensors are compared where the oracle computes them in seconds (calibration, every weight
code and scale, every activation code and scale); the layer output and D are compared on a row
sample (every 64th row plus all text and audio rows and the last rows)."""
import numpy as np
import pytest

import synth
from oracle import calib as OC, svd as OS, layer as OL
from tests.gpu_common import dev_bf16, host_bits, check_y, check_d, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _sample_rows(seg):
    M = seg[3]
    rows = set(range(0, M, 64)) | set(range(seg[0], seg[1])) | set(range(seg[2], seg[3]))
    rows |= set(range(max(0, M - 5), M))
    return np.array(sorted(rows))


@pytest.mark.parametrize("idx", [1, 2])
def test_full_workload(L, idx):
    torch = torch_mod()
    cfg = synth.config(idx)
    fmt = "nvfp4" if cfg["fmt"] == "nvfp4" else "int4"
    f = 0 if fmt == "nvfp4" else 1
    M, K, N, r, seg = cfg["M"], cfg["K"], cfg["N"], cfg["r"], cfg["seg"]
    print(f"[fullsize] {cfg['name']}", flush=True)
    X = synth.x_bits(cfg)
    W = synth.weight_bits(N, K)
    ax, aw, lam, amax = OC.calibrate(X, seg, W, 7)
    down, up = OS.lowrank_factors(W, lam, r)

    Xd, Wd = dev_bf16(X), dev_bf16(W)
    cal = L.calibrate(Xd, seg, Wd, 7)
    pw = L.prepare_weight(Wd, cal["lambda"], dev_bf16(down), dev_bf16(up), f)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    codes, scales, g, D = L.quantize_activation(Xd, cal["lambda"], cal["act_amax"], dev_bf16(down),
                                                f, sat_count=sat)
    Y = L.gemm(codes, scales, g, D, pw, M)
    torch.cuda.synchronize()

    assert np.array_equal(cal["ax"].cpu().numpy(), ax)
    assert np.array_equal(cal["aw"].cpu().numpy(), aw)
    assert np.array_equal(cal["lambda"].cpu().numpy(), lam)
    assert cal["act_amax"].cpu().numpy()[0] == amax

    wt = OL.prepare_weight(W, lam, down, up, fmt)
    assert np.array_equal(pw.codes.cpu().numpy(), wt["codes"])
    sv = pw.scales.cpu().numpy()
    assert np.array_equal(sv.view(np.uint8), np.asarray(wt["scales"]).view(np.uint8))
    if f == 0:
        assert pw.g.cpu().numpy()[0] == wt["g"]

    # all activation codes and scales, in row blocks to bound host memory
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    n_sat = 0
    for r0 in range(0, M, 4096):
        act = OL.prepare_activation(X[r0:r0 + 4096], lam, amax, down[:0], fmt)
        assert np.array_equal(gc[r0:r0 + 4096], act["codes"]), r0
        assert np.array_equal(gs[r0:r0 + 4096].view(np.uint8),
                              np.asarray(act["scales"]).view(np.uint8)), r0
        n_sat += act["n_sat"]
    if f == 0:
        assert int(sat.cpu()[0]) == n_sat
        assert g.cpu().numpy()[0] == OL.prepare_activation(X[:16], lam, amax, down[:0], fmt)["g"]

    rows = _sample_rows(seg)
    act = OL.prepare_activation(X[rows], lam, amax, down, fmt)
    check_d(D.cpu().numpy()[rows], act["D"])
    _, y = OL.forward(act, wt, up, fmt)
    rel = check_y(host_bits(Y)[rows], y)
    print(f"[fullsize] {cfg['name']}: {len(rows)} sampled rows, rel-L2 {rel:.2e}", flush=True)
