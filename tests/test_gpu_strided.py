"""GPU parity with padded leading dimensions: X, W and Y are views into wider buffers
(ldx = K + 256, ldw = K + 256, ldy = N + 256), so every kernel's row addressing runs with a row
stride different from the row length.  Codes and scales must be bit-exact to the oracle and Y
within the layer tolerance, exactly as with packed rows; the padding columns of Y must stay
untouched."""
import numpy as np
import pytest

import synth
from oracle import calib as OC, svd as OS, layer as OL, delta as DQ, score as SC
from tests.gpu_common import dev_bf16, host_bits, dev, check_y, check_d, torch_mod

pytestmark = pytest.mark.gpu
PAD = 256


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _padded(bits, pad=PAD, fill=0x7FC0):
    """Device bf16 view [rows, cols] into a [rows, cols + pad] buffer whose padding holds NaN
    patterns (a kernel that read the padding would poison its results)."""
    rows, cols = bits.shape
    buf = np.full((rows, cols + pad), fill, np.uint16)
    buf[:, :cols] = bits
    return dev_bf16(buf)[:, :cols]


@pytest.mark.parametrize("fmt", [0, 1, 2, 3], ids=["nvfp4", "int4", "mxfp4", "mxfp8"])
def test_padded_leading_dimensions_layer(L, fmt):
    torch = torch_mod()
    M, K, N, r = 333, 512, 512, 16
    cfg = dict(M=M, K=K, N=N, seg=synth.segments(M), gen="outlier")
    X, W = synth.x_bits(cfg, 21), synth.weight_bits(N, K, 21)
    name = {0: "nvfp4", 1: "int4", 2: "mxfp4", 3: "mxfp8"}[fmt]
    ax, aw, lam, amax = OC.calibrate(X, cfg["seg"], W, 7)
    down, up = OS.lowrank_factors(W, lam, r)
    wt = OL.prepare_weight(W, lam, down, up, name)
    act = OL.prepare_activation(X, lam, amax, down, name)
    _, y = OL.forward(act, wt, up, name)

    Xd, Wd = _padded(X), _padded(W)
    assert Xd.stride(0) == K + PAD and Wd.stride(0) == K + PAD
    cal = L.calibrate(Xd, cfg["seg"], Wd, 7)
    assert np.array_equal(cal["ax"].cpu().numpy(), ax)
    assert np.array_equal(cal["aw"].cpu().numpy(), aw)
    assert np.array_equal(cal["lambda"].cpu().numpy(), lam)
    assert cal["act_amax"].cpu().numpy()[0] == amax
    pw = L.prepare_weight(Wd, cal["lambda"], dev_bf16(down), dev_bf16(up), fmt)
    codes, scales, g, D = L.quantize_activation(Xd, cal["lambda"], cal["act_amax"],
                                                dev_bf16(down), fmt)
    Ybuf = torch.full((M, N + PAD), 3.0, dtype=torch.bfloat16, device="cuda")
    Y = L.gemm(codes, scales, g, D, pw, M, out=Ybuf[:, :N])
    torch.cuda.synchronize()
    assert np.array_equal(pw.codes.cpu().numpy(), wt["codes"])
    assert np.array_equal(codes.cpu().numpy(), act["codes"])
    sv = (lambda a: a.view(np.uint16)) if fmt == 1 else (lambda a: a)
    assert np.array_equal(sv(pw.scales.cpu().numpy()), sv(wt["scales"]))
    assert np.array_equal(sv(scales.cpu().numpy()), sv(act["scales"]))
    if fmt == 0:
        assert pw.g.cpu().numpy()[0] == wt["g"] and g.cpu().numpy()[0] == act["g"]
    check_d(D.cpu().numpy(), act["D"])
    check_y(host_bits(Y), y)
    assert torch.all(Ybuf[:, N:] == 3.0), "the GEMM wrote into the padding of Y"

    # scoring reads Y, X and W through their row strides as well
    rows, grp = synth.sample_rows(cfg["seg"], n_per=64, seed=5)
    want = SC.rel_l2(SC.modal_sums(y[rows], SC.reference_rows(X, W, rows), grp))
    from w4a4_quantized_dit_amd import _lib
    sums = torch.zeros(8, dtype=torch.float64, device="cuda")
    _lib.svdq_score_modal_rel_l2(Y, Xd, Wd, dev(rows), dev(grp), sums)
    got = SC.rel_l2(sums.cpu().numpy().reshape(4, 2))
    assert np.all(np.abs(got - want) <= 1e-4), (got, want)


def test_padded_leading_dimension_deltaquant(L):
    """DeltaQuant activations read X through its row stride (gathered cube members)."""
    torch = torch_mod()
    from w4a4_quantized_dit_amd import _lib
    T, H, Wg, nt, na = 5, 6, 7, 13, 9
    M, K, N, r = nt + T * H * Wg + na, 512, 256, 32
    cfg = dict(synth.config(4))
    cfg.update(grid=(T, H, Wg), n_text=nt, n_audio=na, K=K, N=N, r=r, M=M,
               seg=(0, nt, nt + T * H * Wg, M))
    X, W = synth.x_bits(cfg, 3), synth.weight_bits(N, K, 3)
    ax, aw, lam, amax = OC.calibrate(X, cfg["seg"], W, 7)
    down, up = OS.lowrank_factors(W, lam, r)
    r2c, ptr, crow = DQ.cube_geometry(T, H, Wg, 2, 2, 2, nt, na, 4)
    xhat = OC.smooth(X, lam)
    core = DQ.cube_core(xhat, ptr, crow)
    cc, cs = DQ.core_fp8(core)
    dc, dsc, gd, _ = DQ.delta_quantize(DQ.delta_rows(xhat, core, r2c), amax)
    from oracle import gemm as OG
    D_ref = OG.lowrank_down(xhat, down)

    Xd = _padded(X)
    geo = L.cube_geometry(T, H, Wg, 2, 2, 2, nt, na, 4)
    out = L.delta_quantize_activation(Xd, dev(lam), dev(np.array([amax], np.float32)), geo,
                                      dev_bf16(down))
    torch.cuda.synchronize()
    assert np.array_equal(out["cc"].cpu().numpy(), cc)
    assert np.array_equal(out["cs"].cpu().numpy(), cs)
    assert np.array_equal(out["dc"].cpu().numpy(), dc)
    assert np.array_equal(out["dsc"].cpu().numpy(), dsc)
    assert out["gd"].cpu().numpy()[0] == gd
    check_d(out["D"].cpu().numpy(), D_ref)
