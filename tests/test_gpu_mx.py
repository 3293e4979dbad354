"""GPU parity of the MX variant (E8M0 scale per 32; MXFP4 W4A4 and MXFP8 W8A8 on the hardware
block-scaled MFMA) against the oracle ("MiniMax-H3 — MXFP8 (weight-quantized, vLLM-Omni native
layout)", section "Quant format").  Bit-exact: every weight and activation code and scale.  Within
tolerance: D and Y (see gpu_common).  Small ragged shapes, then the 5120x5120, M=16384 attention
projection in both formats on a row sample."""
import numpy as np
import pytest

import synth
from oracle import calib as OC, svd as OS, layer as OL
from tests.gpu_common import dev_bf16, host_bits, check_y, check_d, oracle_case, torch_mod

pytestmark = pytest.mark.gpu

FMTS = {2: "mxfp4", 3: "mxfp8"}


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _run(L, X, seg, W, mask, f, down, up):
    torch = torch_mod()
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    cal = L.calibrate(Xd, seg, Wd, mask)
    r = down.shape[0]
    pw = L.prepare_weight(Wd, cal["lambda"], dev_bf16(down) if r else None,
                          dev_bf16(up) if r else None, f)
    codes, scales, g, D = L.quantize_activation(Xd, cal["lambda"], None, dev_bf16(down) if r else None, f)
    Y = L.gemm(codes, scales, g, D, pw, X.shape[0])
    torch.cuda.synchronize()
    return pw, codes, scales, D, Y


@pytest.mark.parametrize("f", [2, 3])
@pytest.mark.parametrize("M,K,N,r,mask", [
    (333, 512, 512, 16, 7),      # ragged M over several tiles
    (1, 256, 256, 8, 2),         # a single row
    (517, 768, 256, 0, 0),       # no low-rank branch, λ = 1
    (260, 256, 768, 128, 1),     # rank 128
    (100, 1280, 256, 8, 7),      # K stages not a multiple of the scale fetch (5 of MXFP4, 10 of MXFP8)
])
def test_mx_shapes(L, f, M, K, N, r, mask):
    cfg = dict(M=M, K=K, N=N, seg=synth.segments(M), gen="outlier")
    X, W, seg = synth.x_bits(cfg, 0), synth.weight_bits(N, K, 0), cfg["seg"]
    o = oracle_case(X, seg, W, mask, r, FMTS[f])
    pw, codes, scales, D, Y = _run(L, X, seg, W, mask, f, o["down"], o["up"])
    assert np.array_equal(pw.codes.cpu().numpy(), o["wt"]["codes"])
    assert np.array_equal(pw.scales.cpu().numpy(), o["wt"]["scales"])
    assert np.array_equal(codes.cpu().numpy(), o["act"]["codes"])
    assert np.array_equal(scales.cpu().numpy(), o["act"]["scales"])
    if r:
        check_d(D.cpu().numpy(), o["act"]["D"])
    rel = check_y(host_bits(Y), o["y"])
    print(f"[mx] fmt={FMTS[f]} M={M} K={K} N={N} r={r}: rel-L2 {rel:.2e}", flush=True)


@pytest.mark.parametrize("f", [2, 3])
def test_mx_full_attention_projection(L, f):
    cfg = synth.config(1)
    M, K, N, r, seg = cfg["M"], cfg["K"], cfg["N"], cfg["r"], cfg["seg"]
    print(f"[mx-full] {FMTS[f]} {cfg['name']}", flush=True)
    X, W = synth.x_bits(cfg), synth.weight_bits(N, K)
    ax, aw, lam, amax = OC.calibrate(X, seg, W, 7)
    down, up = OS.lowrank_factors(W, lam, r)
    pw, codes, scales, D, Y = _run(L, X, seg, W, 7, f, down, up)
    wt = OL.prepare_weight(W, lam, down, up, FMTS[f])
    assert np.array_equal(pw.codes.cpu().numpy(), wt["codes"])
    assert np.array_equal(pw.scales.cpu().numpy(), wt["scales"])
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    for r0 in range(0, M, 4096):
        act = OL.prepare_activation(X[r0:r0 + 4096], lam, amax, down, FMTS[f])
        assert np.array_equal(gc[r0:r0 + 4096], act["codes"]), r0
        assert np.array_equal(gs[r0:r0 + 4096], act["scales"]), r0
    rows = np.array(sorted(set(range(0, M, 64)) | set(range(seg[0], seg[1]))
                           | set(range(seg[2], seg[3])) | set(range(M - 5, M))))
    act = OL.prepare_activation(X[rows], lam, amax, down, FMTS[f])
    check_d(D.cpu().numpy()[rows], act["D"])
    _, y = OL.forward(act, wt, up, FMTS[f])
    rel = check_y(host_bits(Y)[rows], y)
    print(f"[mx-full] {FMTS[f]}: {len(rows)} sampled rows, rel-L2 {rel:.2e}", flush=True)


def test_mxfp8_codes_at_every_e4m3_midpoint(L):
    """MXFP8 activation codes at the inputs where an E4M3 encoder can go wrong: every midpoint
    between neighbouring E4M3 values (a tie, to even), the bf16 values on either side of it, the
    subnormal range, and values past 448 that must saturate (the kernels' conversion turns those
    into NaN unless clamped first).  Each 32-block holds 448 (block exponent 0, so the elements
    are converted unscaled) and 31 such values; codes and scales bit-exact against the oracle."""
    torch = torch_mod()
    from oracle import mx as OM
    from oracle.formats import bf16_bits_to_f32
    vals = []
    def dec(c):
        e, m = (c >> 3) & 15, c & 7
        return m / 512.0 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    for c in range(0x7E):
        mid = np.float32(0.5 * (dec(c) + dec(c + 1)))
        b = int(np.array([mid], np.float32).view(np.uint32)[0] >> 16)
        vals += [b, b - 1, b + 1]                 # the midpoint (exact in bf16) and its neighbours
    over = np.array([448.5, 456, 463.9, 464, 464.1, 472, 480, 496, 504, 511], np.float32)
    vals += list((over.view(np.uint32) >> 16).astype(int))
    vals = np.array(vals, np.uint16)
    vals = np.concatenate([vals, vals | 0x8000])  # both signs
    n_blocks = -(-len(vals) // 31)
    blocks = np.zeros((n_blocks, 32), np.uint16)
    blocks[:, 0] = 0x43E0                          # 448
    fill = np.resize(vals, n_blocks * 31).reshape(n_blocks, 31)
    blocks[:, 1:] = fill
    K = 1024
    rows = -(-n_blocks * 32 // K)
    X = np.zeros(rows * K, np.uint16)
    X[:blocks.size] = blocks.reshape(-1)
    X = X.reshape(rows, K)
    codes, scales, g, D = L.quantize_activation(dev_bf16(X), None, None, None, 3)
    torch.cuda.synchronize()
    ref_codes, ref_scales = OM.mx_quantize(bf16_bits_to_f32(X), "e4m3")
    assert np.array_equal(scales.cpu().numpy(), ref_scales)
    assert np.array_equal(codes.cpu().numpy(), ref_codes)
