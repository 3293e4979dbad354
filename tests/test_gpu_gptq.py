"""GPU parity of the GPTQ entry points (svdq_gptq_hessian, svdq_gptq_quantize_weight) with the
oracle ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph; GPTQ as
published).  The Hessian is a float64 sum of exact products, so only the order of the sums
differs: relative 1e-12.  The GPU sweep is the inverse-free form of the published one, in
float64 on both sides; a rounding decision could only differ where the two float64 working
values straddle a float32 rounding boundary, so codes and scales are compared bit for bit."""
import numpy as np
import pytest

import synth
from oracle import gptq as OG, calib as OC, svd as OS
from tests.gpu_common import dev_bf16, dev, torch_mod

pytestmark = pytest.mark.gpu

FMT = {"nvfp4": 0, "int4": 1, "mxfp4": 2, "mxfp8": 3}


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _case(M, K, N, r, seed=0):
    cfg = dict(synth.config(0), M=M, K=K, N=N, seg=synth.segments(M, 16, 16))
    X = synth.x_bits(cfg, seed=seed)
    W = synth.weight_bits(N, K, seed=seed)
    _, _, lam, _ = OC.calibrate(X, cfg["seg"], W, 7)
    down, up = OS.lowrank_factors(W, lam, r)
    return X, W, lam, down, up


@pytest.fixture(scope="module")
def small():
    return _case(600, 512, 256, 8)


def test_hessian_and_accumulation(L, small):
    torch = torch_mod()
    X, W, lam, _, _ = small
    H = L.gptq_hessian(dev_bf16(X), dev(lam))
    Ha = L.gptq_hessian(dev_bf16(X[:250]), dev(lam))
    L.gptq_hessian(dev_bf16(X[250:]), dev(lam), Ha)
    H0 = L.gptq_hessian(dev_bf16(X[:7]), None)
    torch.cuda.synchronize()
    ref = OG.hessian(X, lam)
    for got in (H.cpu().numpy(), Ha.cpu().numpy()):
        assert np.all(np.abs(got - ref) <= 1e-12 * np.abs(ref).max())
        assert np.array_equal(got, got.T)
    assert np.allclose(H0.cpu().numpy(), OG.hessian(X[:7], None), rtol=1e-12, atol=0)


def _codes_equal(pw, ref, fmt, what):
    gc = pw.codes.cpu().numpy()
    gs = pw.scales.cpu().numpy().view(np.uint8)
    rs = np.asarray(ref["scales"]).view(np.uint8)
    nbad = int(np.count_nonzero(gc != ref["codes"]))
    print(f"[gptq] {what}: {nbad} of {gc.size} code bytes differ, "
          f"{int(np.count_nonzero(gs != rs))} scale bytes", flush=True)
    assert nbad == 0 and np.array_equal(gs, rs)
    if fmt == "nvfp4":
        assert pw.g.cpu().numpy()[0] == ref["g"]


@pytest.mark.parametrize("fmt", ["int4", "nvfp4", "mxfp4", "mxfp8"])
def test_gptq_codes_match_the_oracle(L, small, fmt):
    torch = torch_mod()
    X, W, lam, down, up = small
    Hd = L.gptq_hessian(dev_bf16(X), dev(lam))
    pw = L.prepare_weight_gptq(dev_bf16(W), dev(lam), dev_bf16(down), dev_bf16(up), Hd, FMT[fmt])
    torch.cuda.synchronize()
    ref = OG.gptq_quantize(OS.residual_f32(W, lam, down, up), OG.hessian(X, lam), fmt)
    _codes_equal(pw, ref, fmt, f"{fmt} 256x512 r=8")


def test_gptq_without_branch_or_lambda(L, small):
    torch = torch_mod()
    X, W, lam, down, up = small
    Hd = L.gptq_hessian(dev_bf16(X), None)
    pw = L.prepare_weight_gptq(dev_bf16(W), None, None, None, Hd, FMT["int4"])
    torch.cuda.synchronize()
    ref = OG.gptq_quantize(OS.residual_f32(W, None, down[:0], up[:, :0]), OG.hessian(X, None),
                           "int4")
    _codes_equal(pw, ref, "int4", "int4 no λ, r=0")


def test_diagonal_hessian_gives_round_to_nearest(L, small):
    torch = torch_mod()
    X, W, lam, down, up = small
    K = W.shape[1]
    for fmt in ("nvfp4", "int4", "mxfp8"):
        Hd = dev(np.diag(np.linspace(0.5, 2.0, K)))
        Wd, ld, dd, ud = dev_bf16(W), dev(lam), dev_bf16(down), dev_bf16(up)
        pg = L.prepare_weight_gptq(Wd, ld, dd, ud, Hd, FMT[fmt])
        pr = L.prepare_weight(Wd, ld, dd, ud, FMT[fmt])
        torch.cuda.synchronize()
        assert torch.equal(pg.codes, pr.codes) and torch.equal(pg.scales.view(torch.uint8),
                                                               pr.scales.view(torch.uint8))
        if fmt == "nvfp4":
            assert torch.equal(pg.g, pr.g)


def test_all_zero_hessian_is_the_identity(L, small):
    torch = torch_mod()
    X, W, lam, down, up = small
    K = W.shape[1]
    Wd, ld, dd, ud = dev_bf16(W), dev(lam), dev_bf16(down), dev_bf16(up)
    pg = L.prepare_weight_gptq(Wd, ld, dd, ud, torch.zeros(K, K, dtype=torch.float64,
                                                           device="cuda"), FMT["mxfp4"])
    pr = L.prepare_weight(Wd, ld, dd, ud, FMT["mxfp4"])
    torch.cuda.synchronize()
    assert torch.equal(pg.codes, pr.codes) and torch.equal(pg.scales, pr.scales)


def test_full_size_attention_projection(L):
    """5120 x 5120, rank 32, NVFP4 and int4, Hessian of 2048 calibration rows: codes and scales
    of 48 sampled weight rows against the oracle (rows are independent given H); timed."""
    torch = torch_mod()
    cfg = synth.config(1)
    K, N, r = cfg["K"], cfg["N"], cfg["r"]
    print(f"[gptq] full size {cfg['name']}", flush=True)
    Xc = synth.x_bits(cfg, rows=slice(4096, 6144))      # 2048 consecutive rows
    W = synth.weight_bits(N, K)
    lam = np.exp(np.random.default_rng(12).normal(0, 0.5, K)).astype(np.float32)
    omega = np.random.default_rng(13).standard_normal((N, r + 8)).astype(np.float32)
    down, up = OS.randomized_factors(W, lam, r, omega, 2)[:2]
    R32 = OS.residual_f32(W, lam, down, up)
    Href = OG.hessian(Xc, lam)
    pick = np.sort(np.random.default_rng(14).choice(N, 48, replace=False))
    Wd, ld, dd, ud = dev_bf16(W), dev(lam), dev_bf16(down), dev_bf16(up)
    for fmt in ("nvfp4", "int4"):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        Hd = L.gptq_hessian(dev_bf16(Xc), ld)
        t1.record()
        torch.cuda.synchronize()
        th = t0.elapsed_time(t1)
        t0.record()
        pw = L.prepare_weight_gptq(Wd, ld, dd, ud, Hd, FMT[fmt])
        t1.record()
        torch.cuda.synchronize()
        print(f"[gptq] {fmt} 5120x5120: Hessian of 2048 rows {th:.1f} ms, GPTQ "
              f"{t0.elapsed_time(t1):.1f} ms", flush=True)
        ref = OG.gptq_quantize(R32[pick], Href, fmt, amax=np.abs(R32).max())
        gc = pw.codes.cpu().numpy()[pick]
        gs = pw.scales.cpu().numpy().view(np.uint8)[pick]
        nbad = int(np.count_nonzero(gc != ref["codes"]))
        print(f"[gptq] {fmt} sampled rows: {nbad} of {gc.size} code bytes differ", flush=True)
        assert nbad == 0 and np.array_equal(gs, np.asarray(ref["scales"]).view(np.uint8))
        if fmt == "nvfp4":
            assert pw.g.cpu().numpy()[0] == ref["g"]
