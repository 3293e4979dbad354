"""GPU parity at the largest reduction length K that the activation kernel accepts at each
rank, in every format ("MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph:
the layer; the limit is the kernel's LDS, which holds 1/λ for all K channels beside the staged
X and the rank-r slice of L1).  At rank 32 the largest K no longer fits two K groups of waves
per workgroup, so the single-group form of the kernel runs; in the MX GEMMs these K are long odd
stage counts (MXFP4: 111 and 104 stages, MXFP8: 222, 208 and 114).  Codes and scales
bit-exact, D and Y within the layer tolerance, on 70 rows (a full workgroup and a ragged one)."""
import numpy as np
import pytest

import synth
from tests.gpu_common import dev, dev_bf16, host_bits, check_y, check_d, oracle_case, torch_mod

pytestmark = pytest.mark.gpu

FMT_NAME = {0: "nvfp4", 1: "int4", 2: "mxfp4", 3: "mxfp8"}
# the largest K (a multiple of 256) whose activation-kernel LDS fits 160 KB, per rank
LARGEST_K = [(28416, 0), (26624, 32), (14592, 128)]


def same_bits(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


@pytest.mark.parametrize("K,r", LARGEST_K)
@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_largest_k_per_rank(L, fmt, K, r):
    torch = torch_mod()
    M, N = 70, 256
    cfg = dict(M=M, K=K, N=N, seg=synth.segments(M), gen="outlier")
    X, W, seg = synth.x_bits(cfg, 0), synth.weight_bits(N, K, 0), cfg["seg"]
    o = oracle_case(X, seg, W, 7, r, FMT_NAME[fmt])
    print(f"[limits] fmt={FMT_NAME[fmt]} K={K} r={r}", flush=True)
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    cal = L.calibrate(Xd, seg, Wd, 7)
    assert np.array_equal(cal["lambda"].cpu().numpy(), o["lam"])
    down = dev_bf16(o["down"]) if r else None
    up = dev_bf16(o["up"]) if r else None
    pw = L.prepare_weight(Wd, cal["lambda"], down, up, fmt)
    amax = dev(np.array([o["amax"]], np.float32)) if fmt == 0 else None
    codes, scales, g, D = L.quantize_activation(Xd, cal["lambda"], amax, down, fmt)
    Y = L.gemm(codes, scales, g, D, pw, M)
    torch.cuda.synchronize()
    assert same_bits(pw.codes.cpu().numpy(), o["wt"]["codes"])
    assert same_bits(pw.scales.cpu().numpy(), o["wt"]["scales"])
    assert same_bits(codes.cpu().numpy(), o["act"]["codes"])
    assert same_bits(scales.cpu().numpy(), o["act"]["scales"])
    if fmt == 0:
        assert pw.g.cpu().numpy()[0] == o["wt"]["g"]
        assert g.cpu().numpy()[0] == o["act"]["g"]
    if r:
        check_d(D.cpu().numpy(), o["act"]["D"])
    rel = check_y(host_bits(Y), o["y"])
    print(f"[limits] fmt={FMT_NAME[fmt]} K={K} r={r}: rel-L2 {rel:.2e}", flush=True)
