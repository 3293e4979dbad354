"""Pins of the oracle's GEMM and whole-layer composition: naive loops, the integer-exact case,
and an exactly quantisable layer where Y must equal X·Wᵀ bit for bit."""
import numpy as np

from oracle import gemm as G
from oracle import quant as Q
from oracle import formats as F
from oracle import layer as L
from oracle import calib as C
import synth

F32 = np.float32


def test_float64_linear_equals_naive_loops():
    rng = np.random.default_rng(0)
    M, N, K, r = 3, 5, 32, 2
    A = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K))
    D = rng.standard_normal((M, r))
    up = synth.to_bf16_bits(rng.standard_normal((N, r)))
    y = G.linear_f64(A, W, D, up)
    Df, Uf = D, F.bf16_bits_to_f32(up)
    for m in range(M):
        for n in range(N):
            acc = sum(A[m, k] * W[n, k] for k in range(K))
            acc += sum(float(Df[m, i]) * float(Uf[n, i]) for i in range(r))
            assert np.isclose(y[m, n], acc, rtol=1e-13, atol=1e-13)


def test_lowrank_down_equals_naive_loops():
    rng = np.random.default_rng(1)
    xhat = rng.standard_normal((4, 32)).astype(F32)
    down = synth.to_bf16_bits(rng.standard_normal((3, 32)))
    D = G.lowrank_down(xhat, down)
    xb = F.bf16_round_f32(xhat)
    df = F.bf16_bits_to_f32(down)
    for m in range(4):
        for i in range(3):
            acc = sum(float(xb[m, k]) * float(df[i, k]) for k in range(32))
            assert np.isclose(D[m, i], acc, rtol=1e-14, atol=1e-14)


def test_integer_exact_case_unit_scales():
    # all block scales 1.0 (E4M3 0x38) and g = 1: the layer is a plain integer-valued sum
    rng = np.random.default_rng(2)
    M, N, K = 6, 10, 64
    an = rng.integers(0, 16, (M, K)).astype(np.uint8)
    wn = rng.integers(0, 16, (N, K)).astype(np.uint8)
    ones_a = np.full((M, K // 16), 0x38, np.uint8)
    ones_w = np.full((N, K // 16), 0x38, np.uint8)
    D = np.zeros((M, 0))
    up = np.zeros((N, 0), np.uint16)
    y64, y = G.linear_nvfp4(F.pack_nibbles(an), ones_a, F32(1), F.pack_nibbles(wn), ones_w,
                            F32(1), D, up)
    av, wv = F.e2m1_decode(an), F.e2m1_decode(wn)
    for m in range(M):
        for n in range(N):
            assert y64[m, n] == sum(av[m, k] * wv[n, k] for k in range(K))
    assert np.all(y64 * 4 == np.round(y64 * 4))


def _exact_case(rng, fmt):
    """Inputs on which every quantiser is exact, so the layer must reproduce X·Wᵀ exactly."""
    M, N, K, r = 5, 8, 128, 3
    lam = (2.0 ** rng.integers(-1, 2, K)).astype(F32)
    if fmt == "nvfp4":
        def grid_rows(R, jlo, jhi):
            v = rng.choice(F.E2M1_VALUES, (R, K // 16, 16)) * rng.choice([-1.0, 1.0], (R, K // 16, 16))
            v[:, :, 0] = 6.0
            j = rng.integers(jlo, jhi, (R, K // 16, 1))
            return (v * 2.0 ** j).reshape(R, K)
    else:
        def grid_rows(R, jlo, jhi):
            c = rng.integers(-7, 8, (R, K // 64, 64)).astype(np.float64)
            c[:, :, 0] = 7.0
            s = 2.0 ** rng.integers(jlo, jhi, (R, K // 64, 1))
            return (c * s).reshape(R, K)
    xhat = grid_rows(M, -2, 2)
    X = synth.to_bf16_bits(xhat * lam)                     # X = X̂·λ, exact in bf16
    assert np.array_equal(F.bf16_bits_to_f32(X).astype(np.float64), xhat * lam)
    R = grid_rows(N, -1, 1)
    down = np.zeros((r, K))
    for i in range(r):
        down[i, rng.integers(0, K)] = rng.choice([-1.0, 1.0])
    up = rng.integers(-2, 3, (N, r)).astype(np.float64)
    Wp = R + up @ down
    W = synth.to_bf16_bits(Wp / lam)
    assert np.array_equal(F.bf16_bits_to_f32(W).astype(np.float64) * lam, Wp)
    return X, W, lam, synth.to_bf16_bits(down), synth.to_bf16_bits(up)


def test_exactly_quantisable_layer_reproduces_x_w_transpose():
    rng = np.random.default_rng(3)
    for fmt in ("nvfp4", "int4"):
        for _ in range(3):
            X, W, lam, down, up = _exact_case(rng, fmt)
            # tensor amax 2688·2^p gives a power-of-two tensor scale, so NVFP4 is exact on grid
            amax = F32(2688.0 * 4)
            act = L.prepare_activation(X, lam, amax, down, fmt)
            wt = L.prepare_weight(W, lam, down, up, fmt)
            if fmt == "nvfp4":
                assert wt["g"] == Q.nvfp4_tensor_scale(np.abs(wt["R32"]).max())
                c, s, g, _ = Q.nvfp4_quantize(wt["R32"], F32(2688.0))
                wt = dict(codes=c, scales=s, g=g)
            y64, y = L.forward(act, wt, up, fmt)
            xf = F.bf16_bits_to_f32(X).astype(np.float64)
            wf = F.bf16_bits_to_f32(W).astype(np.float64)
            M, N, K = xf.shape[0], wf.shape[0], xf.shape[1]
            naive = np.array([[sum(xf[m, k] * wf[n, k] for k in range(K)) for n in range(N)]
                              for m in range(M)])
            assert np.array_equal(y64, naive), fmt
            assert np.array_equal(y, F.bf16_rne(naive))


def test_layer_on_outlier_workload_is_a_faithful_approximation():
    cfg = synth.config(0)
    X = synth.x_bits(cfg)
    W = synth.weight_bits(cfg["N"], cfg["K"])
    from oracle import svd
    ref = F.bf16_bits_to_f32(X).astype(np.float64) @ F.bf16_bits_to_f32(W).astype(np.float64).T
    errs = {}
    for mask, r in ((0, 0), (0, 8), (7, 8)):
        _, _, lam, amax = C.calibrate(X, cfg["seg"], W, mask)
        down, up = svd.lowrank_factors(W, lam, r)
        act = L.prepare_activation(X, lam, amax, down, "nvfp4")
        wt = L.prepare_weight(W, lam, down, up, "nvfp4")
        y64, _ = L.forward(act, wt, up, "nvfp4")
        errs[(mask, r)] = np.linalg.norm(y64 - ref) / np.linalg.norm(ref)
        # dropping the low-rank term makes the result much worse whenever r > 0
        if r:
            y_no = y64 - G.lowrank_up(act["D"], up)
            assert np.linalg.norm(y_no - ref) / np.linalg.norm(ref) > 3 * errs[(mask, r)]
    assert all(e < 0.2 for e in errs.values()), errs
    assert errs[(7, 8)] < errs[(0, 0)]
