"""GPU parity of the randomized low-rank factors (svdq_lowrank_factors) with the oracle's
randomized factors for the same random matrix.  Factors are unique only up to signs and
rotations, so what is compared is what the method fixes: the singular value estimates (fp32
path against float64: relative 1e-4), the approximation error ||A − L1·L2||_F of the bf16
factors (within 1 % of the oracle's bf16 factors, and never below the optimal error where that
is known), the orthonormality of the right factor (to bf16 rounding), exact recovery of an
exactly low-rank weight, and run-to-run determinism."""
import numpy as np
import pytest

import synth
from oracle import svd as OS
from oracle.formats import bf16_rne, bf16_bits_to_f32
from tests.gpu_common import dev_bf16, dev, host_bits, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _gpu(L, W_bits, lam, omega, r, q):
    down, up, sig = L.lowrank_factors(dev_bf16(W_bits), dev(lam) if lam is not None else None,
                                      dev(omega.astype(np.float32)), r, q)
    torch_mod().cuda.synchronize()
    return host_bits(down), host_bits(up), sig.cpu().numpy().astype(np.float64)


def _err(A, down_bits, up_bits):
    L1 = bf16_bits_to_f32(down_bits).astype(np.float64).T
    L2 = bf16_bits_to_f32(up_bits).astype(np.float64).T
    return np.linalg.norm(A - L1 @ L2)


def _compare(W_bits, lam, omega, r, q, gpu, optimal=None):
    down, up, sig = gpu
    o_down, o_up, o_sig, _, _ = OS.randomized_factors(W_bits, lam, r, omega.astype(np.float32), q)
    A = OS.smoothed_weight(W_bits, lam).T
    assert np.all(np.abs(sig - o_sig) <= 1e-4 * o_sig[0]), (sig[:4], o_sig[:4])
    e_gpu, e_ora = _err(A, down, up), _err(A, o_down, o_up)
    assert e_gpu <= 1.01 * e_ora, (e_gpu, e_ora)
    if optimal is not None:
        assert e_gpu >= optimal * (1 - 1e-6)
    V = bf16_bits_to_f32(up).astype(np.float64)
    assert np.abs(V.T @ V - np.eye(r)).max() < 2e-2
    print(f"[lowrank] {W_bits.shape} r={r} q={q}: error {e_gpu:.5g} (oracle {e_ora:.5g}"
          + (f", optimal {optimal:.5g}" if optimal is not None else "") + ")", flush=True)


def test_exactly_low_rank_weight_is_recovered(L):
    rng = np.random.default_rng(0)
    N, K, rank = 200, 256, 6
    Wb = bf16_rne((rng.integers(-2, 3, (N, rank)) @ rng.integers(-2, 3, (rank, K))).astype(float))
    lam = np.exp(rng.normal(0, 0.3, K)).astype(np.float32)
    A = OS.smoothed_weight(Wb, lam).T
    down, up, sig = _gpu(L, Wb, lam, rng.standard_normal((N, 12)), rank, 1)
    exact = np.linalg.svd(A, compute_uv=False)[:rank]
    assert np.all(np.abs(sig - exact) <= 1e-4 * exact[0])
    assert _err(A, down, up) <= 1e-2 * np.linalg.norm(A)     # bf16 rounding of the factors


# ell up to 64 keeps every small factorisation in LDS; 72 puts the eigensolver in global memory;
# 136 and 160 (the largest ell) put both the Cholesky-inverse and the eigensolver there
@pytest.mark.parametrize("N,K,r,ell,q", [(320, 512, 16, 24, 2), (333, 264, 8, 16, 0),
                                         (256, 1024, 32, 40, 1), (384, 512, 64, 72, 2),
                                         (512, 768, 128, 136, 1), (400, 640, 120, 160, 1)])
def test_decaying_spectrum_against_oracle(L, N, K, r, ell, q):
    rng = np.random.default_rng(N + K)
    n = min(N, K)
    decay = 0.8 if r <= 32 else 0.97
    s_true = np.concatenate([20.0 * decay ** np.arange(r + 4), 0.05 * np.ones(n - r - 4)])
    U = np.linalg.qr(rng.standard_normal((N, n)))[0]
    Vm = np.linalg.qr(rng.standard_normal((K, n)))[0]
    Wb = bf16_rne(U @ np.diag(s_true) @ Vm.T)
    lam = None if q == 0 else np.exp(rng.normal(0, 0.2, K)).astype(np.float32)
    omega = rng.standard_normal((N, ell))
    A = OS.smoothed_weight(Wb, lam).T
    sv = np.linalg.svd(A, compute_uv=False)
    _compare(Wb, lam, omega, r, q, _gpu(L, Wb, lam, omega, r, q),
             optimal=np.sqrt((sv[r:] ** 2).sum()))


def test_attention_projection_weight(L):
    cfg = synth.config(1)
    K, N, r = cfg["K"], cfg["N"], cfg["r"]
    X, W = synth.x_bits(cfg), synth.weight_bits(N, K)
    cal = L.calibrate(dev_bf16(X), cfg["seg"], dev_bf16(W), 7)
    lam = cal["lambda"].cpu().numpy()
    omega = np.random.default_rng(5).standard_normal((N, r + 8))
    g1 = _gpu(L, W, lam, omega, r, 2)
    g2 = _gpu(L, W, lam, omega, r, 2)
    assert all(np.array_equal(a, b) for a, b in zip(g1, g2))     # deterministic
    _compare(W, lam, omega, r, 2, g1)
