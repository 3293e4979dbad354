"""GPU parity of the DeltaQuant path ("DeltaQuant on MiniMax-H3") against the oracle: cube
geometry, FP8 cube-mean core, NVFP4 delta, D at rank r, core GEMM, delta GEMM with the core term.
Covers the 2x2x2 workload (31x24x42 grid, prime T, ragged edge cubes) and the geometry variants
of section "Deviations from the paper, and one replication" at full size — uniform cube-64
(4x4x4) and divisor-aligned edges — plus small grids with every cube shape class, rank 0 and
128, 1-row cubes, and a caller-built CSR with a 64-row cube of scattered rows.

Bit-exact: geometry, core codes and scales, delta codes and scales, g_delta, the saturation
count.  core_out per element within 2^-16·|c| + 1e-5·rms(c) of the float64 value: the products
are exact, and K/16 fp32 roundings of partial sums of rms ~ rms(c)·sqrt(16/K) give an rms error
near 5e-7·rms(c) at K = 5120 (about 2.5e-6 at the 5.5σ tail of 2·10^7 elements), plus one
rounding of the scale product.  D and Y as in the other layer tests."""
import numpy as np
import pytest

import synth
from oracle import calib as OC, svd as OS, layer as OL, delta as DQ, gemm as OG
from tests.gpu_common import dev_bf16, host_bits, dev, check_y, check_d, torch_mod

pytestmark = pytest.mark.gpu
CORE_OUT_REL = 2.0 ** -16
CORE_OUT_RMS = 1e-5


@pytest.fixture(scope="module")
def L():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return layer


def _cfg(grid, n_text, n_audio, K, N, r, field=(2, 2, 2), field1d=4):
    cfg = dict(synth.config(4))
    T, H, W = grid
    M = n_text + T * H * W + n_audio
    cfg.update(grid=grid, n_text=n_text, n_audio=n_audio, K=K, N=N, r=r, M=M,
               seg=(0, n_text, n_text + T * H * W, M), cube=field, cube1d=field1d)
    return cfg


def _delta_case(cfg, geo, seed=0, csr=None):
    """Oracle side of the DeltaQuant layer for geometry geo = (ct, ch, cw, cube1d) (or a
    caller's CSR (row_to_cube, cube_ptr, cube_rows))."""
    T, H, Wd = cfg["grid"]
    X = synth.x_bits(cfg, seed)
    W = synth.weight_bits(cfg["N"], cfg["K"], seed)
    ax, aw, lam, amax = OC.calibrate(X, cfg["seg"], W, 7)
    r = cfg["r"]
    down, up = OS.lowrank_factors(W, lam, r) if r else (np.zeros((0, cfg["K"]), np.uint16),
                                                        np.zeros((cfg["N"], 0), np.uint16))
    if csr is None:
        ct, ch, cw, c1 = geo
        r2c, ptr, crow = DQ.cube_geometry(T, H, Wd, ct, ch, cw, cfg["n_text"], cfg["n_audio"], c1)
    else:
        r2c, ptr, crow = csr
    xhat = OC.smooth(X, lam)
    core = DQ.cube_core(xhat, ptr, crow)
    cc, cs = DQ.core_fp8(core)
    dc, dsc, gd, sat = DQ.delta_quantize(DQ.delta_rows(xhat, core, r2c), amax)
    wt = OL.prepare_weight(W, lam, down, up, "nvfp4")
    co = DQ.core_out_f64(cc, cs, wt["codes"], wt["scales"], wt["g"])
    return dict(X=X, W=W, lam=lam, amax=amax, down=down, up=up, r2c=r2c, ptr=ptr, crow=crow,
                xhat=xhat, cc=cc, cs=cs, dc=dc, dsc=dsc, gd=gd, sat=sat, wt=wt, co=co)


def _gpu_delta(L, o, cfg, geo, csr=None):
    torch = torch_mod()
    from w4a4_quantized_dit_amd import _lib
    T, H, Wg = cfg["grid"]
    if csr is None:
        ct, ch, cw, c1 = geo
        g = L.cube_geometry(T, H, Wg, ct, ch, cw, cfg["n_text"], cfg["n_audio"], c1)
        host = (g["host"]["row_to_cube"], g["host"]["cube_ptr"], g["host"]["cube_rows"])
    else:
        r2c, ptr, crow = csr
        g = dict(row_to_cube=dev(r2c), cube_ptr=dev(ptr), cube_rows=dev(crow),
                 group_ptr=dev(_lib.svdq_cube_groups(ptr)), n_cubes=len(ptr) - 1)
        host = csr
    M, K, N, r = cfg["M"], cfg["K"], cfg["N"], cfg["r"]
    nc = g["n_cubes"]
    Xd, Wd = dev_bf16(o["X"]), dev_bf16(o["W"])
    cal = L.calibrate(Xd, cfg["seg"], Wd, 7)
    downd = dev_bf16(o["down"]) if r else None
    pw = L.prepare_weight(Wd, cal["lambda"], downd, dev_bf16(o["up"]) if r else None, 0)
    sat = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq = L.delta_quantize_activation(Xd, cal["lambda"], cal["act_amax"], g, downd, sat_count=sat)
    co = torch.empty(nc, N, device="cuda")
    _lib.svdq_gemm_core(nc, N, K, dq["cc"], dq["cs"], pw.codes, pw.scales, pw.g, co)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    _lib.svdq_w4a4_gemm(0, M, N, K, dq["dc"], dq["dsc"], dq["gd"], pw.codes, pw.scales, pw.g,
                        dq["D"], pw.lora_up, r, Y, core_out=co, row_to_cube=g["row_to_cube"])
    torch.cuda.synchronize()
    return dict(geo=host, cal=cal, cc=dq["cc"], cs=dq["cs"], dc=dq["dc"], dsc=dq["dsc"],
                gd=dq["gd"], D=dq["D"], sat=sat, co=co, Y=Y)


def _check_core_out(got, want):
    got = np.asarray(got, np.float64)
    rms = np.sqrt(np.mean(want * want))
    bad = np.abs(got - want) > CORE_OUT_REL * np.abs(want) + CORE_OUT_RMS * rms
    assert not bad.any(), (f"core_out: {bad.sum()} elements out of tolerance, worst "
                           f"{np.abs(got - want).max():.3e} (rms {rms:.3e})")


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
    _check_core_out(g["co"].cpu().numpy(), o["co"])
    r = o["down"].shape[0]
    D_full = np.zeros((o["xhat"].shape[0], r))
    if r:
        D_rows = OG.lowrank_down(o["xhat"][rows], o["down"])
        check_d(g["D"].cpu().numpy()[rows], D_rows)
        D_full[rows] = D_rows          # only the sampled rows are read below
    _, y = DQ.delta_linear(o["co"], o["r2c"], o["dc"], o["dsc"], o["gd"], o["wt"]["codes"],
                           o["wt"]["scales"], o["wt"]["g"], D_full, o["up"], rows=rows)
    return check_y(host_bits(g["Y"])[rows], y)


@pytest.mark.parametrize("geo,r", [
    ((2, 2, 2, 4), 32),
    ((4, 4, 4, 64), 128),     # uniform cube-64, 1-D cubes of 64
    ((4, 4, 4, 4), 0),        # no low-rank branch
    ((1, 1, 1, 1), 16),       # every row its own cube: zero deltas, 16 cubes per group
    ((2, 3, 4, 5), 8),        # 24-row cubes, ragged in every axis
    ((1, 3, 3, 7), 40),       # divisor-aligned edges of a requested 4x4x4 on a 5x6x9 grid
])
def test_deltaquant_small_grids(L, geo, r):
    cfg = _cfg((5, 6, 9), 13, 9, 512, 256, r, field=geo[:3], field1d=geo[3])
    o = _delta_case(cfg, geo)
    g = _gpu_delta(L, o, cfg, geo)
    rows = np.arange(cfg["M"])
    print(f"deltaquant small {geo} r={r} rel-L2 {_compare_delta(o, g, rows):.2e}")


def test_deltaquant_caller_csr_with_a_64_row_cube(L):
    """A CSR the caller builds: one cube of 64 rows spread over the whole sequence (every third
    row), the remaining rows in cubes of 1 to 7 consecutive leftovers."""
    cfg = _cfg((4, 5, 9), 12, 8, 512, 256, 32)
    M = cfg["M"]
    big = list(range(0, 192, 3))
    rest = [m for m in range(M) if m not in set(big)]
    cubes, i, s = [], 0, 1
    while i < len(rest):
        cubes.append(rest[i:i + s])
        i += s
        s = s % 7 + 1
    cubes.append(big)
    cubes.sort(key=lambda c: c[0])                      # numbered by first row
    r2c = np.zeros(M, np.int32)
    for c, mem in enumerate(cubes):
        r2c[mem] = c
    ptr = np.concatenate([[0], np.cumsum([len(c) for c in cubes])]).astype(np.int32)
    crow = np.array([m for c in cubes for m in c], np.int32)
    csr = (r2c, ptr, crow)
    o = _delta_case(cfg, None, csr=csr)
    g = _gpu_delta(L, o, cfg, None, csr=csr)
    _compare_delta(o, g, np.arange(M))


def _full_rows(cfg):
    M, nt = cfg["M"], cfg["n_text"]
    T, H, W = cfg["grid"]
    last = nt + (T - 1) * H * W
    return np.array(sorted(set(range(0, M, 97)) | set(range(0, nt)) | set(range(M - 128, M))
                           | set(range(last, last + 60))))


@pytest.mark.parametrize("geo", [(2, 2, 2, 4), (4, 4, 4, 4), (1, 4, 3, 4)],
                         ids=["cube8", "cube64", "divisor-aligned"])
def test_deltaquant_full_size(L, geo):
    """The DeltaQuant workload (31x24x42 video grid, prime T, 312 text and 128 audio rows,
    K = N = 5120, rank 128) under the standing 2x2x2 cubes, uniform cube-64 (ragged in T and W),
    and the divisor-aligned edges of a requested 4x4x4 (1x4x3: no ragged cube)."""
    from w4a4_quantized_dit_amd import _lib
    cfg = dict(synth.config(4))
    if geo != (2, 2, 2, 4):
        assert _lib.svdq_cube_divisor_aligned(*cfg["grid"], 4, 4, 4) == (1, 4, 3)
    cfg["cube"] = geo[:3] if geo == (4, 4, 4, 4) else (2, 2, 2)
    print(f"[delta] {cfg['name']} cubes {geo}", flush=True)
    o = _delta_case(cfg, geo)
    g = _gpu_delta(L, o, cfg, geo)
    rows = _full_rows(cfg)
    print(f"[delta] {geo}: {len(rows)} sampled rows rel-L2 {_compare_delta(o, g, rows):.2e}",
          flush=True)


def test_exact_deltaquant_layer_is_bit_exact(L):
    """The exactly quantisable DeltaQuant layer (every scale a power of two or E4M3-exact, every
    value on its grid, every fp32 partial sum exact): the GPU's core GEMM plus delta GEMM must
    give bf16(X·Wᵀ) bit for bit."""
    torch = torch_mod()
    from w4a4_quantized_dit_amd import _lib
    from tests.test_oracle_delta_score import _exact_deltaquant_case
    from oracle.formats import bf16_bits_to_f32, bf16_rne
    Xb, Wb, seg, geo = _exact_deltaquant_case(P=128, K=256, N=256, seed=4)
    M, K, N = Xb.shape[0], 256, 256
    want = bf16_rne(bf16_bits_to_f32(Xb).astype(np.float64)
                    @ bf16_bits_to_f32(Wb).astype(np.float64).T)
    Xd, Wd = dev_bf16(Xb), dev_bf16(Wb)
    cal = L.calibrate(Xd, seg, Wd, 0)
    pw = L.prepare_weight(Wd, cal["lambda"], None, None, 0)
    g = L.cube_geometry(*geo)
    assert g["n_cubes"] == 129
    dq = L.delta_quantize_activation(Xd, cal["lambda"], cal["act_amax"], g, None)
    co = torch.empty(g["n_cubes"], N, device="cuda")
    _lib.svdq_gemm_core(g["n_cubes"], N, K, dq["cc"], dq["cs"], pw.codes, pw.scales, pw.g, co)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    _lib.svdq_w4a4_gemm(0, M, N, K, dq["dc"], dq["dsc"], dq["gd"], pw.codes, pw.scales, pw.g,
                        None, None, 0, Y, core_out=co, row_to_cube=g["row_to_cube"])
    torch.cuda.synchronize()
    assert cal["act_amax"].cpu().numpy()[0] == 1344.0
    assert dq["gd"].cpu().numpy()[0] == 1.0
    assert np.array_equal(host_bits(Y), want)
