"""Pins of the oracle's DeltaQuant steps (geometry counts, brute-force small grids, exact core on
identical rows, the |x − core| ≤ 2·max|x| bound, FP8 core round trip, core GEMM loops) and of the
per-modality scoring sums; plus the synthetic-input recipe (split counts, boosted channels,
cross-modal correlation, chunk independence)."""
import os

import numpy as np

from oracle import delta as DQ
from oracle import formats as F
from oracle import quant as Q
from oracle import score as SC
from oracle import calib as C
import synth

F32 = np.float32
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_workloads():
    splits, geo = {}, {}
    with open(os.path.join(GOLD, "workloads.txt")) as f:
        for line in f:
            p = line.split()
            if not p or p[0].startswith("#"):
                continue
            if p[0].isdigit():
                splits[int(p[0])] = tuple(int(v) for v in p[1:])
            else:
                geo[p[0]] = int(p[1])
    return splits, geo


def test_workload_geometry_counts_match_golden():
    _, geo = _golden_workloads()
    cfg = synth.config(4)
    T, H, W = cfg["grid"]
    r2c, ptr, rows = DQ.cube_geometry(T, H, W, 2, 2, 2, cfg["n_text"], cfg["n_audio"], 4)
    sizes = np.diff(ptr)
    assert len(sizes) == geo["n_cubes"]
    assert len(r2c) == cfg["M"] and sorted(rows.tolist()) == list(range(cfg["M"]))
    nt, na = geo["text_cubes"], geo["audio_cubes"]
    video = sizes[nt:len(sizes) - na]
    assert len(video) == geo["video_cubes"] and np.count_nonzero(video == 4) == geo["ragged_video_cubes"]
    assert np.all((video == 8) | (video == 4)) and np.all(sizes[:nt] == 4) and np.all(sizes[-na:] == 4)
    firsts = rows[ptr[:-1]]
    assert np.all(np.diff(firsts) > 0)                     # numbered by first row
    for c in range(len(sizes)):
        assert np.all(r2c[rows[ptr[c]:ptr[c + 1]]] == c)


def test_geometry_small_grid_by_hand():
    # T,H,W = 3,2,3 with 2x2x2 cubes, 5 text rows, 2 audio rows, 1-D cubes of 2
    r2c, ptr, rows = DQ.cube_geometry(3, 2, 3, 2, 2, 2, 5, 2, 2)
    text = [0, 0, 1, 1, 2]
    # video raster index v = t*6 + h*3 + w; cube (t//2, w//2) (h//2 always 0)
    vid = []
    for t in range(3):
        for h in range(2):
            for w in range(3):
                vid.append(3 + (t // 2) * 2 + (w // 2))
    audio = [7, 7]
    assert r2c.tolist() == text + vid + audio
    assert np.diff(ptr).tolist() == [2, 2, 1, 8, 4, 4, 2, 2]


def test_core_is_exact_on_identical_rows_and_delta_codes_are_zero():
    rng = np.random.default_rng(0)
    K = 64
    base = F.bf16_round_f32(rng.standard_normal((3, K)))
    xhat = np.concatenate([np.repeat(base[0:1], 8, 0), np.repeat(base[1:2], 4, 0),
                           np.repeat(base[2:3], 3, 0)]).astype(F32)
    ptr = np.array([0, 8, 12, 15], np.int32)
    rows = np.arange(15, dtype=np.int32)
    r2c = np.repeat(np.arange(3), [8, 4, 3]).astype(np.int32)
    core = DQ.cube_core(xhat, ptr, rows)
    assert np.array_equal(core, base)
    d = DQ.delta_rows(xhat, core, r2c)
    codes, scales, g, sat = DQ.delta_quantize(d, F32(np.abs(xhat).max()))
    assert np.all(codes == 0) and np.all(scales == 0) and sat == 0


def test_core_sum_order_and_divisor():
    x = np.array([[1e8], [1.0], [-1e8], [1.0]], dtype=F32)
    core = DQ.cube_core(x, np.array([0, 4], np.int32), np.array([0, 1, 2, 3], np.int32))
    # ascending float32 sum: ((1e8 + 1) - 1e8) + 1 = 1 (1e8 + 1 rounds to 1e8), /4
    assert core[0, 0] == F32(0.25)


def test_delta_bound_holds_and_no_saturation_on_cube_field():
    cfg = dict(synth.config(4))
    cfg.update(grid=(5, 6, 8), n_text=12, n_audio=8, M=12 + 240 + 8, K=256,
               seg=(0, 12, 252, 260))
    X = synth.x_bits(cfg)
    r2c, ptr, rows = DQ.cube_geometry(5, 6, 8, 2, 2, 2, 12, 8, 4)
    ax, aw, lam, amax = C.calibrate(X, cfg["seg"], None, 7)
    xhat = C.smooth(X, lam)
    core = DQ.cube_core(xhat, ptr, rows)
    d = DQ.delta_rows(xhat, core, r2c)
    assert np.abs(d).max() <= 2 * np.abs(xhat).max()
    _, _, _, sat = DQ.delta_quantize(d, amax)
    assert sat == 0
    ratio = np.linalg.norm(d) / np.linalg.norm(xhat)
    assert 0.3 < ratio < 0.9            # the core absorbs part of the magnitude


def test_core_fp8_roundtrip():
    rng = np.random.default_rng(1)
    core = (rng.standard_normal((20, 64)) * rng.uniform(0.01, 10, (20, 1))).astype(F32)
    core[3] = 0
    codes, s = DQ.core_fp8(core)
    deq = F.e4m3_decode(codes) * s.astype(np.float64)[:, None]
    rel = np.abs(deq - core) / np.maximum(np.abs(core), 1e-30)
    big = np.abs(core) >= s[:, None] * 2.0 ** -6 * 2
    assert np.all(rel[big] <= 2.0 ** -4 + 1e-6)
    assert np.all(np.abs(F.e4m3_decode(codes)).max(axis=1)[np.arange(20) != 3] == 448.0)
    assert s[3] == 0 and np.all(codes[3] == 0)
    codes2, s2 = DQ.core_fp8((F.e4m3_decode(codes) * s[:, None]).astype(F32))
    assert np.array_equal(codes2, codes)


def test_core_out_and_delta_linear_equal_naive_loops():
    rng = np.random.default_rng(2)
    C_, N, K, M = 3, 4, 32, 5
    ccodes = rng.integers(0, 255, (C_, K)).astype(np.uint8)
    ccodes[(ccodes & 0x7F) == 0x7F] = 0x38
    cs = rng.uniform(0.1, 2, C_).astype(F32)
    w = rng.standard_normal((N, K)).astype(F32)
    wc, ws, gw, _ = Q.nvfp4_quantize(w, F32(np.abs(w).max()))
    co = DQ.core_out_f64(ccodes, cs, wc, ws, gw)
    Wd = Q.nvfp4_dequantize(wc, ws, gw)
    cv = F.e4m3_decode(ccodes)
    for c in range(C_):
        for n in range(N):
            assert np.isclose(co[c, n], float(cs[c]) * sum(cv[c, k] * Wd[n, k] for k in range(K)),
                              rtol=1e-12, atol=1e-12)
    d = rng.standard_normal((M, K)).astype(F32)
    dc, dsc, gd, _ = Q.nvfp4_quantize(d, F32(np.abs(d).max()))
    r2c = np.array([0, 0, 1, 2, 2], np.int32)
    D = rng.standard_normal((M, 2))
    up = synth.to_bf16_bits(rng.standard_normal((N, 2)))
    y64, _ = DQ.delta_linear(co, r2c, dc, dsc, gd, wc, ws, gw, D, up)
    Ad = Q.nvfp4_dequantize(dc, dsc, gd)
    Df, Uf = D, F.bf16_bits_to_f32(up)
    for m in range(M):
        for n in range(N):
            want = co[r2c[m], n] + sum(Ad[m, k] * Wd[n, k] for k in range(K)) \
                + sum(float(Df[m, i]) * float(Uf[n, i]) for i in range(2))
            assert np.isclose(y64[m, n], want, rtol=1e-12, atol=1e-12)
    y_sub, _ = DQ.delta_linear(co, r2c, dc, dsc, gd, wc, ws, gw, D, up, rows=np.array([3, 1]))
    assert np.array_equal(y_sub, y64[[3, 1]])


def test_modal_sums_equal_naive_loops_and_special_values():
    rng = np.random.default_rng(3)
    Y = synth.to_bf16_bits(rng.standard_normal((7, 5)))
    R = synth.to_bf16_bits(rng.standard_normal((7, 5)))
    grp = np.array([0, 1, 1, 2, 3, 3, 0], np.int8)
    s = SC.modal_sums(Y, R, grp)
    yf, rf = F.bf16_bits_to_f32(Y).astype(float), F.bf16_bits_to_f32(R).astype(float)
    for mu in range(4):
        d2 = sum((yf[i, n] - rf[i, n]) ** 2 for i in range(7) if grp[i] == mu for n in range(5))
        r2 = sum(rf[i, n] ** 2 for i in range(7) if grp[i] == mu for n in range(5))
        assert np.isclose(s[mu, 0], d2, rtol=1e-14) and np.isclose(s[mu, 1], r2, rtol=1e-14)
    assert np.all(SC.rel_l2(SC.modal_sums(R, R, grp)) == 0)
    assert np.allclose(SC.rel_l2(SC.modal_sums(np.zeros_like(R), R, grp)), 1)


def test_synthetic_recipe_counts_correlation_and_chunks():
    splits, _ = _golden_workloads()
    for i in range(5):
        seg = synth.config(i)["seg"]
        assert (seg[1], seg[2] - seg[1], seg[3] - seg[2]) == splits[i]
    for K in (256, 5120, 13824):
        c, boosted = synth.profiles(K)
        assert all(len(b) == round(0.02 * K) for b in boosted)
        lz = np.log(c)
        for a, b in ((0, 1), (0, 2), (1, 2)):
            assert abs(np.corrcoef(lz[a], lz[b])[0, 1]) < 0.1
    cfg = synth.config(0)
    X = synth.x_bits(cfg)
    assert np.array_equal(synth.x_bits(cfg, rows=slice(100, 230)), X[100:230])
    W = synth.weight_bits(300, 64)
    assert np.array_equal(synth.weight_bits(300, 64, rows=slice(250, 300)), W[250:])
    rows, grp = synth.sample_rows(synth.config(3)["seg"])
    n = np.bincount(grp, minlength=4)
    assert n.tolist() == [655, 4096, 262, 4096]
    assert len(np.unique(rows[grp == 1])) == 4096


def _exact_deltaquant_case(P=6, K=64, N=32, seed=0):
    """A DeltaQuant layer whose every quantisation step is exact (power-of-two and E4M3-exact
    scales, values on their grids): pair cubes x = c ± d with core c on the E4M3 grid (row amax
    448, so s_c = 1) and delta d on the E2M1 grid (every non-zero block holds a ±6; with
    act_amax = 1344 the delta tensor scale is 2·1344/2688 = 1); one 1-row cube [1344, 0, ...]
    sets act_amax; the weight has tensor scale 2^-10 (amax 6·448·2^-10) and E4M3-exact block
    scales (a ±6 code in every block).  Returns (X bits, W bits, seg, geometry args)."""
    rng = np.random.default_rng(seed)
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    rows = []
    for _ in range(P):
        c = rng.choice([0.0, 1, 2, 4, 8, 16], K) * rng.choice([-1.0, 1.0], K)
        d = rng.choice(e2m1, K) * rng.choice([-1.0, 1.0], K)
        j = rng.integers(K)                       # the channel of the core's 448
        c[j], d[j] = 448.0 * rng.choice([-1.0, 1.0]), 0.0
        for b in range(K // 16):                  # a ±6 in every delta block, away from j
            i = 16 * b + rng.integers(16)
            i = i if i != j else 16 * b + (i - 16 * b + 1) % 16
            d[i] = 6.0 * rng.choice([-1.0, 1.0])
        rows += [c + d, c - d]
    big = np.zeros(K)
    big[0] = 1344.0
    rows.append(big)
    X = np.array(rows)
    W = np.zeros((N, K))
    for n in range(N):
        for b in range(K // 16):
            s = 448.0 if (n == 0 and b == 0) else 256.0
            codes = rng.choice(e2m1, 16) * rng.choice([-1.0, 1.0], 16)
            codes[rng.integers(16)] = 6.0
            W[n, 16 * b:16 * b + 16] = codes * s * 2.0 ** -10
    Xb, Wb = synth.gen.to_bf16_bits(X), synth.gen.to_bf16_bits(W)
    assert np.array_equal(F.bf16_bits_to_f32(Xb), X) and np.array_equal(F.bf16_bits_to_f32(Wb), W)
    M = 2 * P + 1
    # video grid 1 x 1 x 2P with 1x1x2 cubes (the pairs), then one audio row in a 1-D cube
    return Xb, Wb, (0, 0, 2 * P, M), (1, 1, 2 * P, 1, 1, 2, 0, 1, 1)


def test_exact_deltaquant_layer_reproduces_x_w_transpose():
    """With every step exact, core term + delta term = X̂·W'ᵀ exactly: a dropped core term, a
    wrong cube index, a sign error in the delta or a mis-scaled core would all break it."""
    from oracle import layer as OL
    Xb, Wb, seg, geo = _exact_deltaquant_case()
    ax, aw, lam, amax = C.calibrate(Xb, seg, Wb, 0)
    assert np.all(lam == 1) and amax == F32(1344)
    r2c, ptr, crow = DQ.cube_geometry(*geo)
    assert np.array_equal(np.diff(ptr), [2] * 6 + [1])
    xhat = C.smooth(Xb, lam)
    core = DQ.cube_core(xhat, ptr, crow)
    cc, cs = DQ.core_fp8(core)
    assert np.all(cs[:-1] == 1) and cs[-1] == 3
    d = DQ.delta_rows(xhat, core, r2c)
    dc, dsc, gd, sat = DQ.delta_quantize(d, amax)
    assert gd == 1 and sat == 0
    assert np.array_equal(Q.nvfp4_dequantize(dc, dsc, gd), d.astype(np.float64))
    wt = OL.prepare_weight(Wb, lam, np.zeros((0, 64), np.uint16), np.zeros((32, 0), np.uint16),
                           "nvfp4")
    assert wt["g"] == F32(2.0 ** -10)
    co = DQ.core_out_f64(cc, cs, wt["codes"], wt["scales"], wt["g"])
    y64, y = DQ.delta_linear(co, r2c, dc, dsc, gd, wt["codes"], wt["scales"], wt["g"],
                             np.zeros((13, 0)), np.zeros((32, 0), np.uint16))
    want = F.bf16_bits_to_f32(Xb).astype(np.float64) @ F.bf16_bits_to_f32(Wb).astype(np.float64).T
    assert np.array_equal(y64, want)
    assert np.array_equal(y, F.bf16_rne(want))
