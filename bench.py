#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 layer on one MI355X.

Default workload (the JSON line's `value`): the attention-projection-sized layer, M = 16384
packed rows (164 text / 16154 video / 66 audio), K = N = 5120, rank 32, NVFP4.  One step is the
whole per-batch path:
    λ calibration over the batch -> residual-weight quantisation -> activation quantisation
    with the low-rank down-projection -> W4A4 GEMM with the up-projection (bf16 out).
Inputs are seeded synthetic tensors resident in HBM before the timed region; enough copies of X
are rotated (at least 1 GiB in all) that the 256 MB last-level cache cannot serve the activation
reads of one step from the previous one.

`--workload` also times the int4-g64 MLP up-projection (M = 32768, K = 5120, N = 13824), the
MLP down-projection λ sweep (M = 65536, K = 13824, N = 5120: calibration, layer and
per-modality scoring for each of λ = 1, all rows, video rows, text rows), the DeltaQuant
cube-field layer (31x24x42 grid, K = N = 5120, rank 128) and the MX formats (MXFP4 W4A4, MXFP8
W8A8) on the attention-projection shape.

Timing: untimed steps for `--settle-ms` of wall time (the GPU's clock ramps up over tens of
milliseconds of load; without this the first timed steps run several per cent slower than
the steady state), W warm-up steps, then exactly K timed steps between two synchronisations
(the step time, and per-kernel means from HIP events on the launch stream); then a separate
pass of `--stat-reps` steps gives each kernel's p10 / p50 / p90.  A plain streaming kernel
(libsvdq_probe.so) that reads X and writes as many bytes as the activation kernel writes is
timed the same way, as the measured bandwidth that kernel is compared against.
`--copy-probe` runs a plain 1 GiB device copy whose hardware byte counters calibrate the
per-kernel traffic figures.

Prints ONE JSON line: metric, value (TFLOP/s of the layer per step), per-kernel timings, the
roofline of the dominant kernel, and the CPU-oracle baseline.
"""
import argparse
import gc
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 SVDQuant linear TFLOP/s + % MFMA peak; quant kernel GB/s, 5120² M=16k"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 MFMA
PEAK_I8_TOPS = 5000.0         # MI355X dense int8 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense fp4 / fp6 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# Vector ALU, one fp32 lane operation per lane and clock without packed instructions: 256 CUs x
# 4 SIMDs x 16 lanes x 2.4 GHz, in tera-operations per second.
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
WORKLOADS = {"attn": 1, "attn-mxfp4": 1, "attn-mxfp8": 1, "mlp-up-int4": 2,
             "mlp-down-sweep": 3, "delta": 4}
MX_FORMATS = {"attn-mxfp4": (2, "mxfp4"), "attn-mxfp8": (3, "mxfp8")}
# Sources of each GEMM kernel: the PMC traffic figure is valid only for the source it was taken on.
GEMM_SOURCES = {"attn": ("gemm_w4a4.hip", "gemm_common.h", "device.h"),
                "mlp-up-int4": ("gemm_int4.hip", "gemm_common.h", "device.h"),
                "mlp-down-sweep": ("gemm_w4a4.hip", "gemm_common.h", "device.h"),
                "delta": ("gemm_w4a4.hip", "gemm_common.h", "device.h"),
                "attn-mxfp4": ("gemm_mx.hip", "gemm_common.h", "device.h"),
                "attn-mxfp8": ("gemm_mx.hip", "gemm_common.h", "device.h")}
GEMM_KERNELS = {"mlp-up-int4": "k_gemm_int4", "attn-mxfp4": "k_gemm_mxfp4",
                "attn-mxfp8": "k_gemm_mx_dma"}
SWEEP_MASKS = (0, 7, 2, 1)    # λ = 1, all rows, video rows, text rows
ROTATION_BYTES = 1 << 30      # at least this much of X is rotated through


def workload_config(workload):
    """The synthetic configuration of a workload (the MX ones: the attention projection in that
    format)."""
    import synth
    cfg = synth.config(WORKLOADS[workload])
    if workload in MX_FORMATS:
        cfg["fmt"] = MX_FORMATS[workload][1]
        cfg["name"] = f"{cfg['name']}-{cfg['fmt']}"
    return cfg


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "w4a4_quantized_dit_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per GEMM launch from the committed hardware-counter summary, if it was taken on
    the current kernel source; otherwise None."""
    kern = GEMM_KERNELS.get(workload, "k_gemm_nvfp4")
    name = workload_config(workload)["name"]
    path = os.path.join(ROOT, "profiles", f"{kern}_{name}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    dig = re.search(r"kernel source digest:\s*`?([0-9a-f]+)", text)
    val = re.search(r"traffic bytes per launch:\s*`?([0-9.eE+]+)", text)
    if not dig or not val or dig.group(1) != source_digest(GEMM_SOURCES[workload]):
        return None
    return float(val.group(1))


def gpu_cotenants():
    """Other processes holding a GPU context on this machine (the kernel module lists one directory per
    process under /sys/class/kfd/kfd/proc), read just before the timed steps; None where that
    listing does not exist."""
    root = "/sys/class/kfd/kfd/proc"
    try:
        pids = sorted(int(p) for p in os.listdir(root) if p.isdigit())
    except OSError:
        return None
    others = []
    for pid in pids:
        if pid == os.getpid():
            continue
        try:
            with open(f"/proc/{pid}/comm") as f:
                name = f.read().strip()
        except OSError:
            name = "?"
        others.append({"pid": pid, "name": name})
    return {"source": root, "count": len(others), "processes": others[:16]}


def percentiles(v):
    v = np.asarray(v, dtype=np.float64)
    return {"mean": round(float(v.mean()), 4), "p10": round(float(np.percentile(v, 10)), 4),
            "p50": round(float(np.percentile(v, 50)), 4),
            "p90": round(float(np.percentile(v, 90)), 4), "n": int(v.size)}


def lowrank_factors_gpu(torch, layer, Wd, lam, r, seed=0, power_iters=2, reps=5):
    """Rank-r factors of diag(λ)·Wᵀ for the benchmark inputs, computed by the library's
    randomized SVD (sketch of r + 8 seeded Gaussian columns, two power iterations), and its
    median time over `reps` calls (milliseconds; set-up, outside the timed step)."""
    N = Wd.shape[0]
    omega = torch.from_numpy(np.random.default_rng([seed, 9]).standard_normal((N, r + 8))
                             .astype(np.float32)).to("cuda")
    times = []
    for _ in range(reps + 1):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        down, up, _ = layer.lowrank_factors(Wd, lam, omega, r, power_iters)
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) * 1e3)
    return down, up, float(np.median(times[1:]))


def weight_side_gpu(torch, layer, st, fmt, seed=0):
    """One-off (set-up side, outside the timed step) times in milliseconds of the calibration
    search and GPTQ on the benchmark inputs: the 39-point λ grid scored on 1024 uniform rows
    with the rank-r branch, and GPTQ of the residual under the Hessian of 2048 rows."""
    cfg = st["cfg"]
    M, K, N, r = cfg["M"], cfg["K"], cfg["N"], cfg["r"]
    Xd, Wd = st["Xs"][0], st["Wd"]
    rng = np.random.default_rng([seed, 10])
    rows = torch.from_numpy(np.sort(rng.choice(M, 1024, replace=False)).astype(np.int32)).cuda()
    omega = torch.from_numpy(rng.standard_normal((N, r + 8)).astype(np.float32)).cuda()
    state = dict(ax=st["ax"], aw=st["aw"])
    grid = list(layer.ALPHA_GRID)
    t = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    layer.lambda_search(Xd, Wd, state, grid[:1], rows, fmt, omega, r)       # warm-up
    t[0].record()
    out = layer.lambda_search(Xd, Wd, state, grid, rows, fmt, omega, r)
    t[1].record()
    n_cal = min(2048, M)
    H = layer.gptq_hessian(Xd[:n_cal], st["lam"])
    t[2].record()
    layer.prepare_weight_gptq(Wd, st["lam"], st["downd"], st["upd"], H, fmt)
    t[3].record()
    torch.cuda.synchronize()
    return {"lambda_search_39": round(t[0].elapsed_time(t[1]), 2),
            "lambda_search_best_alpha": grid[int(out["index"].cpu()[0])],
            "gptq_hessian_2048_rows": round(t[1].elapsed_time(t[2]), 2),
            "gptq": round(t[2].elapsed_time(t[3]), 2)}


def _cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def cpu_baseline(cfg, X, W, down, up, rows):
    """The oracle, as it stands, on the first `rows` rows of the workload (whole weight)."""
    from oracle import calib as OC, layer as OL
    rows = min(rows, cfg["M"])
    s = cfg["seg"]
    seg = (0, min(s[1], rows), min(s[2], rows), rows)
    Xs = X[:rows]
    fmt = cfg["fmt"] if cfg["fmt"] in ("int4", "mxfp4", "mxfp8") else "nvfp4"
    t0 = time.perf_counter()
    ax, aw, lam, amax = OC.calibrate(Xs, seg, W, 7)
    wt = OL.prepare_weight(W, lam, down, up, fmt)
    act = OL.prepare_activation(Xs, lam, amax, down, fmt)
    OL.forward(act, wt, up, fmt)
    dt = time.perf_counter() - t0
    K, N, r = cfg["K"], cfg["N"], cfg["r"]
    flops = 2.0 * rows * N * K + 2.0 * rows * K * r + 2.0 * rows * r * N
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{rows} of {cfg['M']} rows of the same workload, whole {N}x{K} weight "
                      f"(calibration, fp64 residual + quantisation, activation quantisation, "
                      f"float64 GEMM); {dt:.2f} s"}


def cpu_baseline_delta(cfg, X, W, down, up, frames):
    """The oracle, as it stands, on the DeltaQuant layer restricted to the text rows and the
    first `frames` video frames (whole cubes), with the whole weight."""
    from oracle import calib as OC, layer as OL, delta as DQ
    T, H, Wg = cfg["grid"]
    ct, ch, cw = cfg["cube"]
    frames = max(ct, (min(frames, T) // ct) * ct)
    nt = cfg["n_text"]
    rows = nt + frames * H * Wg
    Xs = X[:rows]
    seg = (0, nt, rows, rows)
    t0 = time.perf_counter()
    ax, aw, lam, amax = OC.calibrate(Xs, seg, W, 7)
    r2c, ptr, crow = DQ.cube_geometry(frames, H, Wg, ct, ch, cw, nt, 0, cfg["cube1d"])
    xhat = OC.smooth(Xs, lam)
    core = DQ.cube_core(xhat, ptr, crow)
    cc, cs = DQ.core_fp8(core)
    dc, dsc, gd, _ = DQ.delta_quantize(DQ.delta_rows(xhat, core, r2c), amax)
    wt = OL.prepare_weight(W, lam, down, up, "nvfp4")
    co = DQ.core_out_f64(cc, cs, wt["codes"], wt["scales"], wt["g"])
    from oracle import gemm as OG
    D = OG.lowrank_down(xhat, down)
    DQ.delta_linear(co, r2c, dc, dsc, gd, wt["codes"], wt["scales"], wt["g"], D, up)
    dt = time.perf_counter() - t0
    K, N, r = cfg["K"], cfg["N"], cfg["r"]
    nc = len(ptr) - 1
    flops = 2.0 * rows * N * K + 2.0 * nc * N * K + 2.0 * rows * K * r + 2.0 * rows * r * N
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{rows} of {cfg['M']} rows ({nt} text rows and video frames 0..{frames - 1}"
                      f" in whole cubes, {nc} cubes), whole {N}x{K} weight (calibration, cube "
                      f"cores, FP8 core, NVFP4 delta, weight preparation, core and delta "
                      f"float64 GEMMs); {dt:.2f} s"}


def cpu_weight_side(st, fmt_name, seed=0):
    """The oracle, as it stands, on bounded samples of the weight-side work: one λ candidate
    (randomized factors, residual quantisation, 1024 sampled rows, score) and GPTQ of 32 weight
    rows under the Hessian of 2048 activation rows (Hessian and inverse factor included)."""
    from oracle import search as OSe, gptq as OG, calib as OC, svd as OS
    cfg = st["cfg"]
    M, K, N, r = cfg["M"], cfg["K"], cfg["N"], cfg["r"]
    X, W = st["X"], st["W"]
    ax = st["ax"].cpu().numpy()
    aw = st["aw"].cpu().numpy()
    rng = np.random.default_rng([seed, 10])
    rows = np.sort(rng.choice(M, 1024, replace=False))
    omega = rng.standard_normal((N, r + 8)).astype(np.float32)
    t0 = time.perf_counter()
    OSe.candidate(X, W, ax, aw, 7, np.float32(0.5), fmt_name, rows, omega, r, 2)
    t_cand = time.perf_counter() - t0
    lam = OC.lambda_from_stats(ax, aw, 7, 0.5)
    t0 = time.perf_counter()
    H = OG.hessian(X[:min(2048, M)], lam)
    R32 = OS.residual_f32(W[:32], lam, st["down"], st["up"][:32])
    OG.gptq_quantize(R32, H, fmt_name if fmt_name != "nvfp4-delta" else "nvfp4")
    t_gptq = time.perf_counter() - t0
    return {"lambda_candidates_per_s": round(1.0 / t_cand, 4), "candidate_s": round(t_cand, 2),
            "gptq_weight_rows_per_s": round(32.0 / t_gptq, 2), "gptq_32_rows_s": round(t_gptq, 2),
            "cores": _cores(), "kind": "oracle",
            "sample": "one λ candidate on 1024 rows; GPTQ of 32 weight rows (Hessian of 2048 rows "
                      "and its inverse Cholesky factor included)"}


def copy_probe(torch, nbytes=1 << 30, reps=3):
    """A plain elementwise device kernel that reads `nbytes` and writes `nbytes` per launch."""
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": nbytes, "launches": reps}), flush=True)


def copy_mix_rate(torch, Xs, write_bytes, reps):
    """Measured bandwidth of a plain streaming copy with the activation kernel's byte mix: the
    library's memory probe reads all of X (16-byte nontemporal loads) and writes `write_bytes`
    (the kernel's codes, scales and D) in the same pass, rotating over the same copies of X.
    Returns (GB/s of the median launch, dict of ms percentiles)."""
    import ctypes
    from w4a4_quantized_dit_amd import build as B
    lib = ctypes.CDLL(B.PROBE_LIB)
    fn = lib.svdq_probe_stream
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_void_p]
    M, K = Xs[0].shape
    rd = M * K * 2
    wr = (write_bytes + 15) // 16 * 16
    dst = torch.empty(max(wr, 16), dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def launch(i):
        if fn(Xs[i % len(Xs)].data_ptr(), rd, dst.data_ptr(), wr, s) != 0:
            raise RuntimeError("memory probe launch failed")
    for i in range(3):
        launch(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(reps):
        launch(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    return (rd + wr) / (np.median(ms) * 1e-3) / 1e9, percentiles(ms)


def to_dev(torch, bits):
    return torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)


def setup(torch, workload):
    """Inputs, outputs and the per-step launch list of one workload."""
    import synth
    from w4a4_quantized_dit_amd import _lib
    from w4a4_quantized_dit_amd import layer
    cfg = workload_config(workload)
    M, K, N, r = cfg["M"], cfg["K"], cfg["N"], cfg["r"]
    seg = cfg["seg"]
    dev = "cuda"
    print(f"[bench] generating {cfg['name']} inputs", file=sys.stderr, flush=True)
    X = synth.x_bits(cfg)
    W = synth.weight_bits(N, K)
    Xd0, Wd = to_dev(torch, X), to_dev(torch, W)
    n_rot = max(1, math.ceil(ROTATION_BYTES / (M * K * 2)))
    Xs = [Xd0] + [Xd0.clone() for _ in range(n_rot - 1)]
    ax = torch.empty(3, K, device=dev); aw = torch.empty(K, device=dev)
    lam = torch.empty(K, device=dev); amax = torch.empty(1, device=dev)
    _lib.svdq_calibrate_lambda(Xd0, seg, Wd, 7, 0.5, 0, ax, aw, lam, amax)
    downd, upd, lowrank_ms = lowrank_factors_gpu(torch, layer, Wd, lam, r)
    down = downd.view(torch.int16).cpu().numpy().view(np.uint16)
    up = upd.view(torch.int16).cpu().numpy().view(np.uint16)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    u8 = torch.uint8
    st = dict(cfg=cfg, X=X, W=W, down=down, up=up, Y=Y, lowrank_ms=lowrank_ms, Wd=Wd, ax=ax,
              aw=aw, lam=lam, downd=downd, upd=upd, n_rot=n_rot)
    flops_one = 2.0 * M * N * K + 2.0 * M * r * N

    def cal(Xi):
        _lib.svdq_calibrate_lambda(Xi, seg, Wd, 7, 0.5, 0, ax, aw, lam, amax)

    if workload in ("attn", "delta", "mlp-down-sweep"):
        w_codes = torch.empty(N, K // 2, dtype=u8, device=dev)
        w_scales = torch.empty(N, K // 16, dtype=u8, device=dev)
        g_w = torch.empty(1, device=dev)
        # the residual formed once and kept in a workspace between the amax and the codes
        nb = _lib.svdq_quantize_weight_workspace_bytes(0, N, K)
        wbuf = torch.empty(nb + 256, dtype=u8, device=dev)
        woff = (-wbuf.data_ptr()) % 256
        wq_ws = wbuf[woff:woff + nb]

        def wq(Xi):
            _lib.svdq_quantize_weight_ws(0, Wd, lam, downd, upd, r, w_codes, w_scales, g_w, wq_ws)
    if workload in ("attn", "mlp-down-sweep"):
        a_codes = torch.empty(M, K // 2, dtype=u8, device=dev)
        a_scales = torch.empty(M, K // 16, dtype=u8, device=dev)
        g_a = torch.empty(1, device=dev)
        D = torch.empty(M, r, device=dev)
        st["qa_bytes"] = M * K * 2 + M * K // 2 + M * K // 16 + M * r * 4 + r * K * 2 + K * 4
        st["gemm_peak"] = PEAK_F16_TFLOPS
    if workload == "attn":
        def qa(Xi):
            _lib.svdq_quant_act_lowrank_down(0, Xi, lam, amax, downd, r, a_codes, a_scales, g_a, D)

        def gemm(Xi):
            _lib.svdq_w4a4_gemm(0, M, N, K, a_codes, a_scales, g_a, w_codes, w_scales, g_w, D,
                                upd, r, Y)
        st["steps"] = [("cal", cal), ("wq", wq), ("qa", qa), ("gemm", gemm)]
        st["gemm_flops"] = flops_one
        st["layer_flops"] = flops_one + 2.0 * M * K * r
    elif workload == "mlp-down-sweep":
        # per λ choice: its own factors (set-up), then calibration under its mask, weight and
        # activation quantisation, the GEMM and the per-modality scoring on the sampled rows
        rows, grp = synth.sample_rows(seg, n_per=4096, seed=0)
        rows_d = torch.from_numpy(rows).to(dev)
        grp_d = torch.from_numpy(grp).to(dev)
        sums = {m: torch.zeros(8, dtype=torch.float64, device=dev) for m in SWEEP_MASKS}
        factors = {}
        for m in SWEEP_MASKS:
            lam_m = torch.empty(K, device=dev)
            _lib.svdq_calibrate_lambda(Xd0, seg, Wd, m, 0.5, 0, ax, aw, lam_m, amax)
            factors[m] = lowrank_factors_gpu(torch, layer, Wd, lam_m, r, reps=1)[:2]
        # the bf16 reference rows of the batch's sampled rows do not depend on λ: computed once
        # per step, and every λ is scored against them
        Yref = torch.empty(len(rows), N, dtype=torch.bfloat16, device=dev)

        def ref_rows(Xi):
            _lib.svdq_score_reference_rows(Xi, Wd, rows_d, Yref)
        steps = [("ref", ref_rows)]
        for m in SWEEP_MASKS:
            fd, fu = factors[m]

            def cal_m(Xi, m=m):
                _lib.svdq_calibrate_lambda(Xi, seg, Wd, m, 0.5, 0, ax, aw, lam, amax)

            def wq_m(Xi, fd=fd, fu=fu):
                _lib.svdq_quantize_weight_ws(0, Wd, lam, fd, fu, r, w_codes, w_scales, g_w, wq_ws)

            def qa_m(Xi, fd=fd):
                _lib.svdq_quant_act_lowrank_down(0, Xi, lam, amax, fd, r, a_codes, a_scales,
                                                 g_a, D)

            def gemm_m(Xi, fu=fu):
                _lib.svdq_w4a4_gemm(0, M, N, K, a_codes, a_scales, g_a, w_codes, w_scales, g_w,
                                    D, fu, r, Y)

            def score_m(Xi, m=m):
                sums[m].zero_()
                _lib.svdq_score_modal_rel_l2_ref(Y, Yref, rows_d, grp_d, sums[m])
            steps += [("cal", cal_m), ("wq", wq_m), ("qa", qa_m), ("gemm", gemm_m),
                      ("score", score_m)]
        st["steps"] = steps
        st["sweep_sums"] = sums
        st["score_rows"] = int(len(rows))
        st["gemm_flops"] = flops_one
        st["layer_flops"] = len(SWEEP_MASKS) * (flops_one + 2.0 * M * K * r)
    elif workload in MX_FORMATS:
        f = MX_FORMATS[workload][0]
        w_codes, w_scales, _ = layer._alloc_codes_scales(f, N, K, dev)
        a_codes, a_scales, _ = layer._alloc_codes_scales(f, M, K, dev)
        D = torch.empty(M, r, device=dev)

        def wq(Xi):
            _lib.svdq_quantize_weight(f, Wd, lam, downd, upd, r, w_codes, w_scales, None)

        def qa(Xi):
            _lib.svdq_quant_act_lowrank_down(f, Xi, lam, None, downd, r, a_codes, a_scales, None,
                                             D)

        def gemm(Xi):
            _lib.svdq_w4a4_gemm(f, M, N, K, a_codes, a_scales, None, w_codes, w_scales, None, D,
                                upd, r, Y)
        st["steps"] = [("cal", cal), ("wq", wq), ("qa", qa), ("gemm", gemm)]
        code_bytes = M * K if f == 3 else M * K // 2
        st["qa_bytes"] = M * K * 2 + code_bytes + M * K // 32 + M * r * 4 + r * K * 2 + K * 4
        st["gemm_flops"] = flops_one
        st["layer_flops"] = flops_one + 2.0 * M * K * r
        st["gemm_peak"] = PEAK_FP8_TFLOPS if f == 3 else PEAK_FP4_TFLOPS
    elif workload == "mlp-up-int4":
        w_codes = torch.empty(N, K // 2, dtype=u8, device=dev)
        w_scales = torch.empty(N, K // 64, dtype=torch.float16, device=dev)
        a_codes = torch.empty(M, K // 2, dtype=u8, device=dev)
        a_scales = torch.empty(M, K // 64, dtype=torch.float16, device=dev)
        D = torch.empty(M, r, device=dev)

        def wq(Xi):
            _lib.svdq_quantize_weight(1, Wd, lam, downd, upd, r, w_codes, w_scales, None)

        def qa(Xi):
            _lib.svdq_quant_act_lowrank_down(1, Xi, lam, None, downd, r, a_codes, a_scales, None,
                                             D)

        def gemm(Xi):
            _lib.svdq_w4a4_gemm(1, M, N, K, a_codes, a_scales, None, w_codes, w_scales, None, D,
                                upd, r, Y)
        st["steps"] = [("cal", cal), ("wq", wq), ("qa", qa), ("gemm", gemm)]
        st["qa_bytes"] = M * K * 2 + M * K // 2 + M * K // 32 + M * r * 4 + r * K * 2 + K * 4
        st["gemm_flops"] = flops_one
        st["layer_flops"] = flops_one + 2.0 * M * K * r
        st["gemm_peak"] = PEAK_I8_TOPS
    else:  # delta
        T, H, Wg = cfg["grid"]
        geo = layer.cube_geometry(T, H, Wg, *cfg["cube"], cfg["n_text"], cfg["n_audio"],
                                  cfg["cube1d"])
        nc = geo["n_cubes"]
        r2c_d = geo["row_to_cube"]
        dq = layer.delta_quantize_activation(Xd0, lam, amax, geo, downd)
        core_out = torch.empty(nc, N, device=dev)

        def qa(Xi):
            layer.delta_quantize_activation(Xi, lam, amax, geo, downd, out=dq)

        def core(Xi):
            _lib.svdq_gemm_core(nc, N, K, dq["cc"], dq["cs"], w_codes, w_scales, g_w, core_out)

        def gemm(Xi):
            _lib.svdq_w4a4_gemm(0, M, N, K, dq["dc"], dq["dsc"], dq["gd"], w_codes, w_scales, g_w,
                                dq["D"], upd, r, Y, core_out=core_out, row_to_cube=r2c_d)
        st["steps"] = [("cal", cal), ("wq", wq), ("qa", qa), ("core", core), ("gemm", gemm)]
        st["qa_bytes"] = (M * K * 2 + nc * K + nc * 4 + M * K // 2 + M * K // 16 + M * r * 4
                          + r * K * 2 + K * 4)
        st["gemm_flops"] = flops_one
        st["core_flops"] = 2.0 * nc * N * K
        st["layer_flops"] = flops_one + 2.0 * M * K * r + st["core_flops"]
        st["gemm_peak"] = PEAK_F16_TFLOPS
    st["Xs"] = Xs
    return st


def run_steps(torch, st, n, warm, record, settle_s=0.0):
    """Clock settling (untimed steps until `settle_s` seconds of them have run), `warm` warm-up
    steps, then n steps; with `record`, HIP events around every launch.  Returns (wall seconds
    of the n steps, {kernel name: [ms of every launch]}).

    The GPU's power management slows the first milliseconds of work that follow an idle gap,
    so all host-side preparation (event creation, garbage collection) happens while earlier
    work is still queued, and the only idle moment before the measured steps is the
    synchronisation that opens them."""
    names = [nm for nm, _ in st["steps"]]
    n_rot = len(st["Xs"])
    evs = None
    if record:
        # every event exists and has been recorded once before the measured region: the first
        # creation of a timing event costs tens of milliseconds of host time
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
               for _ in range(n)]
        for e in evs:
            for x in e:
                x.record()

    def one(i):
        for _, fn in st["steps"]:
            fn(st["Xs"][i % n_rot])

    # the collector runs before the settling steps, not after them: a collection takes tens of
    # milliseconds, long enough for the GPU to drain its queue and idle, and the launches that
    # follow such an idle gap run slower for a while
    gc.collect()
    gc.disable()           # no collector pause from here to the end of the measured region
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < settle_s:
        one(i)         # no synchronisation: once the launch queue is full the host waits in it
        i += 1
    for j in range(warm):
        one(i + j)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        Xi = st["Xs"][i % n_rot]
        if record:
            e = evs[i]
            e[0].record()
            for j, (_, fn) in enumerate(st["steps"]):
                fn(Xi)
                e[j + 1].record()
        else:
            for _, fn in st["steps"]:
                fn(Xi)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    per = {nm: [] for nm in names}
    if record:
        for e in evs:
            for j, nm in enumerate(names):
                per[nm].append(e[j].elapsed_time(e[j + 1]))
    return wall, per


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--stat-reps", type=int, default=50,
                    help="steps of the separate pass that gives per-kernel p10/p50/p90 "
                         "(0: skip)")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="attn")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps run before the warm-up until this much wall time has "
                         "passed, so that the timed steps run at the GPU's settled clock")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--weight-side", action="store_true",
                    help="also time the one-off λ search and GPTQ (after the timed steps; their "
                         "small GEMMs then share the kernel names of the step's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer is "
              "data-parallel over rows and the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from w4a4_quantized_dit_amd import _lib

    _lib.load()
    if args.copy_probe:
        copy_probe(torch)
        return
    st = setup(torch, args.workload)
    cfg = st["cfg"]
    M, K, N, r = cfg["M"], cfg["K"], cfg["N"], cfg["r"]
    seg = cfg["seg"]
    names = list(dict.fromkeys(nm for nm, _ in st["steps"]))

    cotenants = gpu_cotenants()
    print("[bench] warmup + timed steps", file=sys.stderr, flush=True)
    wall, per = run_steps(torch, st, args.steps, args.warmup, record=True,
                          settle_s=args.settle_ms * 1e-3)
    ms = {k: float(np.mean(v)) for k, v in per.items()}
    ms_step = wall * 1e3 / args.steps
    stats = None
    if args.stat_reps > 0:
        print(f"[bench] {args.stat_reps} steps for the per-kernel distribution", file=sys.stderr,
              flush=True)
        _, per2 = run_steps(torch, st, args.stat_reps, 1, record=True,
                            settle_s=min(0.1, args.settle_ms * 1e-3))
        stats = {k: percentiles(v) for k, v in per2.items()}
    print("[bench] copy probe with the activation kernel's byte mix", file=sys.stderr, flush=True)
    copy_gbs, copy_ms = copy_mix_rate(torch, st["Xs"], st["qa_bytes"] - M * K * 2,
                                      max(args.stat_reps, 20))

    gemm_flops = st["gemm_flops"]
    layer_flops = st["layer_flops"]
    fwd_ms = ms["qa"] + ms["gemm"] + ms.get("core", 0.0)
    n_fwd = len(SWEEP_MASKS) if args.workload == "mlp-down-sweep" else 1
    gemm_tflops = gemm_flops / (ms["gemm"] * 1e-3) / 1e12
    peak = st["gemm_peak"]
    qa_gbs = st["qa_bytes"] / (ms["qa"] * 1e-3) / 1e9
    qa_gbs_p50 = st["qa_bytes"] / (stats["qa"]["p50"] * 1e-3) / 1e9 if stats else None
    gemm_tflops_p50 = gemm_flops / (stats["gemm"]["p50"] * 1e-3) / 1e12 if stats else None
    dtype = {"attn": "f16", "mlp-up-int4": "i8", "delta": "f16", "attn-mxfp4": "fp4",
             "attn-mxfp8": "fp8", "mlp-down-sweep": "f16"}[args.workload]
    lam_desc = ("each of lambda = 1, all rows, video rows, text rows (alpha 0.5)"
                if args.workload == "mlp-down-sweep" else "all rows, alpha 0.5")
    out = {
        "metric": METRIC,
        "value": round(layer_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded outlier-channel activations, N(0,1/K) weights)"
                if cfg["gen"] == "outlier" else
                "synthetic (seeded cube-mean field plus noise, N(0,1/K) weights)",
        "config": {"workload": cfg["name"], "M": M, "K": K, "N": N, "rank": r,
                   "format": cfg["fmt"], "rows_text_video_audio": [seg[1], seg[2] - seg[1],
                                                                 seg[3] - seg[2]],
                   "lambda": lam_desc, "step": " + ".join(nm for nm, _ in st["steps"]),
                   "x_copies_rotated": st["n_rot"]},
        "gpu_cotenants": cotenants,
        "kernels_ms": {k: round(v, 4) for k, v in ms.items()},
        "kernel_stats_ms": stats,
        "lowrank_factors_ms": round(st["lowrank_ms"], 3),
        "forward_tflops": round(n_fwd * (gemm_flops + 2.0 * M * K * r + st.get("core_flops", 0.0))
                                / (n_fwd * fwd_ms * 1e-3) / 1e12, 2),
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_tflops_p50": round(gemm_tflops_p50, 2) if gemm_tflops_p50 else None,
        "gemm_frac_of_mfma_peak": round(gemm_tflops / peak, 4),
        "gemm_frac_of_fp4_peak": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
        "quant_act_gbs": round(qa_gbs, 1),
        "quant_act_gbs_p50": round(qa_gbs_p50, 1) if qa_gbs_p50 else None,
        "quant_act_frac_of_hbm": round(qa_gbs / PEAK_HBM_GBS, 4),
        "copy_mix_gbs": round(copy_gbs, 1),
        "copy_mix_ms": copy_ms,
        "quant_act_frac_of_copy": round(qa_gbs / copy_gbs, 4),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / peak, 4),
                     "traffic": measured_traffic(args.workload)},
    }
    if args.workload == "mlp-up-int4":
        # The exact int4 route rescales every 64-group partial sum of every output element on
        # the vector ALU (convert, scale product, fused multiply-add): that, not the MFMA, bounds
        # the kernel, so its roofline is the vector ALU's lane-operation rate.
        valu_tops = 3.0 * M * N * (K // 64) / (ms["gemm"] * 1e-3) / 1e12
        out["roofline"] = {"bound": "alu", "achieved": round(valu_tops, 2),
                           "peak": round(PEAK_VALU_TOPS, 2), "unit": "TOP/s",
                           "frac": round(valu_tops / PEAK_VALU_TOPS, 4),
                           "traffic": measured_traffic(args.workload)}
    if "core" in ms:
        out["core_gemm_tflops"] = round(st["core_flops"] / (ms["core"] * 1e-3) / 1e12, 2)
    if args.workload == "mlp-down-sweep":
        scores = {}
        for m, s in st["sweep_sums"].items():
            v = s.cpu().numpy().reshape(4, 2)
            rel = np.sqrt(v[:, 0]) / np.sqrt(v[:, 1])
            scores[{0: "lambda1", 7: "all", 2: "video", 1: "text"}[m]] = {
                g: round(float(x), 5) for g, x in zip(("text", "video", "audio", "uniform"), rel)}
        out["sweep_rel_l2"] = scores
        out["score_rows_per_lambda"] = st["score_rows"]
    if args.weight_side:
        from w4a4_quantized_dit_amd import layer
        print("[bench] weight side: λ search and GPTQ", file=sys.stderr, flush=True)
        fmt = {"nvfp4": 0, "nvfp4-delta": 0, "int4": 1, "mxfp4": 2, "mxfp8": 3}[cfg["fmt"]]
        ws = weight_side_gpu(torch, layer, st, fmt)
        out["weight_side_ms"] = ws
        out["weight_side_rates"] = {
            "lambda_candidates_per_s": round(39.0 / (ws["lambda_search_39"] * 1e-3), 2),
            "gptq_weight_rows_per_s": round(N / ((ws["gptq_hessian_2048_rows"] + ws["gptq"]) * 1e-3),
                                            1)}
        if not args.no_cpu_baseline:
            print("[bench] weight side on the cpu (oracle)", file=sys.stderr, flush=True)
            fmt_name = "nvfp4" if cfg["fmt"] == "nvfp4-delta" else cfg["fmt"]
            out["weight_side_cpu_baseline"] = cpu_weight_side(st, fmt_name)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        if cfg["fmt"] == "nvfp4-delta":
            out["cpu_baseline"] = cpu_baseline_delta(cfg, st["X"], st["W"], st["down"], st["up"],
                                                     frames=args.cpu_rows or 2)
        else:
            rows = args.cpu_rows or {1: 16384, 2: 4096, 3: 2048}.get(WORKLOADS[args.workload],
                                                                       4096)
            out["cpu_baseline"] = cpu_baseline(cfg, st["X"], st["W"], st["down"], st["up"],
                                               rows=rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
