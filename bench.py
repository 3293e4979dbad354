#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 layer on one MI355X.

Default workload (the JSON line's `value`): the attention-projection-sized layer, M = 16384
packed rows (164 text / 16154 video / 66 audio), K = N = 5120, rank 32, NVFP4.  One step is the
whole per-batch path:
    λ calibration over the batch -> residual-weight quantisation -> activation quantisation
    with the low-rank down-projection -> W4A4 GEMM with the up-projection (bf16 out).
Inputs are seeded synthetic tensors resident in HBM before the timed region; copies of X are
rotated so the 256 MB last-level cache cannot serve the activation reads.

`--workload` also times the int4-g64 MLP up-projection (M = 32768, K = 5120, N = 13824), the
DeltaQuant cube-field layer (31x24x42 grid, K = N = 5120, rank 128) and the MX formats (MXFP4
W4A4, MXFP8 W8A8) on the attention-projection shape, for profiling; the
`--copy-probe` mode runs a plain 1 GiB device copy whose hardware byte counters calibrate the
per-kernel traffic figures.

Prints ONE JSON line: metric, value (TFLOP/s of the layer per step), per-kernel timings from
HIP events on the launch stream, the roofline of the dominant kernel, and the CPU-oracle
baseline.
"""
import argparse
import gc
import hashlib
import json
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
WORKLOADS = {"attn": 1, "attn-mxfp4": 1, "attn-mxfp8": 1, "mlp-up-int4": 2, "delta": 4}
MX_FORMATS = {"attn-mxfp4": (2, "mxfp4"), "attn-mxfp8": (3, "mxfp8")}
# Sources of each GEMM kernel: the PMC traffic figure is valid only for the source it was taken on.
GEMM_SOURCES = {"attn": ("gemm_w4a4.hip", "gemm_common.h", "device.h"),
                "mlp-up-int4": ("gemm_int4.hip", "gemm_common.h", "device.h"),
                "delta": ("gemm_w4a4.hip", "gemm_common.h", "device.h"),
                "attn-mxfp4": ("gemm_mx.hip", "gemm_common.h", "device.h"),
                "attn-mxfp8": ("gemm_mx.hip", "gemm_common.h", "device.h")}
GEMM_KERNELS = {"mlp-up-int4": "k_gemm_int4", "attn-mxfp4": "k_gemm_mxfp4",
                "attn-mxfp8": "k_gemm_mx_dma"}


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
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {cfg['M']} rows of the same workload, whole {N}x{K} weight "
                      f"(calibration, fp64 residual + quantisation, activation quantisation, "
                      f"float64 GEMM); {dt:.2f} s"}


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
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"lambda_candidates_per_s": round(1.0 / t_cand, 4), "candidate_s": round(t_cand, 2),
            "gptq_weight_rows_per_s": round(32.0 / t_gptq, 2), "gptq_32_rows_s": round(t_gptq, 2),
            "cores": cores, "kind": "oracle",
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


def to_dev(torch, bits):
    return torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)


def setup(torch, workload, n_rot):
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
              aw=aw, lam=lam, downd=downd, upd=upd)

    def cal(Xi):
        _lib.svdq_calibrate_lambda(Xi, seg, Wd, 7, 0.5, 0, ax, aw, lam, amax)

    if workload in ("attn", "delta"):
        w_codes = torch.empty(N, K // 2, dtype=u8, device=dev)
        w_scales = torch.empty(N, K // 16, dtype=u8, device=dev)
        g_w = torch.empty(1, device=dev)

        def wq(Xi):
            _lib.svdq_quantize_weight(0, Wd, lam, downd, upd, r, w_codes, w_scales, g_w)
    if workload == "attn":
        a_codes = torch.empty(M, K // 2, dtype=u8, device=dev)
        a_scales = torch.empty(M, K // 16, dtype=u8, device=dev)
        g_a = torch.empty(1, device=dev)
        D = torch.empty(M, r, device=dev)

        def qa(Xi):
            _lib.svdq_quant_act_lowrank_down(0, Xi, lam, amax, downd, r, a_codes, a_scales, g_a, D)

        def gemm(Xi):
            _lib.svdq_w4a4_gemm(0, M, N, K, a_codes, a_scales, g_a, w_codes, w_scales, g_w, D,
                                upd, r, Y)
        st["steps"] = [("cal", cal), ("wq", wq), ("qa", qa), ("gemm", gemm)]
        st["qa_bytes"] = M * K * 2 + M * K // 2 + M * K // 16 + M * r * 4 + r * K * 2 + K * 4
        st["gemm_flops"] = 2.0 * M * N * K + 2.0 * M * r * N
        st["gemm_peak"] = PEAK_F16_TFLOPS
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
        st["gemm_flops"] = 2.0 * M * N * K + 2.0 * M * r * N
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
        st["gemm_flops"] = 2.0 * M * N * K + 2.0 * M * r * N
        st["gemm_peak"] = PEAK_I8_TOPS
    else:  # delta
        T, H, Wg = cfg["grid"]
        r2c, ptr, crow = _lib.svdq_cube_geometry(T, H, Wg, *cfg["cube"], cfg["n_text"],
                                                 cfg["n_audio"], cfg["cube1d"])
        nc = len(ptr) - 1
        r2c_d = torch.from_numpy(r2c).to(dev)
        ptr_d, crow_d = torch.from_numpy(ptr).to(dev), torch.from_numpy(crow).to(dev)
        cc = torch.empty(nc, K, dtype=u8, device=dev)
        cs = torch.empty(nc, device=dev)
        dc = torch.empty(M, K // 2, dtype=u8, device=dev)
        dsc = torch.empty(M, K // 16, dtype=u8, device=dev)
        gd = torch.empty(1, device=dev)
        D = torch.empty(M, r, device=dev)
        core_out = torch.empty(nc, N, device=dev)

        def qa(Xi):
            _lib.svdq_delta_quant_act(Xi, lam, amax, ptr_d, crow_d, nc, downd, r, cc, cs, dc, dsc,
                                      gd, D)

        def core(Xi):
            _lib.svdq_gemm_core(nc, N, K, cc, cs, w_codes, w_scales, g_w, core_out)

        def gemm(Xi):
            _lib.svdq_w4a4_gemm(0, M, N, K, dc, dsc, gd, w_codes, w_scales, g_w, D, upd, r, Y,
                                core_out=core_out, row_to_cube=r2c_d)
        st["steps"] = [("cal", cal), ("wq", wq), ("qa", qa), ("core", core), ("gemm", gemm)]
        st["qa_bytes"] = (M * K * 2 + nc * K + nc * 4 + M * K // 2 + M * K // 16 + M * r * 4
                          + r * K * 2 + K * 4)
        st["gemm_flops"] = 2.0 * M * N * K + 2.0 * M * r * N
        st["core_flops"] = 2.0 * nc * N * K
        st["gemm_peak"] = PEAK_F16_TFLOPS
    st["Xs"] = Xs
    return st


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="attn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=16384)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--weight-side", action="store_true",
                    help="also time the one-off λ search and GPTQ (after the timed steps; their "
                         "small GEMMs then share the kernel names of the step's)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer is "
              "data-parallel over rows and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from w4a4_quantized_dit_amd import _lib

    _lib.load()
    if args.copy_probe:
        copy_probe(torch)
        return
    n_rot = 4
    st = setup(torch, args.workload, n_rot)
    cfg = st["cfg"]
    M, K, N, r = cfg["M"], cfg["K"], cfg["N"], cfg["r"]
    seg = cfg["seg"]
    names = [n for n, _ in st["steps"]]
    ev = {k: [] for k in names}

    # every timing event exists (and has been recorded once) before the timed region: the
    # first creation of a timing event costs tens of milliseconds of host time
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(args.steps)]
    for e in evs:
        for x in e:
            x.record()
    torch.cuda.synchronize()

    def step(i, record):
        Xi = st["Xs"][i % n_rot]
        if not record:
            for _, fn in st["steps"]:
                fn(Xi)
            return
        e = evs[i]
        e[0].record()
        for j, (name, fn) in enumerate(st["steps"]):
            fn(Xi)
            e[j + 1].record()
            ev[name].append((e[j], e[j + 1]))

    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    print("[bench] timed steps", file=sys.stderr, flush=True)
    gc.collect()
    gc.disable()           # no collector pause inside the timed region
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    ms_step = wall * 1e3 / args.steps

    gemm_flops = st["gemm_flops"]
    layer_flops = gemm_flops + 2.0 * M * K * r + st.get("core_flops", 0.0)
    fwd_ms = ms["qa"] + ms["gemm"] + ms.get("core", 0.0)
    gemm_tflops = gemm_flops / (ms["gemm"] * 1e-3) / 1e12
    peak = st["gemm_peak"]
    qa_gbs = st["qa_bytes"] / (ms["qa"] * 1e-3) / 1e9
    dtype = {"attn": "f16", "mlp-up-int4": "i8", "delta": "f16", "attn-mxfp4": "fp4",
             "attn-mxfp8": "fp8"}[args.workload]
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
                   "lambda": "all rows, alpha 0.5",
                   "step": " + ".join(names)},
        "kernels_ms": {k: round(v, 4) for k, v in ms.items()},
        "lowrank_factors_ms": round(st["lowrank_ms"], 3),
        "forward_tflops": round(layer_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_frac_of_mfma_peak": round(gemm_tflops / peak, 4),
        "gemm_frac_of_fp4_peak": round(gemm_tflops / 10100.0, 4),
        "quant_act_gbs": round(qa_gbs, 1),
        "quant_act_frac_of_hbm": round(qa_gbs / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / peak, 4),
                     "traffic": measured_traffic(args.workload)},
    }
    if "core" in ms:
        out["core_gemm_tflops"] = round(st["core_flops"] / (ms["core"] * 1e-3) / 1e12, 2)
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
            out["cpu_baseline"] = None
        else:
            out["cpu_baseline"] = cpu_baseline(cfg, st["X"], st["W"], st["down"], st["up"],
                                               rows=args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
