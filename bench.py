#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 layer on one MI355X.

One step = the whole per-batch path of the attention-projection-sized workload (M = 16384 packed
rows: 164 text / 16154 video / 66 audio, K = N = 5120, rank 32, NVFP4):
    λ calibration over the batch -> residual-weight quantisation -> activation quantisation
    with the low-rank down-projection -> W4A4 GEMM with the up-projection (bf16 out).
Inputs are seeded synthetic tensors resident in HBM before the timed region; four copies of X
are rotated so the 256 MB last-level cache cannot serve the activation reads.

Prints ONE JSON line (rank 0): metric, value (TFLOP/s of the layer per step), per-kernel
timings, the roofline of the dominant kernel, and the CPU-oracle baseline.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 SVDQuant linear TFLOP/s + % MFMA peak; quant kernel GB/s, 5120² M=16k"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16 / bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def lowrank_factors_rangefinder(W_bits, lam, r, seed=0):
    """Rank-r factors of diag(λ)·Wᵀ for the benchmark inputs: a seeded randomized range finder
    (two power iterations) in numpy, rounded to bf16.  Any rank-r pair is a valid input to the
    path; this one is close to the truncated SVD."""
    from synth import to_bf16_bits
    W = (W_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    A = (W * lam.astype(np.float64)[None, :]).T                 # K x N
    rng = np.random.default_rng([seed, 9])
    Q = np.linalg.qr(A @ rng.standard_normal((A.shape[1], r + 8)))[0]
    for _ in range(2):
        Q = np.linalg.qr(A @ (A.T @ Q))[0]
    U, s, Vt = np.linalg.svd(Q.T @ A, full_matrices=False)
    L1 = (Q @ U[:, :r]) * s[:r]
    L2 = Vt[:r]
    return to_bf16_bits(L1.T), to_bf16_bits(L2.T)


def cpu_baseline(cfg, X, W, lam_np, down, up, rows=512):
    """The oracle, as it stands, on the first `rows` rows of the workload (whole weight)."""
    from oracle import calib as OC, layer as OL
    seg = (0, min(cfg["seg"][1], rows), rows, rows)
    Xs = X[:rows]
    t0 = time.perf_counter()
    ax, aw, lam, amax = OC.calibrate(Xs, seg, W, 7)
    wt = OL.prepare_weight(W, lam, down, up, "nvfp4")
    act = OL.prepare_activation(Xs, lam, amax, down, "nvfp4")
    OL.forward(act, wt, up, "nvfp4")
    dt = time.perf_counter() - t0
    K, N, r = cfg["K"], cfg["N"], cfg["r"]
    flops = 2.0 * rows * N * K + 2.0 * rows * K * r + 2.0 * rows * r * N
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {cfg['M']} rows of the same workload, whole 5120x5120 weight "
                      f"(calibration, fp64 residual + quantisation, activation quantisation, "
                      f"float64 GEMM); {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=512)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer is "
              "data-parallel over rows and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from w4a4_quantized_dit_amd import layer, _lib

    _lib.load()
    cfg = synth.config(1)
    M, K, N, r = cfg["M"], cfg["K"], cfg["N"], cfg["r"]
    seg = cfg["seg"]
    print(f"[bench] generating {cfg['name']} inputs", file=sys.stderr, flush=True)
    X = synth.x_bits(cfg)
    W = synth.weight_bits(N, K)
    dev = torch.device("cuda:0")
    Xd0 = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
    Wd = torch.from_numpy(W.view(np.int16)).to(dev).view(torch.bfloat16)
    n_rot = 4
    Xs = [Xd0] + [Xd0.clone() for _ in range(n_rot - 1)]

    cal = layer.calibrate(Xd0, seg, Wd, 7)
    lam_np = cal["lambda"].cpu().numpy()
    down, up = lowrank_factors_rangefinder(W, lam_np, r)
    downd = torch.from_numpy(down.view(np.int16)).to(dev).view(torch.bfloat16)
    upd = torch.from_numpy(up.view(np.int16)).to(dev).view(torch.bfloat16)

    # outputs preallocated once
    ax = torch.empty(3, K, device=dev); aw = torch.empty(K, device=dev)
    lam = torch.empty(K, device=dev); amax = torch.empty(1, device=dev)
    w_codes = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
    w_scales = torch.empty(N, K // 16, dtype=torch.uint8, device=dev)
    g_w = torch.empty(1, device=dev)
    a_codes = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
    a_scales = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
    g_a = torch.empty(1, device=dev)
    D = torch.empty(M, r, dtype=torch.float32, device=dev)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

    ev = {k: [] for k in ("cal", "wq", "qa", "gemm")}

    def step(i, record):
        Xi = Xs[i % n_rot]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if record: e[0].record()
        _lib.svdq_calibrate_lambda(Xi, seg, Wd, 7, 0.5, 0, ax, aw, lam, amax)
        if record: e[1].record()
        _lib.svdq_quantize_weight(0, Wd, lam, downd, upd, r, w_codes, w_scales, g_w)
        if record: e[2].record()
        _lib.svdq_quant_act_lowrank_down(0, Xi, lam, amax, downd, r, a_codes, a_scales, g_a, D)
        if record: e[3].record()
        _lib.svdq_w4a4_gemm(0, M, N, K, a_codes, a_scales, g_a, w_codes, w_scales, g_w, D, upd,
                            r, Y)
        if record:
            e[4].record()
            for k, (a, b) in zip(("cal", "wq", "qa", "gemm"), zip(e[:-1], e[1:])):
                ev[k].append((a, b))

    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    print("[bench] timed steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in ev.items()}
    ms_step = wall * 1e3 / args.steps

    gemm_flops = 2.0 * M * N * K + 2.0 * M * r * N
    layer_flops = gemm_flops + 2.0 * M * K * r
    qa_bytes = M * K * 2 + M * K // 2 + M * K // 16 + M * r * 4 + r * K * 2 + K * 4
    gemm_tflops = gemm_flops / (ms["gemm"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(layer_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded outlier-channel activations, N(0,1/K) weights)",
        "config": {"workload": cfg["name"], "M": M, "K": K, "N": N, "rank": r,
                   "format": "nvfp4", "rows_text_video_audio": [seg[1], seg[2] - seg[1],
                                                                 seg[3] - seg[2]],
                   "lambda": "all rows, alpha 0.5",
                   "step": "calibrate + weight quant + act quant/low-rank down + W4A4 GEMM"},
        "kernels_ms": {k: round(v, 4) for k, v in ms.items()},
        "forward_tflops": round(layer_flops / ((ms["qa"] + ms["gemm"]) * 1e-3) / 1e12, 2),
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_frac_of_f16_peak": round(gemm_tflops / PEAK_F16_TFLOPS, 4),
        "gemm_frac_of_fp4_peak": round(gemm_tflops / 10100.0, 4),
        "quant_act_gbs": round(qa_bytes / (ms["qa"] * 1e-3) / 1e9, 1),
        "quant_act_frac_of_hbm": round(qa_bytes / (ms["qa"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2),
                     "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_F16_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, X, W, lam_np, down, up, rows=args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
