"""Builds the gfx950 shared library libsvdq.so in-tree with hipcc.

Usage: python -m w4a4_quantized_dit_amd.build   (or build() from Python)
"""
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsvdq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "geometry.cpp", "calib.hip", "quant_weight.hip", "quant_act.hip",
           "gemm_w4a4.hip", "gemm_int4.hip", "gemm_mx.hip", "delta.hip", "score.hip",
           "lowrank.hip", "search.hip", "gptq.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # codes are defined by IEEE single operations in a fixed order: no contraction, exact
    # division and square root, denormals kept
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 instructions are not used on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose=False, out=None, defines=()):
    """Compile every source into libsvdq.so (always recompiles).  `out` / `defines` build a
    differently named library with extra -D tuning definitions."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    target = out or LIB
    tmp = target + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + srcs + ["-o", tmp]
    t0 = time.time()
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, target)
    if verbose:
        print(f"built {target} in {time.time() - t0:.1f}s")
    return target


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
