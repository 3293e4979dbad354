"""Builds the gfx950 shared library libsvdq.so in-tree with hipcc.

Every source is compiled to an object file in parallel (one hipcc per source), then the objects
are linked into the shared library.

Usage: python -m w4a4_quantized_dit_amd.build   (or build() from Python)
"""
import os
import shutil
import subprocess
import sys
import tempfile
import time
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsvdq.so")
PROBE_LIB = os.path.join(HERE, "libsvdq_probe.so")   # the benchmark's memory probe
PROBE_SOURCES = ["probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "geometry.cpp", "calib.hip", "quant_weight.hip", "quant_act.hip",
           "gemm_w4a4.hip", "gemm_int4.hip", "gemm_mx.hip", "delta.hip", "score.hip",
           "lowrank.hip", "search.hip", "gptq.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # codes are defined by IEEE single operations in a fixed order: no contraction, exact
    # division and square root, denormals kept
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 instructions are not used on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    return res.returncode, out


def build(verbose=False, out=None, defines=(), jobs=None):
    """Compile every source into libsvdq.so and the benchmark's probe into libsvdq_probe.so
    (always recompiles).  `out` / `defines` build a differently named layer library with extra
    -D definitions (and no probe)."""
    if out is None:
        _link(PROBE_SOURCES, PROBE_LIB, (), jobs, verbose)
    return _link(SOURCES, out or LIB, defines, jobs, verbose)


def _link(sources, target, defines, jobs, verbose):
    jobs = jobs or min(len(sources), max(1, (os.cpu_count() or 4)))
    t0 = time.time()
    tmpdir = tempfile.mkdtemp(prefix="svdq_build_")
    try:
        dflags = ["-D" + d for d in defines]

        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            rc, text = _run([HIPCC] + FLAGS + dflags + ["-c", os.path.join(CSRC, src), "-o", obj])
            return src, obj, rc, text

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(compile_one, sources))
        errors = [f"== {src} ==\n{text}" for src, _, rc, text in results if rc != 0]
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp = target + ".tmp"
        rc, text = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"]
                        + [obj for _, obj, _, _ in results] + ["-o", tmp])
        if rc != 0:
            raise RuntimeError("link failed:\n" + text)
        if verbose:
            for src, _, _, text in results:
                if text.strip():
                    print(f"== {src} ==\n{text}")
        os.replace(tmp, target)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    if verbose:
        print(f"built {target} in {time.time() - t0:.1f}s")
    return target


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
