"""CPU oracle for the SVDQuant W4A4 linear layer of a packed [text | video | audio] video DiT.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct CPU statement of
what the GPU path computes: smoothing, λ calibration, truncated SVD, NVFP4 / int4
round-to-nearest-even quantisation, the MX (E8M0 per 32) variant, a float64 GEMM, per-modality scoring and the DeltaQuant
(cube core + delta) variant.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import it.  It shares no code with the HIP library and imports nothing from it.

Sources (cited by page title and section):
  * "MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on", sections
    "Why" (NVFP4: one E4M3 scale, from the block maximum, per 16 consecutive channels; the
    kernel sees X / λ; the statistics-only bits-lost proxy), "Calibration" (activation
    statistics accumulated under a modality mask feed λ), "The metric that picks the winner also hides the cost" (uniform-row and
    per-modality relative L2).
  * "MiniMax-H3 · SVDQuant W4A4 (int4, rank 32, GPTQ)", opening paragraph (outliers absorbed
    by a 16-bit low-rank branch, 4-bit residual, activations quantised per token at run time).
  * "MiniMax-H3 — MXFP8 (weight-quantized, vLLM-Omni native layout)", section "Quant format"
    (E4M3 elements, E8M0 scale per 32, round to nearest, dynamic activations): the MX variant.
  * "DeltaQuant on MiniMax-H3", sections "Why DeltaQuant does not beat SVDQuant here" (cube
    core + delta), "The audio win has a mechanism" (1-D cubes of consecutive rows for
    non-video rows), "The activation scale bound held" (|x − core| ≤ 2·max|x|, saturated
    groups counted at run time) and "Deviations from the paper" (core branch not on the
    FP4 scaled dot).

Every reading taken where the pages are silent is listed in the module that takes it.
Float32 steps use numpy float32 operations (each one IEEE round-to-nearest-even); exact
steps use float64.
"""
from . import formats, quant, mx, calib, proxy, svd, gemm, delta, score, layer, search, gptq  # noqa: F401
