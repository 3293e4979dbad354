"""Seeded synthetic inputs for the W4A4 layer workloads.

This module only draws inputs (activations, weights, segment offsets, sampled rows, the
DeltaQuant video grid); it holds none of the layer's arithmetic.  Both the CPU oracle side and
the GPU side of every test and of the benchmark take their inputs from here, so the two see
identical bits.
"""
from .configs import CONFIGS, config, segments  # noqa: F401
from .gen import (profiles, weight_bits, x_bits, sample_rows, gen_cube_index,  # noqa: F401
                  to_bf16_bits, ROW_BLOCK)
