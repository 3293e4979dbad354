"""MI355X (gfx950) SVDQuant W4A4 linear layer: C-ABI library libsvdq.so plus a thin binding.

    from w4a4_quantized_dit_amd import layer
    cal = layer.calibrate(X, seg, W, mask=7)            # λ, act_amax (device tensors)
    pw = layer.prepare_weight(W, cal["lambda"], lora_down, lora_up, fmt=layer.NVFP4)
    Y = layer.forward(X, pw, cal["act_amax"], cal["lambda"], lora_down)

The raw entry points (same names as include/svdq.h) live in w4a4_quantized_dit_amd._lib.
"""
from ._lib import (NVFP4, INT4_G64, SvdqError, load, header_entry_points,  # noqa: F401
                   status_string, last_error)
