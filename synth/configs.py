"""The five workloads (sizes, formats, λ choices) of the W4A4 layer.

Modality split of the packed sequence: text ≈1 %, video ≈98.6 %, audio ≈0.4 %, contiguous in
that order ("MiniMax-H3 NVFP4 — what the smoothing scale should be calibrated on", opening and
"The metric that picks the winner also hides the cost" sections give video 98.6 % and text
≈1-1.4 %).  Reading: n_text = round(0.01·M), n_audio = round(0.004·M), video = the rest.

λ choices are modality masks: bit 0 text, bit 1 video, bit 2 audio; 0 means λ = 1.
"""

MASK_NONE, MASK_TEXT, MASK_VIDEO, MASK_AUDIO, MASK_ALL = 0, 1, 2, 4, 7


def segments(M, n_text=None, n_audio=None):
    """Offsets {0, n_text, n_text + n_video, M} of the contiguous [text | video | audio] rows."""
    if n_text is None:
        n_text = round(0.01 * M)
    if n_audio is None:
        n_audio = round(0.004 * M)
    n_video = M - n_text - n_audio
    if n_video < 0:
        raise ValueError("segments do not fit")
    return (0, n_text, n_text + n_video, M)


CONFIGS = [
    dict(idx=0, name="tiny-256", M=256, K=256, N=256, r=8, fmt="nvfp4",
         seg=segments(256, 16, 16), masks=(MASK_ALL,), gen="outlier", alpha=0.5),
    dict(idx=1, name="attn-proj-5120x5120-M16384", M=16384, K=5120, N=5120, r=32, fmt="nvfp4",
         seg=segments(16384), masks=(MASK_ALL,), gen="outlier", alpha=0.5),
    dict(idx=2, name="mlp-up-int4-5120x13824-M32768", M=32768, K=5120, N=13824, r=32,
         fmt="int4", seg=segments(32768), masks=(MASK_ALL,), gen="outlier", alpha=0.5),
    dict(idx=3, name="mlp-down-sweep-13824x5120-M65536", M=65536, K=13824, N=5120, r=32,
         fmt="nvfp4", seg=segments(65536),
         masks=(MASK_NONE, MASK_ALL, MASK_VIDEO, MASK_TEXT), gen="outlier", alpha=0.5),
    dict(idx=4, name="deltaquant-31x24x42-5120x5120", M=312 + 31 * 24 * 42 + 128, K=5120,
         N=5120, r=128, fmt="nvfp4-delta", seg=(0, 312, 312 + 31 * 24 * 42, 31688),
         masks=(MASK_ALL,), gen="cube-field", alpha=0.5,
         grid=(31, 24, 42), cube=(2, 2, 2), cube1d=4, n_text=312, n_audio=128),
]


def config(i):
    return dict(CONFIGS[i])
