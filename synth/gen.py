"""Seeded generators.

Recipe (seed 0 for every workload):
  * outlier-channel activations (workloads 0-3): row m of modality μ is N(0, 1) · c_μ[k], with
    c_μ[k] = exp(0.75 · z), z ~ N(0, 1) drawn independently per modality (near-zero
    cross-modality correlation), and round(0.02·K) channels per modality, drawn without
    replacement independently per modality, multiplied by 30;
  * cube-field activations (workload 4): X[m, k] = μ[cube(m), k] + 0.64 · z with μ ~ N(0, 1)
    per (cube, channel) and z ~ N(0, 1) per element; video cubes are 2x2x2 over the raster
    (t, h, w) grid, text and audio rows form cubes of 4 consecutive rows;
  * weights W ~ N(0, 1/K), stored [N, K] (out, in);
  * values are drawn in float64, cast to float32 and rounded to bf16 (nearest even, integer
    bit arithmetic).
Independent streams: profiles/boosted sets use default_rng([seed, 0]); weight rows in blocks of
ROW_BLOCK use default_rng([seed, 1, block]); activation rows in blocks of ROW_BLOCK use
default_rng([seed, 2, block]); cube means use default_rng([seed, 3, cube]); sampled rows use
default_rng([seed, 4]).  Any row range can therefore be generated on its own, with the same
values as in the full matrix.
"""
import numpy as np

ROW_BLOCK = 256


def to_bf16_bits(x):
    """float -> bf16 bits (uint16): cast to float32, then round to nearest even on the bits."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def profiles(K, seed=0):
    """Per-modality channel scales c [3, K] (float64) and the boosted channel sets."""
    rng = np.random.default_rng([seed, 0])
    z = rng.standard_normal((3, K))
    c = np.exp(0.75 * z)
    n_boost = round(0.02 * K)
    boosted = []
    for mu in range(3):
        b = np.sort(rng.choice(K, size=n_boost, replace=False))
        c[mu, b] *= 30.0
        boosted.append(b)
    return c, boosted


def weight_bits(N, K, seed=0, rows=None):
    """W ~ N(0, 1/K) as bf16 bits [N, K] (or only `rows`, a slice)."""
    r0, r1 = (0, N) if rows is None else (rows.start, rows.stop)
    out = np.empty((r1 - r0, K), dtype=np.uint16)
    b0, b1 = r0 // ROW_BLOCK, (r1 + ROW_BLOCK - 1) // ROW_BLOCK
    for b in range(b0, b1):
        lo, hi = b * ROW_BLOCK, min(N, (b + 1) * ROW_BLOCK)
        rng = np.random.default_rng([seed, 1, b])
        w = rng.standard_normal((hi - lo, K)) / np.sqrt(K)
        s0, s1 = max(lo, r0), min(hi, r1)
        out[s0 - r0:s1 - r0] = to_bf16_bits(w[s0 - lo:s1 - lo])
    return out


def gen_cube_index(cfg):
    """Generator-side cube id of every row for the cube-field workload (its own numbering)."""
    T, H, W = cfg["grid"]
    ct, ch, cw = cfg["cube"]
    n_text, n_audio, c1 = cfg["n_text"], cfg["n_audio"], cfg["cube1d"]
    text = np.arange(n_text) // c1
    n_tc = (n_text + c1 - 1) // c1
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    nH, nW = (H + ch - 1) // ch, (W + cw - 1) // cw
    video = ((t // ct) * nH * nW + (h // ch) * nW + (w // cw)).reshape(-1) + n_tc
    n_vc = ((T + ct - 1) // ct) * nH * nW
    audio = np.arange(n_audio) // c1 + n_tc + n_vc
    return np.concatenate([text, video, audio]).astype(np.int64)


def _modality_of_rows(seg, rows):
    return np.searchsorted(np.asarray(seg[1:3]), rows, side="right")


def x_bits(cfg, seed=0, rows=None):
    """Activations X as bf16 bits [M, K] (or only `rows`, a slice) for workload `cfg`."""
    M, K = cfg["M"], cfg["K"]
    r0, r1 = (0, M) if rows is None else (rows.start, rows.stop)
    out = np.empty((r1 - r0, K), dtype=np.uint16)
    if cfg["gen"] == "outlier":
        c, _ = profiles(K, seed)
    else:
        cube = gen_cube_index(cfg)
        means = {}
    b0, b1 = r0 // ROW_BLOCK, (r1 + ROW_BLOCK - 1) // ROW_BLOCK
    for b in range(b0, b1):
        lo, hi = b * ROW_BLOCK, min(M, (b + 1) * ROW_BLOCK)
        rng = np.random.default_rng([seed, 2, b])
        z = rng.standard_normal((hi - lo, K))
        idx = np.arange(lo, hi)
        if cfg["gen"] == "outlier":
            x = z * c[_modality_of_rows(cfg["seg"], idx)]
        else:
            x = 0.64 * z
            for j, m in enumerate(idx):
                cid = int(cube[m])
                if cid not in means:
                    means[cid] = np.random.default_rng([seed, 3, cid]).standard_normal(K)
                x[j] += means[cid]
        s0, s1 = max(lo, r0), min(hi, r1)
        out[s0 - r0:s1 - r0] = to_bf16_bits(x[s0 - lo:s1 - lo])
    return out


def sample_rows(seg, n_per=4096, seed=0):
    """Rows for scoring: per modality up to n_per rows without replacement (group 0 text,
    1 video, 2 audio), then n_per rows drawn uniformly from all rows (group 3).
    Returns (rows int32, group int8), each group's rows ascending."""
    rng = np.random.default_rng([seed, 4])
    rows, grp = [], []
    for mu in range(3):
        lo, hi = seg[mu], seg[mu + 1]
        n = min(n_per, hi - lo)
        pick = np.sort(rng.choice(np.arange(lo, hi), size=n, replace=False)) if n else np.zeros(0, int)
        rows.append(pick)
        grp.append(np.full(n, mu))
    M = seg[3]
    n = min(n_per, M)
    pick = np.sort(rng.choice(M, size=n, replace=False))
    rows.append(pick)
    grp.append(np.full(n, 3))
    return np.concatenate(rows).astype(np.int32), np.concatenate(grp).astype(np.int8)
