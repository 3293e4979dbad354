"""DeltaQuant variant: cube geometry, FP8 cube-mean core, NVFP4 delta, core GEMM.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"DeltaQuant on MiniMax-H3":
  * "Why DeltaQuant does not beat SVDQuant here": the tokens of one spatiotemporal cube are
    represented by one core plus small deltas;
  * "The audio win has a mechanism": non-video rows are covered by 1-D cubes of consecutive
    rows ("cover_remaining");
  * "The activation scale bound held": the delta's activation tensor scale comes from the
    bound |x − core| ≤ 2·max|x|, and saturated NVFP4 groups are counted at run time;
  * "Deviations from the paper": the core branch does not go through the FP4 scaled dot
    (it runs on a 16-bit path);
  * "Standing configuration": the video grid is derived per request, and the cube sequence
    and their count are fixed for a given grid.
The layer is  Y = Q8(core)·Q(R) + Q4(delta)·Q(R) + X̂·L1·L2.

Readings where the pages are silent:
  * row order [text | video | audio]; video rows in raster (t, h, w) order; a video row at
    (t, h, w) belongs to cube (t//ct, h//ch, w//cw), so edge cubes are ragged when a grid
    dimension is not a multiple of the cube size; text and audio rows form 1-D cubes of
    `cube1d` consecutive rows of their own segment (the last one possibly shorter);
  * cubes are numbered in increasing order of their first row; members are listed ascending;
  * core[c, k] = float32(sum over members, ascending, in float32) / float32(|c|);
  * FP8 core: per core row, s_c = amax_c / 448 (float32), codes = sign | E4M3(|core| · (1/s_c))
    nearest-even, satfinite; s_c == 0 gives signed zero codes;
  * delta = X̂ − core[cube(m)] in float32 with the UNQUANTISED core, so |delta| ≤ 2·max|X̂|
    holds exactly; the delta is NVFP4-quantised with tensor amax 2·act_amax (static);
  * the low-rank branch uses X̂ (not the delta).
"""
import numpy as np

from .formats import e4m3_encode_signed, e4m3_decode
from .quant import nvfp4_quantize, nvfp4_dequantize
from .gemm import lowrank_up
from .formats import bf16_rne

F32 = np.float32


def cube_geometry(T, H, W, ct, ch, cw, n_text, n_audio, cube1d):
    """(row_to_cube int32 [M], cube_ptr int32 [n_cubes+1], cube_rows int32 [M])."""
    keys = []
    for i in range(n_text):
        keys.append(("text", i // cube1d))
    for t in range(T):
        for h in range(H):
            for w in range(W):
                keys.append(("video", t // ct, h // ch, w // cw))
    for i in range(n_audio):
        keys.append(("audio", i // cube1d))
    first_row = {}
    for m, key in enumerate(keys):
        if key not in first_row:
            first_row[key] = m
    ordered = sorted(first_row, key=lambda k: first_row[k])
    cube_id = {key: c for c, key in enumerate(ordered)}
    M = len(keys)
    row_to_cube = np.array([cube_id[k] for k in keys], dtype=np.int32)
    members = [[] for _ in ordered]
    for m in range(M):
        members[row_to_cube[m]].append(m)
    cube_ptr = np.zeros(len(ordered) + 1, dtype=np.int32)
    for c, mem in enumerate(members):
        cube_ptr[c + 1] = cube_ptr[c] + len(mem)
    cube_rows = np.array([m for mem in members for m in mem], dtype=np.int32)
    return row_to_cube, cube_ptr, cube_rows


def divisor_aligned_edges(T, H, W, ct, ch, cw):
    """Cube edges aligned to the grid ("DeltaQuant on MiniMax-H3", section "Deviations from the
    paper, and one replication": divisor-aligned cube shapes as an opt-in variant).  The page
    names the variant but not its rule; the reading here: along each axis the edge becomes the
    largest divisor of that grid dimension not above the requested edge, so no cube is ragged
    and none exceeds the requested shape.  An empty axis keeps the requested edge."""
    def edge(n, e):
        if n <= 0:
            return e
        return max(d for d in range(1, min(n, e) + 1) if n % d == 0)
    return edge(T, ct), edge(H, ch), edge(W, cw)


def padded_video_rows(T, H, W, ct, ch, cw):
    """Rows that a cube-major layout padding every video cube to its full ct·ch·cw volume would
    give the GEMMs (ragged edge cubes padded); equals T·H·W when the edges divide the grid."""
    def up(n, e):
        return -(-n // e) * e
    return up(T, ct) * up(H, ch) * up(W, cw)


def schedule_edges(schedule, step):
    """Cube edges of a denoising step under a timestep cube schedule ("DeltaQuant on MiniMax-H3",
    section "Deviations from the paper, and one replication": a per-timestep cube schedule
    replicates against uniform cube-64).  The page does not print the schedule; the reading is a
    table of (first_step, ct, ch, cw) rows with strictly increasing first_step starting at 0,
    and a step takes the shape of the last row whose first_step is not above it."""
    rows = [tuple(int(v) for v in r) for r in schedule]
    if not rows or rows[0][0] != 0:
        raise ValueError("a schedule starts at step 0")
    for a, b in zip(rows, rows[1:]):
        if b[0] <= a[0]:
            raise ValueError("first steps must increase")
    if step < 0:
        raise ValueError("negative step")
    cur = rows[0]
    for r in rows:
        if r[0] <= step:
            cur = r
    return cur[1], cur[2], cur[3]


def cube_core(xhat32, cube_ptr, cube_rows):
    """core[c, k]: float32 ascending sum over the cube's rows, divided by the member count."""
    xhat32 = np.asarray(xhat32, dtype=F32)
    n_cubes = len(cube_ptr) - 1
    core = np.empty((n_cubes, xhat32.shape[1]), dtype=F32)
    for c in range(n_cubes):
        mem = cube_rows[cube_ptr[c]:cube_ptr[c + 1]]
        acc = np.zeros(xhat32.shape[1], dtype=F32)
        for m in mem:
            acc = (acc + xhat32[m]).astype(F32)
        core[c] = (acc / F32(len(mem))).astype(F32)
    return core


def core_fp8(core):
    """Per-row FP8 E4M3 core: (codes uint8 [C, K], row scale float32 [C])."""
    core = np.asarray(core, dtype=F32)
    amax = np.abs(core).max(axis=1).astype(F32)
    s = (amax / F32(448.0)).astype(F32)
    inv = np.zeros_like(s)
    nz = s != 0
    inv[nz] = (F32(1.0) / s[nz]).astype(F32)
    y = (core * inv[:, None]).astype(F32)
    return e4m3_encode_signed(y), s


def delta_rows(xhat32, core, row_to_cube):
    """delta[m, k] = X̂[m, k] − core[cube(m), k] in float32."""
    return (np.asarray(xhat32, dtype=F32) - core[row_to_cube]).astype(F32)


def delta_quantize(delta32, act_amax):
    """NVFP4 delta with the static bound amax_t = 2·act_amax: (codes, scales, g, n_saturated)."""
    amax_t = F32(F32(2.0) * F32(act_amax))
    return nvfp4_quantize(delta32, amax_t)


def core_out_f64(core_codes, core_scale, w_codes, w_scales, g_w):
    """core_out[c, n] = s_c · Σ_k e4m3(code[c, k]) · W_deq[n, k]  (float64, W_deq includes g_w)."""
    Wd = nvfp4_dequantize(w_codes, w_scales, g_w)
    cv = e4m3_decode(core_codes)
    return np.asarray(core_scale, dtype=F32).astype(np.float64)[:, None] * (cv @ Wd.T)


def delta_linear(core_out64, row_to_cube, d_codes, d_scales, g_d, w_codes, w_scales, g_w,
                 D, lora_up_bits, rows=None):
    """Y64 = core_out[cube(m)] + delta_deq @ W_deqᵀ + D @ L2, and its bf16 bits.

    `rows` (optional) restricts the output to those rows (the inputs are then the full tensors).
    """
    if rows is None:
        rows = np.arange(d_codes.shape[0])
    Ad = nvfp4_dequantize(d_codes[rows], d_scales[rows], g_d)
    Wd = nvfp4_dequantize(w_codes, w_scales, g_w)
    y64 = core_out64[row_to_cube[rows]] + Ad @ Wd.T + lowrank_up(np.asarray(D)[rows], lora_up_bits)
    return y64, bf16_rne(y64)
