"""Pins of the oracle's DeltaQuant geometry variants ("DeltaQuant on MiniMax-H3", section
"Deviations from the paper, and one replication"): uniform cube-64, divisor-aligned cube edges
and the per-step cube schedule, against counts derived by hand (tests/golden/workloads.txt) and
small cases worked out below; plus the host C functions of the same steps against the oracle."""
import os

import numpy as np
import pytest

from oracle import delta as DQ
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _geo_golden():
    out = {}
    with open(os.path.join(GOLD, "workloads.txt")) as f:
        for line in f:
            p = line.split()
            if p and not p[0].startswith("#") and not p[0].isdigit():
                out[p[0]] = int(p[1])
    return out


def test_cube64_counts_match_hand_derivation():
    g = _geo_golden()
    cfg = synth.config(4)
    T, H, W = cfg["grid"]
    r2c, ptr, rows = DQ.cube_geometry(T, H, W, 4, 4, 4, cfg["n_text"], cfg["n_audio"], 4)
    sizes = np.diff(ptr)
    assert len(sizes) == g["cube64_n_cubes"]
    video = sizes[78:len(sizes) - 32]
    assert len(video) == g["cube64_video_cubes"]
    assert np.count_nonzero(video == 64) == g["cube64_full_cubes"]
    assert np.count_nonzero(video == 48) == g["cube64_t_ragged_cubes"]
    assert np.count_nonzero(video == 32) == g["cube64_w_ragged_cubes"]
    assert np.count_nonzero(video == 24) == g["cube64_corner_cubes"]
    assert sorted(rows.tolist()) == list(range(cfg["M"]))
    # the members of a full cube are its 4x4x4 raster neighbourhood, ascending
    c = 78                                   # first video cube: corner (0, 0, 0)
    mem = rows[ptr[c]:ptr[c + 1]]
    want = sorted(312 + t * 24 * 42 + h * 42 + w for t in range(4) for h in range(4)
                  for w in range(4))
    assert mem.tolist() == want


@pytest.mark.parametrize("dims,req,want", [
    ((31, 24, 42), (4, 4, 4), (1, 4, 3)),     # prime T collapses to single frames
    ((31, 24, 42), (2, 2, 2), (1, 2, 2)),
    ((37, 15, 27), (4, 4, 4), (1, 3, 3)),     # the grid the page measured later
    ((32, 24, 42), (4, 4, 4), (4, 4, 3)),
    ((30, 20, 12), (4, 4, 4), (3, 4, 4)),
    ((1, 1, 1), (4, 4, 4), (1, 1, 1)),
    ((0, 24, 42), (4, 4, 4), (4, 4, 3)),      # an empty axis keeps its edge
])
def test_divisor_aligned_edges_by_hand(dims, req, want):
    assert DQ.divisor_aligned_edges(*dims, *req) == want


def test_divisor_aligned_geometry_has_no_ragged_cube():
    g = _geo_golden()
    T, H, W = 31, 24, 42
    for req, key in (((4, 4, 4), "aligned444_video_cubes"), ((2, 2, 2), "aligned222_video_cubes")):
        e = DQ.divisor_aligned_edges(T, H, W, *req)
        _, ptr, _ = DQ.cube_geometry(T, H, W, *e, 0, 0, 4)
        sizes = np.diff(ptr)
        assert len(sizes) == g[key]
        assert np.all(sizes == e[0] * e[1] * e[2])
        assert DQ.padded_video_rows(T, H, W, *e) == T * H * W


def test_padded_rows_by_hand():
    g = _geo_golden()
    assert DQ.padded_video_rows(31, 24, 42, 4, 4, 4) == g["padded444_video_rows"]
    assert DQ.padded_video_rows(31, 24, 42, 2, 2, 2) == g["padded222_video_rows"]
    assert DQ.padded_video_rows(37, 15, 27, 2, 2, 2) == 38 * 16 * 28
    # the padded rows are exactly the sum over video cubes of the full cube volume
    _, ptr, _ = DQ.cube_geometry(31, 24, 42, 4, 4, 4, 0, 0, 4)
    assert len(np.diff(ptr)) * 64 == g["padded444_video_rows"]


def test_schedule_lookup_by_hand():
    sched = [(0, 4, 4, 4), (10, 2, 4, 4), (30, 2, 2, 2)]
    assert DQ.schedule_edges(sched, 0) == (4, 4, 4)
    assert DQ.schedule_edges(sched, 9) == (4, 4, 4)
    assert DQ.schedule_edges(sched, 10) == (2, 4, 4)
    assert DQ.schedule_edges(sched, 29) == (2, 4, 4)
    assert DQ.schedule_edges(sched, 30) == (2, 2, 2)
    assert DQ.schedule_edges(sched, 1000) == (2, 2, 2)
    assert DQ.schedule_edges([(0, 1, 2, 3)], 7) == (1, 2, 3)
    for bad in ([], [(1, 2, 2, 2)], [(0, 2, 2, 2), (0, 4, 4, 4)], [(0, 2, 2, 2), (5, 1, 1, 1), (3, 4, 4, 4)]):
        with pytest.raises(ValueError):
            DQ.schedule_edges(bad, 0)
    with pytest.raises(ValueError):
        DQ.schedule_edges(sched, -1)
