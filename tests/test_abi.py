"""CPU tests of the C ABI: the library loads without a GPU, exports every entry point declared in
include/svdq.h, validates arguments before enqueuing anything, and computes the host-side cube
geometry exactly like the oracle."""
import ctypes

import numpy as np
import pytest

from w4a4_quantized_dit_amd import _lib
from oracle import delta as DQ

OK, INVALID, SHAPE, NULLP, HIPERR, NOTIMPL = 0, 1, 2, 3, 4, 5
P = 1 << 20          # a fake, 16-byte aligned, non-NULL "device pointer" (never dereferenced)
MIS = P + 4          # misaligned


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_entry_point_is_exported(lib):
    names = _lib.header_entry_points()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert lib.svdq_abi_version() == 1
    for s in range(6):
        assert lib.svdq_status_string(s).decode().startswith("SVDQ_")


def _seg(*v):
    return ctypes.cast((ctypes.c_int64 * 4)(*v), ctypes.c_void_p)


def _err(lib):
    return lib.svdq_last_error().decode()


def test_calibrate_validation(lib):
    f = lib.svdq_calibrate_lambda
    good = dict(X=P, M=64, K=256, ldx=256, seg=_seg(0, 1, 60, 64), W=P, N=32, ldw=256, mask=7,
                alpha=0.5, acc=0, ax=P, aw=P, lam=P, amax=P, s=None)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["X"], a["M"], a["K"], a["ldx"], a["seg"], a["W"], a["N"], a["ldw"], a["mask"],
                 a["alpha"], a["acc"], a["ax"], a["aw"], a["lam"], a["amax"], a["s"])
    assert call(X=None) == NULLP and "X" in _err(lib)
    assert call(K=100) == SHAPE and "K=100" in _err(lib)
    assert call(ldx=200) == SHAPE
    assert call(X=MIS) == SHAPE
    assert call(seg=_seg(0, 10, 5, 64)) == INVALID
    assert call(seg=_seg(0, 1, 60, 63)) == INVALID
    assert call(mask=8) == INVALID
    assert call(alpha=1.0) == INVALID
    assert call(M=0, seg=_seg(0, 0, 0, 0)) == SHAPE
    assert call(lam=None) == NULLP


def test_quantize_weight_validation(lib):
    f = lib.svdq_quantize_weight
    assert f(7, P, 64, 256, 256, None, P, P, 32, P, P, P, None) == INVALID
    assert f(0, P, 64, 256, 256, None, P, P, 32, P, P, None, None) == NULLP   # NVFP4 needs g
    assert f(0, P, 64, 256, 256, None, P, P, 12, P, P, P, None) == SHAPE      # r % 8
    assert f(0, P, 64, 256, 256, None, P, P, 136, P, P, P, None) == SHAPE     # r > 128
    assert f(0, P, 64, 256, 256, None, None, P, 32, P, P, P, None) == NULLP
    assert f(0, P, 64, 320, 320, None, P, P, 32, P, P, P, None) == SHAPE


def test_quantize_weight_workspace_validation(lib):
    f = lib.svdq_quantize_weight_ws
    need = lib.svdq_quantize_weight_workspace_bytes(0, 64, 256)
    assert need == 4 * 64 * 256
    assert lib.svdq_quantize_weight_workspace_bytes(1, 64, 256) == 0      # single-pass formats
    assert lib.svdq_quantize_weight_workspace_bytes(2, 64, 256) == 0
    # the workspace variant validates like svdq_quantize_weight, then the workspace (NVFP4);
    # every case here fails before any launch
    assert f(7, P, 64, 256, 256, None, P, P, 32, P, P, P, P, need, None) == INVALID
    assert f(0, P, 64, 256, 256, None, P, P, 12, P, P, P, P, need, None) == SHAPE
    assert f(0, P, 64, 256, 256, None, P, P, 32, P, P, P, None, need, None) == NULLP
    assert f(0, P, 64, 256, 256, None, P, P, 32, P, P, P, P + 16, need, None) == SHAPE
    assert "aligned" in _err(lib)
    assert f(0, P, 64, 256, 256, None, P, P, 32, P, P, P, P, need - 1, None) == SHAPE
    assert "workspace" in _err(lib)


def test_quant_act_and_gemm_validation(lib):
    qa = lib.svdq_quant_act_lowrank_down
    assert qa(0, P, 64, 256, 256, None, None, P, 32, P, P, None, P, None, None) == NULLP
    assert qa(0, P, 64, 256, 128, None, None, P, 32, P, P, P, P, None, None) == SHAPE
    assert qa(1, P, 64, 256, 256, None, None, P, 32, P, P, None, None, None, None) == NULLP
    # row strides past 2^24 elements are refused (32-bit byte offsets inside a workgroup)
    assert qa(0, P, 64, 256, (1 << 24) + 8, None, None, P, 32, P, P, P, P, None, None) == SHAPE
    # at rank 128 the L1 slice and 1/λ of K = 16384 channels do not fit one CU's 160 KB of LDS
    assert qa(0, P, 64, 16384, 16384, None, None, P, 128, P, P, P, P, None, None) == SHAPE
    assert "LDS" in _err(lib)
    # one step of 256 past the largest K at each rank (28416 at r = 0, 26624 at r = 32, 14592 at
    # r = 128, which the GPU suite runs) is refused
    for K, r in ((28672, 0), (26880, 32), (14848, 128)):
        assert qa(0, P, 64, K, K, None, None, P if r else None, r, P, P, P, P if r else None,
                  None, None) == SHAPE, (K, r)
        assert "LDS" in _err(lib)
    g = lib.svdq_w4a4_gemm
    assert g(0, 64, 128, 256, P, P, P, P, P, P, P, P, 32, None, None, P, 128, None) == SHAPE
    assert g(0, 64, 256, 256, P, P, P, P, P, P, P, P, 32, None, None, P, 128, None) == SHAPE
    assert g(0, 64, 256, 256, P, P, P, P, P, P, P, P, 32, P, None, P, 256, None) == INVALID
    assert g(1, 64, 256, 256, P, P, None, P, P, None, P, P, 32, P, P, P, 256, None) == INVALID
    assert g(0, 64, 256, 256, P, P, None, P, P, P, P, P, 32, None, None, P, 256, None) == NULLP
    assert g(0, 64, 256, 256, P, P, P, P, P, P, P, P, 32, None, None, P, 260, None) == SHAPE
    assert g(0, 64, 256, 256, P, P, P, P, P, P, P, P, 32, None, None, MIS, 256, None) == SHAPE
    assert g(0, 64, 256, 256, P, MIS, P, P, P, P, P, P, 32, None, None, P, 256, None) == SHAPE
    assert g(0, 64, 256, 256, P, P, P, P, MIS, P, P, P, 32, None, None, P, 256, None) == SHAPE


def test_other_validation(lib):
    assert lib.svdq_gemm_core(0, 256, 256, P, P, P, P, P, P, None) == SHAPE
    assert lib.svdq_score_modal_rel_l2(P, 256, P, 256, P, 256, 10, 256, 256, P, P, 4, None,
                                       None) == NULLP
    # the two-part scoring: reference rows, then sums against them
    ref = lib.svdq_score_reference_rows
    assert ref(P, 256, P, 256, 10, 256, 256, P, 4, None, 256, None) == NULLP
    assert ref(P, 256, P, 256, 10, 128, 256, P, 4, P, 128, None) == SHAPE    # N % 256
    assert ref(P, 256, P, 256, 10, 256, 256, P, 4, P, 200, None) == SHAPE    # ldr < N
    assert ref(P, 256, P, 256, 10, 256, 200, P, 4, P, 256, None) == SHAPE    # K % 256
    assert ref(P, 256, MIS, 256, 10, 256, 256, P, 4, P, 256, None) == SHAPE    # misaligned W
    assert ref(P, 256, P, 256, 10, 256, 256, P, 0, P, 256, None) == OK       # nothing to do
    sr = lib.svdq_score_modal_rel_l2_ref
    assert sr(P, 256, P, 256, 10, 256, P, P, 4, None, None) == NULLP
    assert sr(P, 256, P, 256, 10, 12, P, P, 4, P, None) == SHAPE              # N % 8
    assert sr(P, 256, P, 248, 10, 256, P, P, 4, P, None) == SHAPE             # ldr < N
    assert sr(P, 260, P, 256, 10, 256, P, P, 4, P, None) == SHAPE             # ldy % 8
    assert sr(P, 256, P, 256, 0, 256, P, P, 4, P, None) == SHAPE              # M < 1
    assert sr(P, 256, P, 256, 10, 256, P, P, 0, P, None) == OK
    d = lib.svdq_delta_quant_act
    ws = 1 << 30
    need = lib.svdq_delta_workspace_bytes(8, 256)
    assert need == 8 * 256 * 4 and lib.svdq_delta_workspace_bytes(0, 256) == -1

    def dcall(**kw):
        a = dict(X=P, M=10, K=256, ldx=256, lam=None, amax=P, cp=P, cr=P, nc=8, gp=P, ng=2, down=P,
                 r=8, cc=P, cs=P, dc=P, ds=P, gd=P, D=P, sat=None, ws=ws, wsb=need)
        a.update(kw)
        return d(a["X"], a["M"], a["K"], a["ldx"], a["lam"], a["amax"], a["cp"], a["cr"], a["nc"],
                 a["gp"], a["ng"], a["down"], a["r"], a["cc"], a["cs"], a["dc"], a["ds"], a["gd"],
                 a["D"], a["sat"], a["ws"], a["wsb"], None)
    assert dcall(nc=11) == INVALID                        # more cubes than rows
    assert dcall(ng=0) == INVALID and dcall(ng=9) == INVALID
    assert dcall(gp=None) == NULLP
    assert dcall(ws=None) == NULLP
    assert dcall(ws=ws + 16) == SHAPE                     # not 256-byte aligned
    assert dcall(wsb=need - 1) == SHAPE and "workspace" in _err(lib)
    assert dcall(ldx=128) == SHAPE
    assert dcall(K=200, ldx=200) == SHAPE
    assert dcall(r=12) == SHAPE
    assert dcall(D=None) == NULLP
    assert lib.svdq_cube_geometry(2, 2, 2, 4, 4, 4, 0, 0, 4, None, None, None, None) == NULLP


def test_cube_geometry_matches_oracle():
    for args in ((31, 24, 42, 2, 2, 2, 312, 128, 4), (3, 2, 3, 2, 2, 2, 5, 2, 2),
                 (5, 7, 3, 2, 2, 2, 0, 9, 4), (1, 1, 1, 1, 1, 1, 3, 0, 2)):
        got = _lib.svdq_cube_geometry(*args)
        want = DQ.cube_geometry(*args)
        for g, w in zip(got, want):
            assert np.array_equal(g, w), args


def test_cube_geometry_rejects_bad_sizes(lib):
    n = ctypes.c_int64(0)
    pn = ctypes.cast(ctypes.pointer(n), ctypes.c_void_p)
    assert lib.svdq_cube_geometry(2, 2, 2, 0, 2, 2, 0, 0, 4, None, None, None, pn) == INVALID
    assert lib.svdq_cube_geometry(8, 8, 8, 4, 4, 8, 0, 0, 4, None, None, None, pn) == SHAPE
    assert lib.svdq_cube_geometry(8, 8, 8, 2, 2, 2, 0, 0, 65, None, None, None, pn) == SHAPE
    assert lib.svdq_cube_geometry(31, 24, 42, 4, 4, 4, 312, 128, 4, None, None, None, pn) == OK
    assert n.value == 638                                 # uniform cube-64
    assert lib.svdq_cube_geometry(31, 24, 42, 2, 2, 2, 312, 128, 4, None, None, None, pn) == OK
    assert n.value == 4142


def test_bits_lost_validation(lib):
    f = lib.svdq_bits_lost
    assert f(None, None, 256, 16, P, None) == NULLP and "ax" in _err(lib)
    assert f(P, None, 256, 16, None, None) == NULLP
    assert f(P, None, 256, 24, P, None) == INVALID
    assert f(P, None, 200, 16, P, None) == SHAPE
    assert f(P, None, 32, 64, P, None) == SHAPE


def test_lowrank_validation(lib):
    f = lib.svdq_lowrank_factors
    ws = 1 << 30                  # a fake 256-byte aligned workspace address
    need = lib.svdq_lowrank_workspace_bytes(512, 256, 40)
    assert need > 0 and lib.svdq_lowrank_workspace_bytes(512, 256, 161) == -1

    def call(**kw):
        a = dict(W=P, N=512, K=256, ldw=256, lam=None, om=P, ell=40, r=32, q=2, down=P, up=P,
                 sig=None, ws=ws, wsb=need)
        a.update(kw)
        return f(a["W"], a["N"], a["K"], a["ldw"], a["lam"], a["om"], a["ell"], a["r"], a["q"],
                 a["down"], a["up"], a["sig"], a["ws"], a["wsb"], None)
    assert call(W=None) == NULLP
    assert call(om=None) == NULLP
    assert call(ws=ws + 16) == SHAPE                     # not 256-byte aligned
    assert call(r=48) == SHAPE                           # r > ell
    assert call(r=0) == SHAPE
    assert call(ell=161, r=32) == SHAPE
    assert call(N=32, ldw=256) == SHAPE                  # ell > N
    assert call(q=9) == INVALID
    assert call(wsb=need - 1) == SHAPE and "workspace" in _err(lib)
    assert call(ldw=250) == SHAPE


def test_lambda_search_validation(lib):
    import ctypes
    f = lib.svdq_lambda_search
    ws = 1 << 30
    need = lib.svdq_lambda_search_workspace_bytes(0, 512, 256, 40, 32, 1024, 39, 0)
    assert need > 0
    need_refit = lib.svdq_lambda_search_workspace_bytes(0, 512, 256, 40, 32, 1024, 39, 100)
    assert need_refit >= need + 512 * 256 * 4            # the fp32 refit target
    assert lib.svdq_lambda_search_workspace_bytes(0, 512, 256, 161, 32, 1024, 39, 0) == -1
    assert lib.svdq_lambda_search_workspace_bytes(4, 512, 256, 40, 32, 1024, 39, 0) == -1
    assert lib.svdq_lambda_search_workspace_bytes(0, 512, 256, 0, 0, 1024, 39, 0) > 0
    assert lib.svdq_lambda_search_workspace_bytes(0, 512, 256, 0, 0, 1024, 39, 3) == -1
    grid = (ctypes.c_float * 39)(*[i / 40 for i in range(1, 40)])
    bad = (ctypes.c_float * 2)(0.5, 1.0)

    def call(**kw):
        a = dict(X=P, M=4096, K=256, ldx=256, W=P, N=512, ldw=256, ax=P, aw=P, mask=7,
                 al=ctypes.cast(grid, ctypes.c_void_p), na=39, fmt=0, om=P, ell=40, r=32, q=2,
                 T=0, rows=P, nr=1024, sc=P, its=None, best=P, idx=P, bd=None, bu=None, ws=ws,
                 wsb=need)
        a.update(kw)
        return f(a["X"], a["M"], a["K"], a["ldx"], a["W"], a["N"], a["ldw"], a["ax"], a["aw"],
                 a["mask"], a["al"], a["na"], a["fmt"], a["om"], a["ell"], a["r"], a["q"], a["T"],
                 a["rows"], a["nr"], a["sc"], a["its"], a["best"], a["idx"], a["bd"], a["bu"],
                 a["ws"], a["wsb"], None)
    assert call(X=None) == NULLP
    assert call(al=None) == NULLP
    assert call(om=None) == NULLP                        # r > 0 needs Ω
    assert call(fmt=7) == INVALID
    assert call(N=500) == SHAPE
    assert call(K=200, ldx=200, ldw=200) == SHAPE
    assert call(ldx=128) == SHAPE
    assert call(mask=8) == INVALID
    assert call(na=0) == INVALID
    assert call(al=ctypes.cast(bad, ctypes.c_void_p), na=2) == INVALID and "alphas[1]" in _err(lib)
    assert call(r=12) == SHAPE                           # rank not a multiple of 8
    assert call(ell=24) == SHAPE                         # ell < r
    assert call(q=9) == INVALID
    assert call(nr=0) == SHAPE
    assert call(M=0) == SHAPE
    assert call(ws=ws + 64) == SHAPE
    assert call(wsb=need - 1) == SHAPE and "workspace" in _err(lib)
    assert call(T=-1) == INVALID
    assert call(T=1001) == INVALID
    assert call(T=3, r=0, om=None) == INVALID            # refit needs a branch
    assert call(T=3, wsb=need) == SHAPE                  # the refit target needs room
    assert call(bd=P) == NULLP                           # best factors go in pairs
    assert call(bd=P, bu=P, r=0, om=None) == INVALID
    assert call(bd=MIS, bu=P) == SHAPE
    big = lib.svdq_lambda_search_workspace_bytes(0, 512, 16384, 136, 128, 1024, 39, 0)
    assert call(K=16384, ldx=16384, ldw=16384, r=128, ell=136, wsb=big) == SHAPE
    assert "LDS" in _err(lib)


def test_gptq_validation(lib):
    hx = lib.svdq_gptq_hessian
    assert hx(None, 16, 256, 256, None, 0, P, None) == NULLP
    assert hx(P, 16, 256, 256, None, 0, None, None) == NULLP
    assert hx(P, 0, 256, 256, None, 0, P, None) == SHAPE
    assert hx(P, 16, 200, 200, None, 0, P, None) == SHAPE
    assert hx(P, 16, 256, 100, None, 0, P, None) == SHAPE
    ws = 1 << 30
    need = lib.svdq_gptq_workspace_bytes(512, 256)
    assert need >= 16 * 256 * 256 + 12 * 512 * 256
    assert lib.svdq_gptq_workspace_bytes(0, 256) == -1
    f = lib.svdq_gptq_quantize_weight

    def call(**kw):
        a = dict(fmt=0, W=P, N=512, K=256, ldw=256, lam=P, down=P, up=P, r=32, H=P, codes=P,
                 scales=P, g=P, ws=ws, wsb=need)
        a.update(kw)
        return f(a["fmt"], a["W"], a["N"], a["K"], a["ldw"], a["lam"], a["down"], a["up"], a["r"],
                 a["H"], a["codes"], a["scales"], a["g"], a["ws"], a["wsb"], None)
    assert call(fmt=9) == INVALID
    assert call(W=None) == NULLP
    assert call(H=None) == NULLP
    assert call(g=None) == NULLP                          # NVFP4 needs its tensor scale
    assert call(down=None) == NULLP
    assert call(r=12) == SHAPE
    assert call(N=300) == SHAPE
    assert call(K=200, ldw=200) == SHAPE
    assert call(ldw=128) == SHAPE
    assert call(ws=ws + 8) == SHAPE
    assert call(wsb=need - 1) == SHAPE and "workspace" in _err(lib)
    assert call(W=MIS) == SHAPE


def test_cube64_and_aligned_geometry_match_oracle():
    for args in ((31, 24, 42, 4, 4, 4, 312, 128, 4), (31, 24, 42, 4, 4, 4, 312, 128, 64),
                 (31, 24, 42, 1, 4, 3, 312, 128, 4), (31, 24, 42, 1, 2, 2, 312, 128, 4),
                 (5, 7, 9, 4, 4, 4, 3, 70, 64)):
        got = _lib.svdq_cube_geometry(*args)
        want = DQ.cube_geometry(*args)
        for g, w in zip(got, want):
            assert np.array_equal(g, w), args


def test_divisor_aligned_and_schedule_match_oracle(lib):
    for dims in ((31, 24, 42), (37, 15, 27), (32, 24, 42), (30, 20, 12), (1, 1, 1), (0, 5, 7),
                 (64, 60, 49)):
        for req in ((4, 4, 4), (2, 2, 2), (1, 1, 1), (8, 3, 5)):
            assert _lib.svdq_cube_divisor_aligned(*dims, *req) == \
                DQ.divisor_aligned_edges(*dims, *req), (dims, req)
    sched = [(0, 4, 4, 4), (10, 2, 4, 4), (30, 2, 2, 2)]
    for step in (0, 1, 9, 10, 11, 29, 30, 49, 10 ** 6):
        assert _lib.svdq_cube_schedule(sched, step) == DQ.schedule_edges(sched, step)
    for bad in ([(1, 2, 2, 2)], [(0, 2, 2, 2), (0, 4, 4, 4)], [(0, 2, 0, 2)]):
        with pytest.raises(_lib.SvdqError):
            _lib.svdq_cube_schedule(bad, 0)
    with pytest.raises(_lib.SvdqError):
        _lib.svdq_cube_schedule(sched, -1)
    e = (ctypes.c_int64 * 3)()
    assert lib.svdq_cube_divisor_aligned(4, 4, 4, 0, 1, 1, ctypes.cast(e, ctypes.c_void_p)) == INVALID


def _check_groups(ptr, gp):
    sizes = np.diff(ptr)
    assert gp[0] == 0 and gp[-1] == len(sizes) and np.all(np.diff(gp) > 0)
    for a, b in zip(gp[:-1], gp[1:]):
        rows = sizes[a:b].sum()
        assert rows <= 64 and b - a <= 16
        if b < len(sizes):                         # greedy: the next cube would not fit
            assert rows + sizes[b] > 64 or b - a == 16


def test_cube_groups_pack_greedily():
    for args in ((31, 24, 42, 2, 2, 2, 312, 128, 4), (31, 24, 42, 4, 4, 4, 312, 128, 64),
                 (31, 24, 42, 1, 4, 3, 312, 128, 4), (5, 7, 9, 1, 1, 1, 3, 2, 1)):
        _, ptr, _ = DQ.cube_geometry(*args)
        _check_groups(ptr, _lib.svdq_cube_groups(ptr))
    # a caller's CSR with a 64-row cube and a 65-row cube
    ok = np.array([0, 3, 67, 70], np.int32)
    _check_groups(ok, _lib.svdq_cube_groups(ok))
    assert _lib.svdq_cube_groups(ok).tolist() == [0, 1, 2, 3]
    with pytest.raises(_lib.SvdqError):
        _lib.svdq_cube_groups(np.array([0, 3, 68, 70], np.int32))
    with pytest.raises(_lib.SvdqError):
        _lib.svdq_cube_groups(np.array([0, 3, 3, 7], np.int32))      # an empty cube


def test_probe_library_loads_and_validates():
    """The benchmark's memory probe is its own library and refuses bad arguments on the host."""
    from w4a4_quantized_dit_amd import build as B
    lib = ctypes.CDLL(B.PROBE_LIB)
    f = lib.svdq_probe_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p]
    assert f(None, 16, P, 16, None) == 1
    assert f(P, 17, P, 16, None) == 1              # not whole 16-byte pieces
    assert f(P, -16, P, 16, None) == 1
    assert f(P, 0, P, 0, None) == 0                # nothing to do: nothing launched
    assert not hasattr(_lib.load(), "svdq_probe_stream")
