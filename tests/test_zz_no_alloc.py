"""The allocation-free DeltaQuant entry point (svdq_delta_quant_act_noalloc, static scratch inside
the library) against the workspace entry point (svdq_delta_quant_act) through the C ABI: two
calls in a row on one GPU, the first on the 31x24x42 workload (K = 5120, rank 128, 85 MB of
fp32 cores in the scratch), the second on a smaller grid (the scratch then holds the first
call's contents past the second call's cubes).  Every output must be bit for bit the same, as
both run the same kernel on the same inputs; and a call past the scratch's size must be refused
before anything runs."""
import numpy as np
import pytest

import synth
from tests.gpu_common import dev_bf16, dev, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a4_quantized_dit_amd import _lib, layer
    _lib.load()
    return _lib, layer


def _case(layer, grid, n_text, n_audio, K, r, geo, seed):
    torch = torch_mod()
    cfg = dict(synth.config(4))
    T, H, W = grid
    M = n_text + T * H * W + n_audio
    cfg.update(grid=grid, n_text=n_text, n_audio=n_audio, K=K, M=M,
               seg=(0, n_text, n_text + T * H * W, M))
    X = dev_bf16(synth.x_bits(cfg, seed))
    rng = np.random.default_rng(seed)
    lam = dev(rng.uniform(0.5, 2.0, K).astype(np.float32))
    amax = dev(np.array([40.0], np.float32))
    down = dev_bf16(synth.gen.to_bf16_bits(rng.standard_normal((r, K)) * 0.02)) if r else None
    g = layer.cube_geometry(T, H, W, *geo[:3], n_text, n_audio, geo[3])
    return X, lam, amax, down, g, M


def _outputs(torch, M, K, nc, r):
    u8 = torch.uint8
    return dict(cc=torch.full((nc, K), 0x55, dtype=u8, device="cuda"),
                cs=torch.full((nc,), -1.0, device="cuda"),
                dc=torch.full((M, K // 2), 0x55, dtype=u8, device="cuda"),
                dsc=torch.full((M, K // 16), 0x55, dtype=u8, device="cuda"),
                gd=torch.full((1,), -1.0, device="cuda"),
                D=torch.full((M, r), -1.0, device="cuda") if r else None,
                sat=torch.zeros(1, dtype=torch.int32, device="cuda"))


def _same(a, b):
    for k in ("cc", "cs", "dc", "dsc", "gd", "D", "sat"):
        if a[k] is None:
            continue
        assert torch_mod().equal(a[k], b[k]), k


def test_no_alloc_matches_workspace_entry_point_twice(env):
    _lib, layer = env
    torch = torch_mod()
    cases = [((31, 24, 42), 312, 128, 5120, 128, (2, 2, 2, 4), 0),   # the DeltaQuant workload
             ((5, 6, 9), 13, 9, 512, 32, (4, 4, 4, 64), 1)]          # smaller, second
    for grid, nt, na, K, r, geo, seed in cases:
        print(f"[no-alloc] grid {grid} K={K} r={r} cubes {geo}", flush=True)
        X, lam, amax, down, g, M = _case(layer, grid, nt, na, K, r, geo, seed)
        nc = g["n_cubes"]
        ref, got = _outputs(torch, M, K, nc, r), _outputs(torch, M, K, nc, r)
        ws = torch.empty(_lib.svdq_delta_workspace_bytes(nc, K) + 256, dtype=torch.uint8,
                         device="cuda")
        off = (-ws.data_ptr()) % 256
        _lib.svdq_delta_quant_act(X, lam, amax, g["cube_ptr"], g["cube_rows"], nc,
                                  g["group_ptr"], down, r, ref["cc"], ref["cs"], ref["dc"],
                                  ref["dsc"], ref["gd"], ref["D"], ref["sat"],
                                  ws[off:off + _lib.svdq_delta_workspace_bytes(nc, K)])
        _lib.svdq_delta_quant_act_noalloc(X, lam, amax, g["cube_ptr"], g["cube_rows"], nc,
                                          g["group_ptr"], down, r, got["cc"], got["cs"],
                                          got["dc"], got["dsc"], got["gd"], got["D"], got["sat"])
        torch.cuda.synchronize()
        _same(ref, got)
        assert torch.all(got["cs"] >= 0)               # every cube was written


def test_no_alloc_refuses_more_than_its_scratch(env):
    _lib, layer = env
    torch = torch_mod()
    K, nc = 16384, 2100                                 # 2100 * 16384 * 4 B > 128 MiB
    M = 2 * nc
    X = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    u8 = torch.uint8
    ptr = torch.arange(0, M + 1, 2, dtype=torch.int32, device="cuda")
    rows = torch.arange(M, dtype=torch.int32, device="cuda")
    gp = torch.tensor(_lib.svdq_cube_groups(np.arange(0, M + 1, 2, dtype=np.int32)),
                      device="cuda")
    cc = torch.empty(nc, K, dtype=u8, device="cuda")
    dc = torch.empty(M, K // 2, dtype=u8, device="cuda")
    dsc = torch.empty(M, K // 16, dtype=u8, device="cuda")
    with pytest.raises(_lib.SvdqError) as e:
        _lib.svdq_delta_quant_act_noalloc(X, None, torch.ones(1, device="cuda"), ptr, rows, nc,
                                          gp, None, 0, cc, torch.empty(nc, device="cuda"), dc,
                                          dsc, torch.empty(1, device="cuda"), None)
    assert e.value.status == 2 and "static buffer" in str(e.value)
