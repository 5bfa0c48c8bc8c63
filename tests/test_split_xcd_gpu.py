"""The split reduction's two paths.  With the slices of a tile on one XCD
(the default once the device's placement check passes) the partial sums meet
in that XCD's L2; with CVX_SPLIT_XCD=0 they meet in device-coherent memory.
Both must match the fp64 oracle at |gpu - oracle| <= 1e-4*max(1,|oracle|) and
each other bit for bit (the slices are summed in the same order), on split
counts 2-4, both workgroup orders, ragged tiles, and grids that need padding
to a multiple of 8 x splits workgroups."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import say
from test_parity_gpu import PACKED, check, gpu_conv, oracle_conv

pytestmark = pytest.mark.gpu

from conv2d_batchnorm_activation_amd import cvx  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_workgroup_placement():
    """Workgroups whose indices agree modulo 8 run on one XCD: the property the
    L2 reduction path needs (the library checks it once per device)."""
    out = torch.full((4096,), -1, dtype=torch.int32, device="cuda:0")
    say("placement of 4096 workgroups")
    cvx.cvx_workgroup_xcds(out)
    torch.cuda.synchronize()
    x = out.cpu().numpy()
    assert ((x >= 0) & (x < 16)).all(), np.unique(x)
    assert (x == np.tile(x[:8], 512)).all(), "workgroups i and i+8 on different XCDs"
    say(f"XCDs in use: {sorted(set(x[:8].tolist()))}")


# (seed, n, c_in, h, w, c_out, k, stride, pad): tile counts that are not a
# multiple of 8 (padding workgroups), ragged pixel tiles and row blocks
SHAPES = [(400, 1, 128, 20, 20, 100, 3, 1, 1),
          (401, 2, 96, 13, 17, 70, 3, 2, 1),
          (402, 1, 256, 10, 10, 256, 3, 1, 1),
          (403, 3, 160, 9, 11, 40, 1, 1, 0)]
CONFIGS = [(order, kind, tc, sk) for order in ("blocks", "pixels") for kind in (0, 1)
           for tc in (0, 8) for sk in (2, 3, 4)]


@pytest.mark.parametrize("cfg", CONFIGS, ids=[f"{o}-t{k}tc{t}sk{s}" for o, k, t, s in CONFIGS])
def test_split_paths_match_oracle_and_each_other(cfg, monkeypatch):
    order, kind, tc, sk = cfg
    monkeypatch.setenv("CVX_PACKED_ORDER", order)
    monkeypatch.setenv("CVX_IGEMM_TILE", f"{kind},{tc},{sk}")
    for seed, n, cin, h, w, cout, k, s, p in SHAPES:
        x, L = wl.random_conv_case(seed, n, cin, h, w, cout, k, s, p, 1, wl.ACT_SILU, wl.RES_AFTER_ACT)
        d = cvx.make_desc(n, cin, h, w, cout, k, s, p, 1, wl.ACT_SILU, wl.RES_AFTER_ACT, PACKED)
        plan = cvx.cvx_conv_plan(d)
        if f"splitk={sk} " not in plan:
            continue
        oh, ow = cvx.cvx_conv_out_shape(d)
        r = wl.residual_for(seed, (n, cout, oh, ow))
        ref = oracle_conv(x, L, r)
        ys = []
        for path in ("1", "0"):
            monkeypatch.setenv("CVX_SPLIT_XCD", path)
            say(f"split {cfg} seed {seed} xcd={path}: {plan}")
            y, ok = gpu_conv(x, L, r, PACKED)
            assert ok, "write outside the output"
            check(y, ref, f"split {cfg} seed {seed} xcd={path}")
            ys.append(y)
        assert np.array_equal(ys[0], ys[1]), f"paths differ: {cfg} seed {seed}"


@pytest.mark.parametrize("name", ["e_128x40_3x3s2", "g_256x20_3x3"])
@pytest.mark.parametrize("batch", [1, 8])
def test_detector_split_layers(name, batch, monkeypatch):
    """The detector's layers with a split reduction, forced to 2 and 4 slices,
    through the L2 path, repeated (the counters reset themselves).  At batch 8
    the grid is several times what the device holds at once, so workgroups of
    neighbouring tiles share compute units over time."""
    wk = wl.sweep_layer(name, batch=batch)
    L = wk.layers[0]
    r = wk.x if L.res_mode else None
    ref = oracle_conv(wk.x, L, r)
    for sk in (2, 4):
        monkeypatch.setenv("CVX_IGEMM_TILE", f"0,0,{sk}")
        first = None
        for rep in range(4):
            say(f"detector {name} b{batch} split {sk} rep {rep}")
            y, ok = gpu_conv(wk.x, L, r, PACKED)
            assert ok, "write outside the output"
            check(y, ref, f"{name} b{batch} split {sk}")
            if first is None:
                first = y
            else:
                assert np.array_equal(first, y)
