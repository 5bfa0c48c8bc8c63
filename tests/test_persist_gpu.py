"""GPU parity of the persistent form of the packed implicit GEMM
(`k_igemm_persist`): fewer workgroups than tiles, each running a stream of
tiles whose stages continue across tile boundaries.  Forced through
CVX_IGEMM_TILE="kind,tc,1,workgroups" on shapes where every workgroup runs
several tiles (ragged pixel tiles, ragged row blocks, several images, both
workgroup orders, every activation and residual placement), against the fp64
oracle at |gpu - oracle| <= 1e-4*max(1,|oracle|), with NaN guard bands."""
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


# (seed, n, c_in, h, w, c_out, k, stride, pad): widths a multiple of 4 (the
# persistent form stages 16 bytes at a time), at least two stages per tile
# and at least 24 tiles (so that 24 workgroups each get several)
SHAPES = [(300, 2, 48, 19, 28, 70, 3, 1, 1),
          (301, 3, 40, 46, 40, 100, 3, 2, 1),
          (302, 4, 160, 9, 16, 96, 1, 1, 0),
          (303, 2, 128, 10, 20, 100, 1, 1, 0)]
CONFIGS = [(kind, tc, wgs) for kind in (0, 1) for tc in (0, 8, 16) for wgs in (8, 24)]


@pytest.mark.parametrize("order", ["blocks", "pixels"])
@pytest.mark.parametrize("cfg", CONFIGS, ids=[f"t{k}tc{t}wg{g}" for k, t, g in CONFIGS])
def test_persistent_forced(cfg, order, monkeypatch):
    kind, tc, wgs = cfg
    monkeypatch.setenv("CVX_PACKED_ORDER", order)
    monkeypatch.setenv("CVX_IGEMM_TILE", f"{kind},{tc},1,{wgs}")
    tested = 0
    for seed, n, cin, h, w, cout, k, s, p in SHAPES:
        x, L = wl.random_conv_case(seed, n, cin, h, w, cout, k, s, p, 1, wl.ACT_SILU, wl.RES_AFTER_ACT)
        d = cvx.make_desc(n, cin, h, w, cout, k, s, p, 1, wl.ACT_SILU, wl.RES_AFTER_ACT, PACKED)
        plan = cvx.cvx_conv_plan(d)
        if f"tile={kind} " not in plan or f"tc={tc} " not in plan:
            continue  # the forced tile does not fit this shape (its staged region is too large)
        # fewer tiles than asked for: the workgroup count is cut to a multiple of 8 below the tile count
        assert "persist=" in plan and "k_igemm_persist" in plan, plan
        tested += 1
        oh, ow = cvx.cvx_conv_out_shape(d)
        r = wl.residual_for(seed, (n, cout, oh, ow))
        say(f"persist {cfg} {order} seed {seed}: {plan}")
        y, ok = gpu_conv(x, L, r, PACKED)
        assert ok, "write outside the output"
        check(y, oracle_conv(x, L, r), f"persist {cfg} {order} seed {seed}")
    assert tested >= 3, tested


MODES = [(act, res) for act in (wl.ACT_NONE, wl.ACT_RELU, wl.ACT_SILU)
         for res in (wl.RES_NONE, wl.RES_BEFORE_ACT, wl.RES_AFTER_ACT)]


@pytest.mark.parametrize("mode", MODES, ids=[f"act{a}res{r}" for a, r in MODES])
def test_persistent_epilogue_modes(mode, monkeypatch):
    act, res = mode
    monkeypatch.setenv("CVX_IGEMM_TILE", "0,0,1,16")
    for seed, n, cin, h, w, cout, k, s, p in [(310, 2, 64, 12, 16, 64, 3, 1, 1),
                                              (311, 2, 96, 16, 8, 96, 1, 1, 0)]:
        x, L = wl.random_conv_case(seed, n, cin, h, w, cout, k, s, p, 1, act, res)
        d = cvx.make_desc(n, cin, h, w, cout, k, s, p, 1, act, res, PACKED)
        plan = cvx.cvx_conv_plan(d)
        assert "persist=16 " in plan, plan
        oh, ow = cvx.cvx_conv_out_shape(d)
        r = wl.residual_for(seed, (n, cout, oh, ow)) if res else None
        say(f"persist modes act={act} res={res} seed {seed}")
        y, ok = gpu_conv(x, L, r, PACKED)
        assert ok, "write outside the output"
        check(y, oracle_conv(x, L, r), f"persist act={act} res={res} seed {seed}")


@pytest.mark.parametrize("name,kind,tc", [("c_128x40_1x1", 1, 16), ("d_128x40_3x3", 0, 0),
                                          ("e_128x40_3x3s2", 0, 8), ("f_256x20_1x1", 1, 0)])
def test_persistent_detector_layers_b8(name, kind, tc, monkeypatch):
    """The detector's layers at batch 8, each workgroup running several tiles
    (the device holds 256 or 512 workgroups at once)."""
    wk = wl.sweep_layer(name, batch=8)
    L = wk.layers[0]
    x = wk.x
    n, c, h, w = x.shape
    d = cvx.make_desc(n, c, h, w, L.cout, L.k, L.stride, L.pad, L.groups, L.act, L.res_mode, PACKED)
    monkeypatch.setenv("CVX_IGEMM_TILE", f"{kind},{tc},1,256")
    plan = cvx.cvx_conv_plan(d)
    assert "persist=256 " in plan, plan
    r = x if L.res_mode else None
    say(f"persist b8 {name}: {plan}")
    y, ok = gpu_conv(x, L, r, PACKED)
    assert ok, "write outside the output"
    check(y, oracle_conv(x, L, r), f"persist b8 {name}")


def test_persistent_repeat_is_deterministic(monkeypatch):
    monkeypatch.setenv("CVX_IGEMM_TILE", "0,8,1,64")
    wk = wl.sweep_layer("d_128x40_3x3")
    L = wk.layers[0]
    say("persist determinism d")
    y1, _ = gpu_conv(wk.x, L, wk.x)
    y2, _ = gpu_conv(wk.x, L, wk.x)
    assert np.array_equal(y1, y2)
