"""GPU parity of the 1x1 GEMM kernel (k_gemm1x1: a wave per 32 x 32 output
block over the whole reduction) against the fp64 oracle, through the C ABI,
element by element at |gpu - oracle| <= 1e-4*max(1,|oracle|), with NaN guard
bands around every output.

CVX_GEMM1X1=1 makes the planner take the kernel for every 1x1 stride-1 layer
it fits, so the cases can span ragged pixel counts (not a multiple of 32),
partial channel chunks (c_in not a multiple of 16), c_out not a multiple of
32 or of 4 (the scale and bias then load one channel at a time), several
images per launch, every activation and residual placement, and misaligned
scale and bias; the detector's own 1x1 layers run at batch 1 and 8 (at
batch 8 they take the kernel without being forced).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, Guarded, check, dev, say

pytestmark = pytest.mark.gpu

from conv2d_batchnorm_activation_amd import cvx  # noqa: E402
from test_parity_gpu import PACKED, gpu_conv, oracle_conv  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture
def gemm1x1(monkeypatch):
    monkeypatch.setenv("CVX_GEMM1X1", "1")


CASES = [
    # (seed, n, cin, h, w, cout, act, res_mode)
    (700, 1, 128, 40, 40, 128, wl.ACT_SILU, wl.RES_AFTER_ACT),    # the detector's c at b=1
    (701, 1, 256, 20, 20, 256, wl.ACT_SILU, wl.RES_AFTER_ACT),    # f: 400 pixels, a 16-pixel last block
    (702, 2, 48, 7, 9, 40, wl.ACT_RELU, wl.RES_BEFORE_ACT),       # 63 pixels, 40 channels
    (703, 3, 20, 5, 5, 33, wl.ACT_NONE, wl.RES_NONE),             # partial chunk, c_out 33
    (704, 1, 16, 1, 1, 16, wl.ACT_SILU, wl.RES_NONE),             # one pixel
    (705, 5, 96, 14, 14, 192, wl.ACT_RELU, wl.RES_BEFORE_ACT),    # MNIST-like plane, 5 images
    (706, 2, 200, 11, 13, 64, wl.ACT_SILU, wl.RES_AFTER_ACT),     # c_in 200: 13 chunks (odd count)
    (707, 1, 32, 33, 31, 100, wl.ACT_SILU, wl.RES_NONE),          # 1023 pixels, c_out 100
]


@pytest.mark.parametrize("c", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_gemm1x1_cases(c, gemm1x1):
    seed, n, cin, h, w, cout, act, rm = c
    x, L = wl.random_conv_case(seed, n, cin, h, w, cout, 1, 1, 0, 1, act, rm)
    d = cvx.make_desc(n, cin, h, w, cout, 1, 1, 0, 1, act, rm, PACKED)
    plan = cvx.cvx_conv_plan(d)
    assert plan.startswith("gemm1x1"), plan
    r = wl.residual_for(seed, (n, cout, h, w)) if rm else None
    say(f"gemm1x1 case {seed}: n={n} {cin}x{h}x{w} -> {cout} act={act} res={rm} [{plan}]")
    y, ok = gpu_conv(x, L, r, PACKED)
    assert ok, "write outside the output"
    check(y, oracle_conv(x, L, r), f"gemm1x1 case {seed}")


@pytest.mark.parametrize("name", ["c_128x40_1x1", "f_256x20_1x1"])
def test_gemm1x1_detector_b8_layers(name):
    """The detector's 1x1 layers at batch 8 (1600 and 832 output blocks) take
    the kernel by default; every image against the oracle."""
    wk = wl.sweep_layer(name, batch=8)
    L = wk.layers[0]
    n, c, h, w = wk.x.shape
    d = cvx.make_desc(n, c, h, w, L.cout, L.k, L.stride, L.pad, L.groups, L.act, L.res_mode, PACKED)
    plan = cvx.cvx_conv_plan(d)
    assert plan.startswith("gemm1x1"), plan
    say(f"gemm1x1 {name} b=8 [{plan}]")
    r = wk.x if L.res_mode else None
    y, ok = gpu_conv(wk.x, L, r, PACKED)
    assert ok, "write outside the output"
    check(y, oracle_conv(wk.x, L, r), f"{name} b=8")


def test_gemm1x1_misaligned_scale_bias(gemm1x1):
    """Scale and bias off a 16-byte boundary load one channel at a time."""
    seed, n, cin, h, w, cout = 710, 1, 64, 8, 12, 64
    x, L = wl.random_conv_case(seed, n, cin, h, w, cout, 1, 1, 0, 1, wl.ACT_SILU, wl.RES_NONE)
    d = cvx.make_desc(n, cin, h, w, cout, 1, 1, 0, 1, wl.ACT_SILU, wl.RES_NONE, PACKED)
    assert cvx.cvx_conv_plan(d).startswith("gemm1x1")
    p = L.params
    wp = torch.full((cvx.cvx_packed_weights_bytes(d) // 4,), float("nan"), device=DEV)
    cvx.cvx_pack_weights(d, dev(p["w"]), wp)
    g, b, m, v = (dev(p[k]) for k in ("gamma", "beta", "mean", "var"))
    sb = torch.empty(2 * cout + 2, device=DEV)
    scale, bias = sb[1:1 + cout], sb[2 + cout:2 + 2 * cout]  # 4-byte aligned, not 16
    cvx.cvx_fold_bn(g, b, m, v, wl.EPS, scale, bias)
    out = Guarded((n, cout, h, w))
    cvx.cvx_conv_bn_act(d, dev(x), wp, scale, bias, None, out.t, torch.empty(4, dtype=torch.uint8,
                                                                             device=DEV), 0)
    torch.cuda.synchronize()
    assert out.guards_intact()
    check(out.t.cpu().numpy(), oracle_conv(x, L, None), "gemm1x1 misaligned scale/bias")


def test_gemm1x1_deterministic(gemm1x1):
    seed, n, cin, h, w, cout = 711, 2, 64, 10, 10, 96
    x, L = wl.random_conv_case(seed, n, cin, h, w, cout, 1, 1, 0, 1, wl.ACT_RELU, wl.RES_NONE)
    y1, _ = gpu_conv(x, L, None, PACKED)
    y2, _ = gpu_conv(x, L, None, PACKED)
    assert np.array_equal(y1, y2)
