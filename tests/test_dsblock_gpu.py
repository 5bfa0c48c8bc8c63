"""A depthwise-separable block as one launch (k_dsblock) against the oracle.

The block is a depthwise 3x3 layer (BN, activation), the 1x1 layer that alone
reads it (BN) and the block's shortcut -- none, the block input itself added
before or after the activation, or a strided 1x1 convolution of the block input
(BN) added before it ("Как я свертки ускорял", "Пациента на стол" and "А
теперь — хардкор на Metal": one launch instead of three).  Cases cover both
weight layouts, input channels that are not a multiple of 16, output channels
that are not a multiple of 32, pixel runs with a ragged tail, strides 1 and 2,
and several images.  Every case checks that the planner chose the block kernel.
The kernel is opt-in (CVX_DSBLOCK=1; measured slower than the separate kernels
on the MNIST net), so each test turns it on.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import DEV, check, dev, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from conv2d_batchnorm_activation_amd import cvx  # noqa: E402  (raises if libcvx is not built)
from conv2d_batchnorm_activation_amd.net import Net  # noqa: E402


def _block(n, cin, hw, cout, stride, dw_act, shortcut, act=wl.ACT_RELU, seed=31):
    """1x1 -> [dw 3x3 -> pw 1x1 + shortcut] -> 1x1, the middle three as the block."""
    rng = wl.rng_for(seed)
    x = rng.uniform(-1.0, 1.0, (n, cin, hw, hw)).astype(np.float32)
    L = [wl.conv_layer(rng, cin, cin, 1, 1, 0, act=wl.ACT_RELU, name="in1x1")]
    L.append(wl.conv_layer(rng, cin, cin, 3, stride, 1, groups=cin, act=dw_act, inp=0, name="dw"))
    if shortcut in ("proj", "proj_act"):
        # a shortcut with an activation does not run inside: its output is
        # added as a residual tensor
        skip_act = wl.ACT_NONE if shortcut == "proj" else wl.ACT_RELU
        L.append(wl.conv_layer(rng, cin, cout, 1, stride, 0, act=skip_act, inp=0, name="skip"))
        L.append(wl.conv_layer(rng, cin, cout, 1, 1, 0, act=act, res_mode=wl.RES_BEFORE_ACT, inp=1, res=2,
                               name="pw"))
    elif shortcut in ("before", "after"):
        mode = wl.RES_BEFORE_ACT if shortcut == "before" else wl.RES_AFTER_ACT
        L.append(wl.conv_layer(rng, cin, cout, 1, 1, 0, act=act, res_mode=mode, inp=1, res=0, name="pw"))
    else:
        L.append(wl.conv_layer(rng, cin, cout, 1, 1, 0, act=act, inp=1, name="pw"))
    L.append(wl.conv_layer(rng, cout, cout, 1, 1, 0, act=wl.ACT_NONE, inp=len(L) - 1, name="out1x1"))
    return wl.Workload(f"dsblock_n{n}_{cin}x{hw}_{cout}_s{stride}_{shortcut}", x, L)


CASES = [
    # n, cin, hw, cout, stride, dw_act, shortcut, pw act
    (1, 48, 28, 96, 2, wl.ACT_RELU, "proj", wl.ACT_RELU),      # MNIST block 0
    (1, 96, 14, 96, 1, wl.ACT_RELU, "before", wl.ACT_RELU),    # MNIST block 1
    (1, 96, 14, 192, 2, wl.ACT_RELU, "proj", wl.ACT_RELU),     # MNIST block 2
    (1, 192, 7, 192, 1, wl.ACT_RELU, "before", wl.ACT_RELU),   # MNIST block 3
    (2, 40, 9, 40, 1, wl.ACT_SILU, "after", wl.ACT_SILU),      # ragged channels and plane, residual after act
    (3, 24, 11, 56, 2, wl.ACT_NONE, "proj", wl.ACT_RELU),      # odd plane at stride 2, 3 images
    (1, 17, 13, 33, 1, wl.ACT_RELU, "none", wl.ACT_SILU),      # no shortcut, odd channels
    (2, 256, 6, 64, 1, wl.ACT_RELU, "none", wl.ACT_RELU),      # the widest input it takes
    (1, 192, 8, 40, 2, wl.ACT_RELU, "proj", wl.ACT_NONE),      # a projection over a whole 8x8 plane
    (4, 32, 10, 32, 1, wl.ACT_RELU, "before", wl.ACT_RELU),    # four images
    (2, 48, 12, 64, 2, wl.ACT_RELU, "proj_act", wl.ACT_RELU),  # shortcut computed apart
]


@pytest.mark.parametrize("layout", [cvx.CVX_W_PACKED, cvx.CVX_W_OIHW])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"n{c[0]}_{c[1]}x{c[2]}_{c[3]}_s{c[4]}_{c[6]}")
def test_dsblock_matches_oracle(case, layout, monkeypatch):
    monkeypatch.setenv("CVX_CHAIN", "0")
    monkeypatch.setenv("CVX_DSBLOCK", "1")
    wk = _block(*case)
    net = Net(wk.layers, wk.x.shape, device=DEV, w_layout=layout)
    plan = cvx.cvx_forward_plan(net.arr)
    pw = len(wk.layers) - 2
    assert "kernel=cvx::k_dsblock" in plan[pw], plan
    assert plan[1] == f"merged into {pw}", plan
    say(f"dsblock {wk.name} layout={layout}: {plan[pw]}")
    y = net(dev(wk.x))
    torch.cuda.synchronize()
    check(y.cpu().numpy(), oracle.forward(wk.layers, wk.x), wk.name)


def test_mnist_b1_forward_runs_blocks_as_one_launch_each(monkeypatch):
    monkeypatch.setenv("CVX_DSBLOCK", "1")
    wk = wl.mnist_cnn(1)
    net = Net(wk.layers, wk.x.shape, device=DEV)
    plan = cvx.cvx_forward_plan(net.arr)
    assert sum("k_dsblock" in p for p in plan) == 4, plan
    y = net(dev(wk.x))
    torch.cuda.synchronize()
    check(y.cpu().numpy(), oracle.forward(wk.layers, wk.x), wk.name)


def test_dsblock_off_matches_on(monkeypatch):
    """CVX_DSBLOCK=1 runs each block as one kernel, unset the layers run apart;
    both give the oracle's result."""
    wk = wl.mnist_cnn(2)
    x = dev(wk.x)
    monkeypatch.setenv("CVX_DSBLOCK", "1")
    net_on = Net(wk.layers, wk.x.shape, device=DEV)
    y_on = net_on(x).cpu().numpy()
    monkeypatch.delenv("CVX_DSBLOCK")
    net_off = Net(wk.layers, wk.x.shape, device=DEV)
    assert not any("k_dsblock" in p for p in cvx.cvx_forward_plan(net_off.arr))
    y_off = net_off(x).cpu().numpy()
    ref = oracle.forward(wk.layers, wk.x)
    check(y_on, ref, "dsblock on")
    check(y_off, ref, "dsblock off")
