"""The allocation-free forward (cvx_forward_noalloc, workspace in a static
device array) against cvx_forward with a caller workspace, on the same layer
lists and inputs: two calls in a row, the second with a smaller input (the
array keeps the first call's contents), each checked element by element at
|noalloc - forward| <= 1e-4*max(1,|forward|), and the first also against the
oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import DEV, check, dev, say

pytestmark = pytest.mark.gpu

from conv2d_batchnorm_activation_amd import cvx  # noqa: E402
from conv2d_batchnorm_activation_amd.net import Net  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(wk):
    net = Net(wk.layers, wk.x.shape, device=DEV)
    assert net.ws_bytes <= cvx.cvx_static_scratch_bytes(), net.ws_bytes
    x = dev(wk.x)
    ref = net(x).clone()
    got = torch.full(net.out_shape, float("nan"), device=DEV)
    say(f"noalloc forward {wk.name} (workspace {net.ws_bytes} bytes)")
    cvx.cvx_forward_noalloc(net.arr, x, got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def test_noalloc_forward_matches_forward_twice_smaller_second():
    # detector b=1: every kernel family, a split reduction (its partial sums and
    # arrival counters in the static array); then a smaller list on the array
    # the first call left behind
    wk = wl.detector_pipeline(1)
    got, ref = _both(wk)
    check(got, ref, "detector b1 noalloc vs forward")
    check(got, oracle.forward(wk.layers, wk.x), "detector b1 noalloc vs oracle")
    wk2 = wl.mnist_cnn(4)
    got2, ref2 = _both(wk2)
    check(got2, ref2, "mnist b4 noalloc vs forward")
    # and the first list again, after the smaller one
    got3, _ = _both(wk)
    check(got3, ref, "detector b1 noalloc, third call")
