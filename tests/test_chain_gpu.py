"""GPU parity of the chain launch (opt-in with CVX_CHAIN=1): a run of dense
1x1/3x3 layers with packed weights executed as one persistent kernel
(k_chain), whose tiles wait for the rows of earlier layers they read.  Element by element against the oracle at
|gpu - oracle| <= 1e-4*max(1,|oracle|), on the detector chain and on a list
with ragged channels and tiles, residuals from the input, from the layer's own
input and from two layers back (before and after the activation), every tile
configuration the chain takes, split reductions, several images; plus a wait
forced to give up from the host, after which the kernel still ends and the
next launch is correct."""
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


@pytest.fixture(autouse=True)
def chain_on(monkeypatch):
    # the chain launch is opt-in (one launch per layer measured faster); the
    # detector's stem2 chains instead of running with stem1 as one kernel
    monkeypatch.setenv("CVX_CHAIN", "1")
    monkeypatch.setenv("CVX_STEM_PAIR", "0")


def _run(wk, expect_chain=True):
    net = Net(wk.layers, wk.x.shape, device=DEV)
    plan = cvx.cvx_forward_plan(net.arr)
    n_chain = sum(p.startswith("chain") for p in plan)
    if expect_chain:
        assert n_chain >= 2, plan
    say(f"chain forward {wk.name}: {n_chain} chained layers")
    x = dev(wk.x)
    y = net(x)
    torch.cuda.synchronize()
    return net, y.cpu().numpy(), plan


@pytest.mark.parametrize("batch,hw", [(1, 48), (3, 48), (1, 40), (2, 64)])
def test_dense_chain_matches_oracle(batch, hw):
    wk = wl.dense_chain(batch, hw)
    _, got, plan = _run(wk)
    # 40-wide: the last two layers' 10x10 maps have rows of 10 floats, which
    # 16-byte staging cannot take, so the chain stops before them
    first = plan[0].split()[1]
    assert first == ("0-7" if hw % 16 == 0 else "0-5"), plan
    check(got, oracle.forward(wk.layers, wk.x), wk.name)


CHAIN_FORCED = [(tc, sk) for tc in (0, 4, 8, 16, 32) for sk in (1, 2, 3)]


@pytest.mark.parametrize("tc,sk", CHAIN_FORCED, ids=[f"tc{t}sk{s}" for t, s in CHAIN_FORCED])
def test_dense_chain_forced_tiles(tc, sk, monkeypatch):
    # every layer takes the forced 32x32 tile where the chain can run it (else
    # the first tile that fits, unsplit): 2-D and flat tiles, split reductions
    monkeypatch.setenv("CVX_IGEMM_TILE", f"0,{tc},{sk}")
    wk = wl.dense_chain(2, 48)
    _, got, plan = _run(wk)
    say(f"  plan {plan}")
    check(got, oracle.forward(wk.layers, wk.x), f"forced tc={tc} splitk={sk}")


def test_detector_chain_plan_and_parity():
    wk = wl.detector_pipeline(1)
    _, got, plan = _run(wk)
    assert plan[0] == "preprocess" and "k_stem" in plan[1]
    assert all(p.startswith("chain 2-10") for p in plan[2:]), plan
    check(got, oracle.forward(wk.layers, wk.x), "detector chain")


def test_chain_off_matches_oracle(monkeypatch):
    # without CVX_CHAIN=1: one launch per layer, same list
    monkeypatch.delenv("CVX_CHAIN")
    wk = wl.dense_chain(1, 48)
    _, got, plan = _run(wk, expect_chain=False)
    assert not any(p.startswith("chain") for p in plan)
    check(got, oracle.forward(wk.layers, wk.x), "chain off")


def test_chain_repeat_and_dirty_workspace():
    """Back-to-back launches and a workspace filled with ones between them: the
    counters are zeroed by the launch itself and left clear at its end."""
    wk = wl.dense_chain(2, 48)
    net = Net(wk.layers, wk.x.shape, device=DEV)
    x = dev(wk.x)
    ref = oracle.forward(wk.layers, wk.x)
    say("chain repeat")
    first = net(x).clone()
    torch.cuda.synchronize()
    check(first.cpu().numpy(), ref, "first")
    for i in range(3):
        if i == 1:
            net.workspace.fill_(255)
        again = net(x)
        torch.cuda.synchronize()
        assert torch.equal(again, first), f"launch {i + 2} differs"


def test_chain_wait_gives_up_and_kernel_ends(monkeypatch):
    """A layer's inputs made unreachable from the host (CVX_CHAIN_STALL) with a
    tiny poll bound (CVX_CHAIN_SPIN): the waiting tiles give up, the abort word
    makes every later wait return, the kernel ends normally and the output is
    poisoned with NaN; the next launch without the knobs is correct."""
    wk = wl.dense_chain(1, 48)
    net = Net(wk.layers, wk.x.shape, device=DEV)
    x = dev(wk.x)
    monkeypatch.setenv("CVX_CHAIN_STALL", "2")
    monkeypatch.setenv("CVX_CHAIN_SPIN", "64")
    say("chain stall: waits give up")
    y = net(x)
    torch.cuda.synchronize()
    assert torch.isnan(y).any(), "a wait that gave up must poison the output"
    monkeypatch.delenv("CVX_CHAIN_STALL")
    monkeypatch.delenv("CVX_CHAIN_SPIN")
    say("chain after the stall")
    y = net(x)
    torch.cuda.synchronize()
    check(y.cpu().numpy(), oracle.forward(wk.layers, wk.x), "after stall")


def test_chain_graph_replays():
    """The chain launch captured in a HIP graph (its tag frozen) and replayed:
    the last workgroup of each launch clears the flag, so every replay starts
    clean and equals the eager result, with eager launches in between."""
    wk = wl.dense_chain(2, 48)
    net = Net(wk.layers, wk.x.shape, device=DEV)
    x = dev(wk.x)
    eager = net(x).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        net(x)
    torch.cuda.synchronize()
    for i in range(4):
        say(f"chain graph replay {i}")
        net.output.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(net.output, eager), f"replay {i}"
        net(x)
        torch.cuda.synchronize()
