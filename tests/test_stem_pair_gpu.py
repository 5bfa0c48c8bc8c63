"""GPU parity of the stem pair (k_stem_pair): a stem layer (3x3, one or three
input channels, 16 outputs) and the dense 3x3 layer that alone reads it, run
as one kernel by cvx_forward, the stem's output never written.  Against the
fp64 oracle at |gpu - oracle| <= 1e-4*max(1,|oracle|), for both strides of
each layer, ragged tiles and row blocks, several images, every tile the
kernel takes, residual placements of the second layer, and a list input off a
16-byte boundary (the two-kernel fallback); and with the stem prologue
folded in (the pair resizes and normalises the u8 frame itself), at several
resize ratios, against the oracle and beside the separate prologue
(CVX_STEM_PAIR_U8=0), with a frame off a 16-byte boundary taking the
separate prologue.  The two-kernel path
(CVX_STEM_PAIR=0) is checked against the oracle beside it: the pair computes
the stem on matrix cores, in another summation order, so the two agree to
rounding, not bit for bit."""
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


# (seed, n, c_in, h, w, stride 1, stride 2, c_out 2)
CASES = [(400, 1, 3, 64, 64, 2, 2, 32),
         (401, 2, 3, 40, 56, 2, 2, 48),
         (402, 1, 1, 36, 28, 1, 2, 32),
         (403, 1, 3, 24, 32, 2, 1, 64),
         (404, 3, 3, 20, 20, 1, 1, 40)]
TILES = ["", "216", "232", "208", "116", "108", "132"]


def _forward(wk, monkeypatch, pair: bool, x=None):
    monkeypatch.setenv("CVX_STEM_PAIR", "1" if pair else "0")
    net = Net(wk.layers, wk.x.shape, device=DEV)
    plan = cvx.cvx_forward_plan(net.arr)
    xt = dev(wk.x) if x is None else x
    y = net(xt)
    torch.cuda.synchronize()
    return y.cpu().numpy(), plan


@pytest.mark.parametrize("tile", TILES, ids=[t or "auto" for t in TILES])
@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_stem_pair_matches_oracle(case, tile, monkeypatch):
    seed, n, cin, h, w, s1, s2, cout = case
    if tile:
        monkeypatch.setenv("CVX_STEM_PAIR_TILE", tile)
    wk = wl.stem_pair_case(seed, n, cin, h, w, s1, s2, cout)
    got, plan = _forward(wk, monkeypatch, True)
    say(f"stem pair {case} tile {tile or 'auto'}: {plan[-1]}")
    assert plan[0] == "merged into 1" and "k_stem_pair" in plan[1], plan
    if tile:
        nt, tc = int(tile) // 100, int(tile) % 100
        if f"bn={32 * nt} tc={tc} " not in plan[1]:
            pytest.skip(f"tile {tile} does not fit this shape: {plan[1]}")
    ref = oracle.forward(wk.layers, wk.x)
    check(got, ref, f"stem pair {case} tile {tile}")
    apart, plan0 = _forward(wk, monkeypatch, False)
    assert "k_stem<" in plan0[0] and "k_igemm_packed" in plan0[1], plan0
    check(apart, ref, f"two kernels {case}")


MODES = [(a1, a2, r) for a1, a2 in ((wl.ACT_SILU, wl.ACT_SILU), (wl.ACT_RELU, wl.ACT_NONE))
         for r in (wl.RES_BEFORE_ACT, wl.RES_AFTER_ACT)]


@pytest.mark.parametrize("mode", MODES, ids=[f"a{a}b{b}r{r}" for a, b, r in MODES])
def test_stem_pair_residual_and_activations(mode, monkeypatch):
    act1, act2, res = mode
    wk = wl.stem_pair_case(410, 2, 3, 40, 56, 2, 2, 48, act1, act2, res)
    got, plan = _forward(wk, monkeypatch, True)
    say(f"stem pair modes {mode}: {plan}")
    assert plan[1] == "merged into 2" and "k_stem_pair" in plan[2], plan
    check(got, oracle.forward(wk.layers, wk.x), f"stem pair modes {mode}")


def test_stem_pair_misaligned_input_falls_back(monkeypatch):
    """The stem reads the list input: off a 16-byte boundary the two layers run
    apart (the stem's output keeps a region for that)."""
    wk = wl.stem_pair_case(420, 1, 3, 32, 32, 2, 2, 32)
    flat = torch.empty(wk.x.size + 1, device=DEV)
    x = flat[1:].view(wk.x.shape)
    x.copy_(dev(wk.x))
    assert x.data_ptr() % 16 != 0
    got, plan = _forward(wk, monkeypatch, True, x=x)
    assert "k_stem_pair" in plan[1], plan
    check(got, oracle.forward(wk.layers, wk.x), "stem pair misaligned input")


@pytest.mark.parametrize("batch", [1, 2])
def test_detector_stem_pair_in_pipeline(batch, monkeypatch):
    """The detector pipeline: prologue -> (stem1, stem2 as one kernel) -> the
    rest; the whole forward against the oracle."""
    wk = wl.detector_pipeline(batch)
    got, plan = _forward(wk, monkeypatch, True)
    assert plan[1] == "merged into 2" and "k_stem_pair" in plan[2], plan
    say(f"detector b{batch} with the stem pair")
    check(got, oracle.forward(wk.layers, wk.x), f"detector b{batch} stem pair")


# (seed, batch, src_h, src_w, dst_h, dst_w, stride 1, stride 2, c_out 2)
U8_CASES = [(430, 1, 720, 1280, 640, 640, 2, 2, 32),   # the detector's stem: 1.125 x 2 downscale
            (431, 2, 45, 64, 30, 40, 2, 1, 32),
            (432, 1, 20, 16, 40, 32, 2, 2, 48),        # upscale (clamped first source row)
            (433, 1, 100, 160, 48, 80, 1, 2, 32),      # stride-1 stem
            (434, 3, 96, 144, 64, 80, 2, 2, 40)]


@pytest.mark.parametrize("case", U8_CASES, ids=[f"seed{c[0]}" for c in U8_CASES])
def test_prologue_in_stem_pair(case, monkeypatch):
    wk = wl.prologue_stem_pair(*case)
    ref = oracle.forward(wk.layers, wk.x)
    got, plan = _forward(wk, monkeypatch, True)
    say(f"prologue+stem pair {case}: {plan}")
    assert plan[0] == "merged into 2" and plan[1] == "merged into 2" and "from=u8" in plan[2], plan
    check(got, ref, f"prologue+stem pair {case}")
    monkeypatch.setenv("CVX_STEM_PAIR_U8", "0")
    apart, plan0 = _forward(wk, monkeypatch, True)
    assert plan0[0] == "preprocess" and "from=u8" not in plan0[2], plan0
    check(apart, ref, f"prologue apart {case}")


def test_prologue_in_stem_pair_misaligned_frame(monkeypatch):
    """A frame off a 16-byte boundary: the prologue runs apart (its output
    keeps a region for that), then the pair on its output."""
    wk = wl.prologue_stem_pair(440, 1, 48, 64, 32, 32, 2, 2, 32)
    flat = torch.empty(wk.x.size + 4, dtype=torch.uint8, device=DEV)
    x = flat[4:].view(wk.x.shape)
    x.copy_(torch.from_numpy(wk.x).to(DEV))
    assert x.data_ptr() % 16 != 0
    got, plan = _forward(wk, monkeypatch, True, x=x)
    assert "from=u8" in plan[2], plan
    check(got, oracle.forward(wk.layers, wk.x), "prologue+stem pair, misaligned frame")
