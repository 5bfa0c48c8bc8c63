"""Pins of the CPU oracle against facts fixed outside it.

Each test ties an oracle function to something other than itself: a library
routine computing the same definition (torch CPU float64), an independent
brute-force formulation on tiny inputs, closed forms and invariants, or figures
the source pages print (``tests/golden/page_figures.json``).  The cases are
chosen so that a dropped term, a wrong sign or index, or a transposed operand
in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl
from conv2d_batchnorm_activation_amd import accounting

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _rand(rng, *shape, lo=-1.0, hi=1.0):
    return rng.uniform(lo, hi, shape).astype(np.float32)


# ----------------------------------------------------------------------------- conv
CONV_CASES = [
    # n, cin, h, w, cout, k, stride, pad, groups
    (1, 3, 9, 7, 4, 3, 1, 1, 1),
    (2, 4, 8, 11, 6, 3, 2, 1, 1),
    (1, 6, 13, 13, 6, 3, 1, 1, 6),      # depthwise, odd size
    (2, 8, 14, 10, 8, 3, 2, 1, 8),      # depthwise stride 2
    (1, 5, 7, 9, 3, 1, 1, 0, 1),        # pointwise
    (2, 4, 10, 9, 5, 1, 2, 0, 1),       # strided pointwise
    (1, 4, 9, 9, 6, 5, 2, 2, 2),        # grouped 5x5
    (1, 2, 6, 5, 3, 3, 1, 0, 1),        # no padding
    (1, 3, 12, 12, 2, 7, 3, 3, 1),      # 7x7 stride 3
    (1, 2, 5, 6, 4, 3, 1, 2, 1),        # padding wider than the halo
]


@pytest.mark.parametrize("case", CONV_CASES)
def test_conv_matches_torch_float64(case):
    n, cin, h, w, cout, k, s, p, g = case
    rng = np.random.default_rng(hash(case) % (2 ** 32))
    x = _rand(rng, n, cin, h, w)
    wt = _rand(rng, cout, cin // g, k, k)
    ref = F.conv2d(torch.from_numpy(x).double(), torch.from_numpy(wt).double(),
                   stride=s, padding=p, groups=g).numpy()
    got = oracle.conv2d(x, wt, s, p, g)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _bruteforce_conv(x, wt, s, p, g):
    """Independent formulation: pad explicitly, then sum window * kernel."""
    x = x.astype(np.float64)
    wt = wt.astype(np.float64)
    n, cin, h, w = x.shape
    cout, cin_g, kh, kw = wt.shape
    xp = np.zeros((n, cin, h + 2 * p, w + 2 * p))
    xp[:, :, p:p + h, p:p + w] = x
    oh = (h + 2 * p - kh) // s + 1
    ow = (w + 2 * p - kw) // s + 1
    out = np.zeros((n, cout, oh, ow))
    per_g = cout // g
    for b in range(n):
        for co in range(cout):
            gi = co // per_g
            for i in range(oh):
                for j in range(ow):
                    win = xp[b, gi * cin_g:(gi + 1) * cin_g, i * s:i * s + kh, j * s:j * s + kw]
                    out[b, co, i, j] = float((win * wt[co]).sum())
    return out


@pytest.mark.parametrize("case", CONV_CASES[:8])
def test_conv_bruteforce_tiny(case):
    n, cin, h, w, cout, k, s, p, g = case
    rng = np.random.default_rng(7 + sum(case))
    x = _rand(rng, n, cin, h, w)
    wt = _rand(rng, cout, cin // g, k, k)
    np.testing.assert_allclose(oracle.conv2d(x, wt, s, p, g), _bruteforce_conv(x, wt, s, p, g),
                               rtol=1e-12, atol=1e-12)


def test_delta_kernel_is_identity_and_subsample():
    rng = np.random.default_rng(1)
    x = _rand(rng, 2, 5, 9, 8)
    wt = np.zeros((5, 1, 3, 3), np.float32)
    wt[:, 0, 1, 1] = 1.0
    np.testing.assert_array_equal(oracle.conv2d(x, wt, 1, 1, 5), x.astype(np.float64))
    np.testing.assert_array_equal(oracle.conv2d(x, wt, 2, 1, 5), x[:, :, ::2, ::2].astype(np.float64))
    # an off-centre tap shifts the image by one row and zero-fills the edge
    wt2 = np.zeros((5, 1, 3, 3), np.float32)
    wt2[:, 0, 0, 1] = 1.0
    shifted = np.zeros_like(x, dtype=np.float64)
    shifted[:, :, 1:, :] = x[:, :, :-1, :]
    np.testing.assert_array_equal(oracle.conv2d(x, wt2, 1, 1, 5), shifted)


def test_pointwise_is_matmul():
    rng = np.random.default_rng(2)
    x = _rand(rng, 3, 7, 5, 6)
    wt = _rand(rng, 4, 7, 1, 1)
    ref = np.einsum("oc,nchw->nohw", wt[:, :, 0, 0].astype(np.float64), x.astype(np.float64))
    np.testing.assert_allclose(oracle.conv2d(x, wt, 1, 0, 1), ref, rtol=1e-12, atol=1e-13)
    # stride 2 pointwise = matmul on the subsampled grid
    ref2 = np.einsum("oc,nchw->nohw", wt[:, :, 0, 0].astype(np.float64),
                     x[:, :, ::2, ::2].astype(np.float64))
    np.testing.assert_allclose(oracle.conv2d(x, wt, 2, 0, 1), ref2, rtol=1e-12, atol=1e-13)


def test_depthwise_is_per_channel_conv():
    rng = np.random.default_rng(3)
    x = _rand(rng, 2, 6, 11, 9)
    wt = _rand(rng, 6, 1, 3, 3)
    got = oracle.conv2d(x, wt, 2, 1, 6)
    for c in range(6):
        one = oracle.conv2d(x[:, c:c + 1], wt[c:c + 1], 2, 1, 1)
        np.testing.assert_array_equal(got[:, c:c + 1], one)


def test_constant_input_interior_and_linearity():
    rng = np.random.default_rng(4)
    wt = _rand(rng, 3, 4, 3, 3)
    x = np.full((1, 4, 8, 8), 0.75, np.float32)
    y = oracle.conv2d(x, wt, 1, 1, 1)
    inner = 0.75 * wt.astype(np.float64).sum(axis=(1, 2, 3))
    np.testing.assert_allclose(y[0, :, 1:-1, 1:-1], np.broadcast_to(inner[:, None, None], (3, 6, 6)),
                               rtol=1e-13)
    # corners see only 4 of the 9 taps
    corner = 0.75 * wt[:, :, 1:, 1:].astype(np.float64).sum(axis=(1, 2, 3))
    np.testing.assert_allclose(y[0, :, 0, 0], corner, rtol=1e-13)
    a = _rand(rng, 1, 4, 8, 8)
    b = _rand(rng, 1, 4, 8, 8)
    lhs = oracle.conv2d(2.0 * a.astype(np.float64) - 3.0 * b.astype(np.float64), wt, 1, 1, 1)
    rhs = 2.0 * oracle.conv2d(a, wt, 1, 1, 1) - 3.0 * oracle.conv2d(b, wt, 1, 1, 1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-12)


def test_out_extent():
    assert oracle.out_extent(80, 3, 1, 1) == 80
    assert oracle.out_extent(80, 3, 2, 1) == 40
    assert oracle.out_extent(13, 3, 1, 1) == 13
    assert oracle.out_extent(28, 1, 2, 0) == 14
    assert oracle.out_extent(7, 3, 2, 1) == 4
    assert oracle.out_extent(640, 3, 2, 1) == 320


# ----------------------------------------------------------------------------- BN
def test_bn_with_identity_params_is_plain_conv():
    rng = np.random.default_rng(5)
    x = _rand(rng, 1, 3, 6, 6)
    wt = _rand(rng, 4, 3, 3, 3)
    mean = _rand(rng, 4)
    var = rng.uniform(0.5, 1.5, 4)
    gamma = np.sqrt(var + 1e-5)
    y = oracle.conv_bn_act(x, wt, gamma, mean, mean, var, 1e-5, 1, 1, 1, oracle.ACT_NONE)
    np.testing.assert_allclose(y, oracle.conv2d(x, wt, 1, 1, 1), rtol=1e-12, atol=1e-12)


def test_bn_matches_torch_batch_norm():
    rng = np.random.default_rng(6)
    x = _rand(rng, 2, 3, 7, 5)
    wt = _rand(rng, 5, 3, 3, 3)
    bn = wl.draw_bn(rng, 5)
    conv = F.conv2d(torch.from_numpy(x).double(), torch.from_numpy(wt).double(), padding=1)
    ref = F.batch_norm(conv, torch.from_numpy(bn["mean"]).double(), torch.from_numpy(bn["var"]).double(),
                       torch.from_numpy(bn["gamma"]).double(), torch.from_numpy(bn["beta"]).double(),
                       training=False, eps=1e-5).numpy()
    got = oracle.conv_bn_act(x, wt, bn["gamma"], bn["beta"], bn["mean"], bn["var"], 1e-5, 1, 1, 1,
                             oracle.ACT_NONE)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_fold_equals_unfolded():
    rng = np.random.default_rng(8)
    bn = wl.draw_bn(rng, 37)
    scale, bias = oracle.fold_bn(bn["gamma"], bn["beta"], bn["mean"], bn["var"], 1e-5)
    v = rng.normal(size=(11, 37))
    g, b, m, var = (bn[k].astype(np.float64) for k in ("gamma", "beta", "mean", "var"))
    unfolded = (v - m) / np.sqrt(var + 1e-5) * g + b
    np.testing.assert_allclose(scale * v + bias, unfolded, rtol=1e-12, atol=1e-13)
    # gamma = sqrt(var+eps), beta = mean  =>  scale = 1, bias = 0
    s1, b1 = oracle.fold_bn(np.sqrt(var + 1e-5), m, m, var, 1e-5)
    np.testing.assert_allclose(s1, 1.0, rtol=1e-14)
    np.testing.assert_allclose(b1, 0.0, atol=1e-15)


# ----------------------------------------------------------------------------- activation / residual
def test_activation_closed_forms():
    v = np.linspace(-30, 30, 601)
    relu = oracle.activation(v, oracle.ACT_RELU)
    silu = oracle.activation(v, oracle.ACT_SILU)
    np.testing.assert_array_equal(relu, np.maximum(v, 0.0))
    np.testing.assert_array_equal(oracle.activation(relu, oracle.ACT_RELU), relu)
    assert oracle.activation(np.array([0.0]), oracle.ACT_SILU)[0] == 0.0
    # silu(-v) = silu(v) - v
    np.testing.assert_allclose(oracle.activation(-v, oracle.ACT_SILU), silu - v, rtol=0, atol=1e-12)
    np.testing.assert_allclose(silu, F.silu(torch.from_numpy(v)).numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_array_equal(oracle.activation(v, oracle.ACT_NONE), v)


@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_RELU, oracle.ACT_SILU])
def test_residual_modes(act):
    rng = np.random.default_rng(9 + act)
    x = _rand(rng, 1, 4, 6, 6)
    wt = _rand(rng, 4, 4, 3, 3)
    bn = wl.draw_bn(rng, 4)
    r = _rand(rng, 1, 4, 6, 6)
    args = (x, wt, bn["gamma"], bn["beta"], bn["mean"], bn["var"], 1e-5, 1, 1, 1, act)
    plain = oracle.conv_bn_act(*args)
    z = oracle.conv_bn_act(*args[:-1], oracle.ACT_NONE)
    before = oracle.conv_bn_act(*args, oracle.RES_BEFORE_ACT, r)
    after = oracle.conv_bn_act(*args, oracle.RES_AFTER_ACT, r)
    np.testing.assert_allclose(before, oracle.activation(z + r, act), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(after, plain + r.astype(np.float64), rtol=1e-13, atol=1e-14)
    zero = np.zeros_like(r)
    np.testing.assert_array_equal(oracle.conv_bn_act(*args, oracle.RES_BEFORE_ACT, zero), plain)
    if act == oracle.ACT_NONE:
        np.testing.assert_allclose(before, after, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- pool / fc
def test_gap_and_fc():
    rng = np.random.default_rng(10)
    x = np.full((2, 3, 7, 7), 0.3, np.float32)
    np.testing.assert_allclose(oracle.gap(x), np.float32(0.3), rtol=1e-14)
    x = _rand(rng, 2, 5, 7, 7)
    np.testing.assert_allclose(oracle.gap(x), F.adaptive_avg_pool2d(torch.from_numpy(x).double(), 1)
                               .numpy()[:, :, 0, 0], rtol=1e-13)
    v = rng.normal(size=(3, 6))
    w = _rand(rng, 4, 6)
    b = _rand(rng, 4)
    fc = oracle.fc(v, w, b)
    as_conv = oracle.conv2d(v.reshape(3, 6, 1, 1), w.reshape(4, 6, 1, 1), 1, 0, 1)[:, :, 0, 0]
    np.testing.assert_allclose(fc, as_conv + b.astype(np.float64), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(fc, F.linear(torch.from_numpy(v), torch.from_numpy(w).double(),
                                            torch.from_numpy(b).double()).numpy(), rtol=1e-13)


# ----------------------------------------------------------------------------- prologue
MEAN = (0.485, 0.456, 0.406)
STD = (0.229, 0.224, 0.225)


def _normalise(v, mean, std):
    m = np.asarray(mean)[None, :, None, None]
    s = np.asarray(std)[None, :, None, None]
    return (v / 255.0 - m) / s


def test_preprocess_same_size_is_normalise_and_transpose():
    src = wl.frame(11, 2, 5, 7)
    got = oracle.preprocess(src, 5, 7, MEAN, STD)
    ref = _normalise(src.transpose(0, 3, 1, 2).astype(np.float64), MEAN, STD)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-14)


def test_preprocess_half_size_is_box_mean():
    src = wl.frame(12, 1, 720, 1280)
    got = oracle.preprocess(src, 360, 640, (0, 0, 0), (1, 1, 1))
    f = src.astype(np.float64).transpose(0, 3, 1, 2)
    box = 0.25 * (f[:, :, 0::2, 0::2] + f[:, :, 0::2, 1::2] + f[:, :, 1::2, 0::2] + f[:, :, 1::2, 1::2])
    np.testing.assert_allclose(got, box / 255.0, rtol=1e-14, atol=1e-15)


def test_preprocess_constant_image():
    src = np.full((1, 9, 13, 3), 200, np.uint8)
    src[..., 1] = 17
    got = oracle.preprocess(src, 6, 20, MEAN, STD)
    for c, v in enumerate((200, 17, 200)):
        np.testing.assert_allclose(got[0, c], (v / 255.0 - MEAN[c]) / STD[c], rtol=1e-14)


@pytest.mark.parametrize("dst", [(640, 640), (480, 640), (37, 53), (900, 1500), (11, 7)])
def test_preprocess_matches_torch_bilinear(dst):
    src = wl.frame(13, 1, 72 if dst[0] < 100 else 720, 128 if dst[0] < 100 else 1280)
    if dst == (900, 1500):
        src = wl.frame(14, 1, 45, 70)
    got = oracle.preprocess(src, dst[0], dst[1], MEAN, STD)
    t = torch.from_numpy(src.transpose(0, 3, 1, 2).astype(np.float64))
    ref = F.interpolate(t, size=dst, mode="bilinear", align_corners=False, antialias=False).numpy()
    np.testing.assert_allclose(got, _normalise(ref, MEAN, STD), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- whole network
def _bn(t, p):
    return F.batch_norm(t, torch.from_numpy(p["mean"]).double(), torch.from_numpy(p["var"]).double(),
                        torch.from_numpy(p["gamma"]).double(), torch.from_numpy(p["beta"]).double(),
                        training=False, eps=1e-5)


def _conv(t, p, stride, pad, groups):
    return F.conv2d(t, torch.from_numpy(p["w"]).double(), stride=stride, padding=pad, groups=groups)


def _mnist_reference(wk):
    """torch float64 forward written from the page's class structure, reading
    weights by layer name (not by the layer list's wiring)."""
    by = {L.name: L.params for L in wk.layers}
    t = torch.from_numpy(wk.x).double()
    t = F.relu(_bn(_conv(t, by["conv1"], 1, 1, 1), by["conv1"]))
    for bi, (cin, cout, s) in enumerate([(48, 96, 2), (96, 96, 1), (96, 192, 2), (192, 192, 1)]):
        identity = t
        h = F.relu(_bn(_conv(t, by[f"b{bi}.dw"], s, 1, cin), by[f"b{bi}.dw"]))
        h = _bn(_conv(h, by[f"b{bi}.pw"], 1, 0, 1), by[f"b{bi}.pw"])
        if s != 1 or cin != cout:
            identity = _bn(_conv(identity, by[f"b{bi}.skip"], s, 0, 1), by[f"b{bi}.skip"])
        t = F.relu(h + identity)
    t = F.adaptive_avg_pool2d(t, 1).flatten(1)
    return F.linear(t, torch.from_numpy(by["fc"]["w"]).double(), torch.from_numpy(by["fc"]["b"]).double())


def test_mnist_forward_matches_page_structure():
    wk = wl.mnist_cnn(3)
    got = oracle.forward(wk.layers, wk.x)[:, :, 0, 0]
    np.testing.assert_allclose(got, _mnist_reference(wk).numpy(), rtol=1e-11, atol=1e-12)


def test_detector_chain_matches_torch():
    """The stem + bridge + sweep chain on a reduced frame, against torch float64."""
    wk = wl.detector_pipeline(1)
    src = wl.frame(15, 1, 144, 256)
    outs = oracle.forward(wk.layers[:1], src, keep_all=True)
    t = torch.from_numpy(src.transpose(0, 3, 1, 2).astype(np.float64))
    ref = F.interpolate(t, size=(640, 640), mode="bilinear", align_corners=False)
    ref = _normalise(ref.numpy(), wk.layers[0].pre_mean, wk.layers[0].pre_std)
    np.testing.assert_allclose(outs[0], ref, rtol=1e-12, atol=1e-12)
    # the conv part on a smaller map, layer by layer through the oracle's walker
    x = np.random.default_rng(16).uniform(0, 1, (1, 3, 96, 96)).astype(np.float32)
    layers = wk.layers[1:]
    for L in layers:
        L.inp -= 1
        if L.res >= 0:
            L.res -= 1
    got = oracle.forward(layers, x)
    t = torch.from_numpy(x).double()
    for L in layers:
        z = _bn(_conv(t, L.params, L.stride, L.pad, L.groups), L.params)
        t = F.silu(z) + (t if L.res_mode == oracle.RES_AFTER_ACT else 0.0)
    np.testing.assert_allclose(got, t.numpy(), rtol=1e-11, atol=1e-11)


# ----------------------------------------------------------------------------- page figures
def test_mnist_param_count_matches_page():
    wk = wl.mnist_cnn(1)
    trainable = 0
    running = 0
    for L in wk.layers:
        if L.kind == wl.KIND_CONV:
            trainable += L.params["w"].size + L.params["gamma"].size + L.params["beta"].size
            running += L.params["mean"].size + L.params["var"].size
        elif L.kind == wl.KIND_FC:
            trainable += L.params["w"].size + L.params["b"].size
    assert trainable == 101_098
    assert (trainable + running) // 1000 == GOLDEN["mnist_param_count_thousands"]["value"]


def test_depthwise_intensity_matches_page():
    wk = wl.mnist_cnn(1)
    rows = accounting.layer_counts(wk.layers, wk.x.shape)
    shapes = [(1, 1, 28, 28)] + [r["out_shape"] for r in rows]
    ais = []
    for i, L in enumerate(wk.layers):
        if L.kind == wl.KIND_CONV and L.groups > 1:
            n, c, h, w = shapes[L.inp + 1]
            ais.append(accounting.conv_count(n, c, h, w, L.cout, L.k, L.stride, L.pad, L.groups,
                                             with_scale_bias=False).ai)
    g = GOLDEN["depthwise_arithmetic_intensity"]
    assert len(ais) == 4
    assert round(min(ais), 2) == g["lo"]
    assert round(max(ais), 1) == g["hi"]


def test_flop_count_is_near_page_figure():
    """The page's 16.9 M FLOPs per pass is parity unpinned; our 2*MAC count is 15.90 M."""
    wk = wl.mnist_cnn(1)
    rows = accounting.layer_counts(wk.layers, wk.x.shape)
    conv_fc = sum(r["flop"] for L, r in zip(wk.layers, rows) if L.kind in (wl.KIND_CONV, wl.KIND_FC))
    assert abs(conv_fc / 1e6 - 15.90) < 0.01
    assert abs(conv_fc / 1e6 - GOLDEN["flops_per_pass_millions"]["value"]) / 16.9 < 0.07


def test_preprocess_ledger_matches_page():
    g = GOLDEN["preprocess_ledger"]
    args = (1, g["src_h"], g["src_w"], g["dst_h"], g["dst_w"])
    fused = accounting.preprocess_bytes(*args)
    passes = accounting.preprocess_three_pass_bytes(*args)
    assert round(fused / 1e6, 2) == g["fused_mb"]
    assert round(sum(passes) / 1e6, 2) == g["three_pass_mb"]
    assert [round(p / 1e6, 2) for p in passes] == [g["three_pass_lines_mb"][k]
                                                 for k in ("resize", "normalize", "layout")]
    assert round(sum(passes) / (g["three_pass_mean_us"] * 1e-6) / 1e9, 3) == g["three_pass_gbps"]
    assert round(fused / (g["fused_mean_us"] * 1e-6) / 1e9, 3) == g["fused_gbps"]
    assert round(sum(passes) / fused, 2) == g["predicted_ratio"]


def test_edge_overflow_rule():
    g = GOLDEN["tma_edge_overflow"]
    for ow, cols in g["cases"]:
        assert g["block_ow"] - ow % g["block_ow"] == cols
        # a correctly sized row stride (multiple of the tile width) leaves no overrun
        stride = -(-ow // g["block_ow"]) * g["block_ow"]
        assert stride - ow == cols and stride % g["block_ow"] == 0
