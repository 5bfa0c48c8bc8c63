"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module holds inputs and network structure only: random arrays drawn in a
fixed order from ``numpy.random.default_rng(seed)`` and layer lists that say
which layer feeds which.  It contains none of the method's arithmetic (no
convolution, normalisation, activation, resize or shape arithmetic), so the
CPU oracle and the HIP library can both consume it without sharing code.

The workloads stand in for data the source pages used but did not publish:
MNIST digits ("Как я свертки ускорял", "Пациента на стол"), COCO frames
("YOLO26N Inference Optimisation", "mAP caveat") and camera frames
("A fused Ampere preprocess kernel", "The setup").  Convolution run time does
not depend on the values, so uniform random inputs of the same shapes serve.

Recipe (seed = 1000 + workload index unless a test passes its own):
  activations     fp32, U(-1, 1) for the single depthwise layer, U(0, 1) elsewhere
  frames          u8, uniform over 0..255, HWC RGB
  conv weights    fp32, N(0, 1/fan_in) i.e. std = 1/sqrt((cin/groups)*kh*kw)
  BN parameters   gamma U(0.5, 1.5), beta U(-0.1, 0.1), mean U(-0.1, 0.1),
                  var U(0.5, 1.5), eps 1e-5
  fc              weight N(0, 1/192), bias U(-0.1, 0.1)
  draw order      input first, then per layer: weight, gamma, beta, mean, var
                  (fc: weight, bias)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

EPS = 1e-5

ACT_NONE, ACT_RELU, ACT_SILU = 0, 1, 2
RES_NONE, RES_BEFORE_ACT, RES_AFTER_ACT = 0, 1, 2

KIND_CONV, KIND_GAP, KIND_FC, KIND_PREPROC = 0, 1, 2, 3

#: index meaning "the network input" in ``Layer.inp`` / ``Layer.res``
NET_INPUT = -1
#: index meaning "no residual" in ``Layer.res``
NO_RES = -2

#: per-channel normalisation used for the stem prologue (a common convention,
#: not given by the pages: the caller supplies mean/std)
PRE_MEAN = (0.485, 0.456, 0.406)
PRE_STD = (0.229, 0.224, 0.225)


@dataclass
class Layer:
    """One node of a layer list.  ``inp``/``res`` index earlier layers."""

    kind: int
    inp: int = NET_INPUT
    res: int = NO_RES
    cin: int = 0
    cout: int = 0
    k: int = 1
    stride: int = 1
    pad: int = 0
    groups: int = 1
    act: int = ACT_NONE
    res_mode: int = RES_NONE
    name: str = ""
    params: Dict[str, np.ndarray] = field(default_factory=dict)
    # prologue only
    dst_h: int = 0
    dst_w: int = 0
    pre_mean: Tuple[float, float, float] = PRE_MEAN
    pre_std: Tuple[float, float, float] = PRE_STD


@dataclass
class Workload:
    name: str
    x: np.ndarray                 # fp32 NCHW, or u8 NHWC when the first layer is the prologue
    layers: List[Layer]


def rng_for(index: int) -> np.random.Generator:
    return np.random.default_rng(1000 + index)


def draw_bn(rng: np.random.Generator, c: int) -> Dict[str, np.ndarray]:
    f = np.float32
    return {
        "gamma": rng.uniform(0.5, 1.5, c).astype(f),
        "beta": rng.uniform(-0.1, 0.1, c).astype(f),
        "mean": rng.uniform(-0.1, 0.1, c).astype(f),
        "var": rng.uniform(0.5, 1.5, c).astype(f),
    }


def conv_layer(rng: np.random.Generator, cin: int, cout: int, k: int, stride: int, pad: int,
               groups: int = 1, act: int = ACT_RELU, res_mode: int = RES_NONE,
               inp: int = NET_INPUT, res: int = NO_RES, name: str = "") -> Layer:
    fan_in = (cin // groups) * k * k
    w = rng.normal(0.0, 1.0 / np.sqrt(fan_in), (cout, cin // groups, k, k)).astype(np.float32)
    p = {"w": w}
    p.update(draw_bn(rng, cout))
    return Layer(KIND_CONV, inp=inp, res=res, cin=cin, cout=cout, k=k, stride=stride, pad=pad,
                 groups=groups, act=act, res_mode=res_mode, name=name, params=p)


# --------------------------------------------------------------------------- configs
def depthwise_single(seed_index: int = 0) -> Workload:
    """Single depthwise 3x3 s1 p1 layer on [1,48,28,28], BN folded, ReLU."""
    rng = rng_for(seed_index)
    x = rng.uniform(-1.0, 1.0, (1, 48, 28, 28)).astype(np.float32)
    layer = conv_layer(rng, 48, 48, 3, 1, 1, groups=48, act=ACT_RELU, name="dw48")
    return Workload("dw3x3_48x28x28", x, [layer])


def mnist_cnn(batch: int, seed_index: int = 1) -> Workload:
    """The depthwise-separable MNIST CNN ("Как я свертки ускорял", "Пациента на стол").

    conv1 3x3 1->48 + BN + ReLU; four blocks (48->96 s2, 96->96, 96->192 s2,
    192->192), each dw3x3 + BN + ReLU -> pw1x1 + BN, plus a shortcut (1x1
    stride-s conv + BN when the block changes stride or width, else identity),
    added before the block's final ReLU; global average pool; fc 192->10.
    """
    rng = rng_for(seed_index)
    x = rng.uniform(0.0, 1.0, (batch, 1, 28, 28)).astype(np.float32)
    L: List[Layer] = [conv_layer(rng, 1, 48, 3, 1, 1, act=ACT_RELU, name="conv1")]
    for bi, (cin, cout, s) in enumerate([(48, 96, 2), (96, 96, 1), (96, 192, 2), (192, 192, 1)]):
        block_in = len(L) - 1
        L.append(conv_layer(rng, cin, cin, 3, s, 1, groups=cin, act=ACT_RELU,
                            inp=block_in, name=f"b{bi}.dw"))
        dw_idx = len(L) - 1
        if s != 1 or cin != cout:
            L.append(conv_layer(rng, cin, cout, 1, s, 0, act=ACT_NONE, inp=block_in,
                                name=f"b{bi}.skip"))
            short = len(L) - 1
        else:
            short = block_in
        L.append(conv_layer(rng, cin, cout, 1, 1, 0, act=ACT_RELU, res_mode=RES_BEFORE_ACT,
                            inp=dw_idx, res=short, name=f"b{bi}.pw"))
    last = len(L) - 1
    L.append(Layer(KIND_GAP, inp=last, cin=192, cout=192, name="gap"))
    fc_w = rng.normal(0.0, 1.0 / np.sqrt(192), (10, 192)).astype(np.float32)
    fc_b = rng.uniform(-0.1, 0.1, 10).astype(np.float32)
    L.append(Layer(KIND_FC, inp=len(L) - 1, cin=192, cout=10, name="fc",
                   params={"w": fc_w, "b": fc_b}))
    return Workload(f"mnist_dwsep_b{batch}", x, L)


def shortcut_block(batch: int, cin: int, hw: int, cout: int, stride: int, act: int,
                   seed_index: int = 7) -> Workload:
    """One block with a projection shortcut, between two 1x1 layers.

    1x1 cin->cin + BN + ReLU; dw3x3 stride s + BN + ReLU; 1x1 stride-s cin->cout
    shortcut + BN (no activation) of the same input; pw1x1 cin->cout + BN, the
    shortcut added before `act`; then 1x1 cout->cout + BN (no activation), so
    the block's output is compared through a full-rank channel mix.
    """
    rng = rng_for(seed_index)
    x = rng.uniform(-1.0, 1.0, (batch, cin, hw, hw)).astype(np.float32)
    L: List[Layer] = [conv_layer(rng, cin, cin, 1, 1, 0, act=ACT_RELU, name="in1x1")]
    L.append(conv_layer(rng, cin, cin, 3, stride, 1, groups=cin, act=ACT_RELU, inp=0, name="dw"))
    L.append(conv_layer(rng, cin, cout, 1, stride, 0, act=ACT_NONE, inp=0, name="skip"))
    L.append(conv_layer(rng, cin, cout, 1, 1, 0, act=act, res_mode=RES_BEFORE_ACT, inp=1, res=2,
                        name="pw"))
    L.append(conv_layer(rng, cout, cout, 1, 1, 0, act=ACT_NONE, inp=3, name="out1x1"))
    return Workload(f"shortcut_block_b{batch}_{cin}x{hw}_{cout}_s{stride}", x, L)


def dw_block(batch: int, cin: int, hw: int, cout: int, stride: int, dw_act: int, residual: bool,
             seed_index: int = 8) -> Workload:
    """A depthwise-separable block without a projection shortcut, between two 1x1 layers.

    1x1 cin->cin + BN + ReLU; dw3x3 stride s + BN + dw_act; pw1x1 cin->cout +
    BN + ReLU, with the block input added before the ReLU when `residual`
    (stride 1, cin == cout); then 1x1 cout->cout + BN (no activation).
    """
    rng = rng_for(seed_index)
    x = rng.uniform(-1.0, 1.0, (batch, cin, hw, hw)).astype(np.float32)
    L: List[Layer] = [conv_layer(rng, cin, cin, 1, 1, 0, act=ACT_RELU, name="in1x1")]
    L.append(conv_layer(rng, cin, cin, 3, stride, 1, groups=cin, act=dw_act, inp=0, name="dw"))
    if residual:
        L.append(conv_layer(rng, cin, cout, 1, 1, 0, act=ACT_RELU, res_mode=RES_BEFORE_ACT, inp=1, res=0,
                            name="pw"))
    else:
        L.append(conv_layer(rng, cin, cout, 1, 1, 0, act=ACT_RELU, inp=1, name="pw"))
    L.append(conv_layer(rng, cout, cout, 1, 1, 0, act=ACT_NONE, inp=2, name="out1x1"))
    return Workload(f"dw_block_b{batch}_{cin}x{hw}_{cout}_s{stride}", x, L)


def _stem_layers(rng: np.random.Generator, first_inp: int) -> List[Layer]:
    return [
        conv_layer(rng, 3, 16, 3, 2, 1, act=ACT_SILU, inp=first_inp, name="stem1"),
        conv_layer(rng, 16, 32, 3, 2, 1, act=ACT_SILU, inp=first_inp + 1, name="stem2"),
    ]


def detector_stem(seed_index: int = 2) -> Workload:
    """[1,3,640,640] -> 3x3 s2 3->16 +BN+SiLU -> 3x3 s2 16->32 +BN+SiLU."""
    rng = rng_for(seed_index)
    x = rng.uniform(0.0, 1.0, (1, 3, 640, 640)).astype(np.float32)
    return Workload("stem_640", x, _stem_layers(rng, NET_INPUT))


#: the per-layer sweep of nano-detector shapes:
#: (name, cin, h=w, cout, k, stride, groups, residual?)
SWEEP = [
    ("a_64x80_3x3", 64, 80, 64, 3, 1, 1, True),
    ("b_64x80_3x3s2", 64, 80, 128, 3, 2, 1, False),
    ("c_128x40_1x1", 128, 40, 128, 1, 1, 1, True),
    ("d_128x40_3x3", 128, 40, 128, 3, 1, 1, True),
    ("e_128x40_3x3s2", 128, 40, 256, 3, 2, 1, False),
    ("f_256x20_1x1", 256, 20, 256, 1, 1, 1, True),
    ("g_256x20_3x3", 256, 20, 256, 3, 1, 1, True),
    ("h_64x13_dw3x3", 64, 13, 64, 3, 1, 64, True),
]


def sweep_layer(name: str, seed_index: int = 3, batch: int = 1) -> Workload:
    """One layer of the sweep, alone: x U(0,1), SiLU, residual = the layer's own input
    on the stride-1 equal-width layers (added after the activation)."""
    names = [s[0] for s in SWEEP]
    i = names.index(name)
    rng = np.random.default_rng(1000 + seed_index + 100 * (i + 1))
    _, cin, hw, cout, k, s, g, has_res = SWEEP[i]
    x = rng.uniform(0.0, 1.0, (batch, cin, hw, hw)).astype(np.float32)
    layer = conv_layer(rng, cin, cout, k, s, k // 2, groups=g, act=ACT_SILU,
                       res_mode=RES_AFTER_ACT if has_res else RES_NONE,
                       res=NET_INPUT if has_res else NO_RES, name=name)
    return Workload(f"sweep_{name}", x, [layer])


def detector_pipeline(batch: int, seed_index: int = 4) -> Workload:
    """u8 frame [N,720,1280,3] -> fused resize/normalise/CHW to [N,3,640,640] ->
    stem (3->16 s2, 16->32 s2) -> bridge 3x3 s2 32->64 -> sweep layers a..g in order,
    each stride-1 equal-width layer adding its own input after the SiLU."""
    rng = rng_for(seed_index)
    x = rng.integers(0, 256, (batch, 720, 1280, 3), dtype=np.uint8)
    L: List[Layer] = [Layer(KIND_PREPROC, inp=NET_INPUT, cin=3, cout=3, name="preprocess",
                            dst_h=640, dst_w=640)]
    L += _stem_layers(rng, 0)
    L.append(conv_layer(rng, 32, 64, 3, 2, 1, act=ACT_SILU, inp=len(L) - 1, name="bridge"))
    for (name, cin, hw, cout, k, s, g, has_res) in SWEEP[:7]:
        prev = len(L) - 1
        L.append(conv_layer(rng, cin, cout, k, s, k // 2, groups=g, act=ACT_SILU,
                            res_mode=RES_AFTER_ACT if has_res else RES_NONE,
                            inp=prev, res=prev if has_res else NO_RES, name=name))
    return Workload(f"detector_640_b{batch}", x, L)


def dense_chain(batch: int, hw: int = 48, seed_index: int = 10) -> Workload:
    """Eight dense 1x1/3x3 layers in a row (the shapes a chain launch runs),
    with ragged channel counts (24, 40, 96), ragged tiles (hw/2 and hw/4 wide
    maps), residuals from the list input, from the layer's own input and from
    two layers back, added before or after the activation:

      0 3x3 s1 24->24 SiLU  + input (after)      4 3x3 s1 64->64 SiLU  + out 2 (before)
      1 3x3 s1 24->40 SiLU                       5 3x3 s2 64->96 SiLU
      2 3x3 s2 40->64 ReLU                       6 1x1 s1 96->96 ReLU  + out 5 (before)
      3 1x1 s1 64->64 SiLU  + out 2 (after)      7 3x3 s1 96->96 none  + out 5 (after)
    """
    rng = rng_for(seed_index)
    x = rng.uniform(-1.0, 1.0, (batch, 24, hw, hw)).astype(np.float32)
    S, R = ACT_SILU, ACT_RELU
    spec = [  # (cin, cout, k, stride, act, res_mode, inp, res)
        (24, 24, 3, 1, S, RES_AFTER_ACT, NET_INPUT, NET_INPUT),
        (24, 40, 3, 1, S, RES_NONE, 0, NO_RES),
        (40, 64, 3, 2, R, RES_NONE, 1, NO_RES),
        (64, 64, 1, 1, S, RES_AFTER_ACT, 2, 2),
        (64, 64, 3, 1, S, RES_BEFORE_ACT, 3, 2),
        (64, 96, 3, 2, S, RES_NONE, 4, NO_RES),
        (96, 96, 1, 1, R, RES_BEFORE_ACT, 5, 5),
        (96, 96, 3, 1, ACT_NONE, RES_AFTER_ACT, 6, 5),
    ]
    L: List[Layer] = []
    for i, (cin, cout, k, st, act, rm, inp, res) in enumerate(spec):
        L.append(conv_layer(rng, cin, cout, k, st, k // 2, act=act, res_mode=rm, inp=inp, res=res,
                            name=f"d{i}"))
    return Workload(f"dense_chain_b{batch}_{hw}", x, L)


def prologue_stem(batch: int, src_h: int, src_w: int, dst_h: int, dst_w: int, cout: int,
                  stride: int, act: int, tail: bool = False, seed_index: int = 9) -> Workload:
    """u8 frames [N,src_h,src_w,3] -> resize/normalise to [N,3,dst_h,dst_w] ->
    3x3 pad-1 conv 3->cout (stride 1 or 2) +BN+act, optionally followed by a
    3x3 stride-1 conv cout->cout (so that the first convolution's output is an
    intermediate rather than the list's output)."""
    rng = rng_for(seed_index)
    x = rng.integers(0, 256, (batch, src_h, src_w, 3), dtype=np.uint8)
    L: List[Layer] = [Layer(KIND_PREPROC, inp=NET_INPUT, cin=3, cout=3, name="preprocess",
                            dst_h=dst_h, dst_w=dst_w)]
    L.append(conv_layer(rng, 3, cout, 3, stride, 1, act=act, inp=0, name="stem"))
    if tail:
        L.append(conv_layer(rng, cout, cout, 3, 1, 1, act=act, inp=1, name="tail"))
    return Workload(f"prologue_{src_h}x{src_w}_{dst_h}x{dst_w}_s{stride}_b{batch}", x, L)


def prologue_stem_pair(seed: int, n: int, src_h: int, src_w: int, dst_h: int, dst_w: int, s1: int,
                       s2: int, cout: int) -> Workload:
    """u8 frames [N,src_h,src_w,3] -> resize/normalise to [N,3,dst_h,dst_w] ->
    stem 3x3 3->16 (stride s1) +BN+SiLU -> 3x3 16->cout (stride s2) +BN+SiLU."""
    rng = np.random.default_rng(1000 + seed)
    x = rng.integers(0, 256, (n, src_h, src_w, 3), dtype=np.uint8)
    L: List[Layer] = [Layer(KIND_PREPROC, inp=NET_INPUT, cin=3, cout=3, name="preprocess",
                            dst_h=dst_h, dst_w=dst_w)]
    L.append(conv_layer(rng, 3, 16, 3, s1, 1, act=ACT_SILU, inp=0, name="stem1"))
    L.append(conv_layer(rng, 16, cout, 3, s2, 1, act=ACT_SILU, inp=1, name="stem2"))
    return Workload(f"prologue_pair_{seed}", x, L)


def stem_pair_case(seed: int, n: int, cin: int, h: int, w: int, s1: int, s2: int, cout: int,
                   act1: int = ACT_SILU, act2: int = ACT_SILU, res_mode: int = RES_NONE) -> Workload:
    """A stem layer (3x3 pad 1, cin -> 16, stride s1) and the 3x3 pad-1 layer
    16 -> cout (stride s2) that alone reads it; with a residual, a 1x1 layer of
    stride s1*s2 on the input provides it (layer 0), the stem is layer 1."""
    rng = np.random.default_rng(1000 + seed)
    x = rng.uniform(0.0, 1.0, (n, cin, h, w)).astype(np.float32)
    L: List[Layer] = []
    if res_mode != RES_NONE:
        L.append(conv_layer(rng, cin, cout, 1, s1 * s2, 0, act=ACT_NONE, name="res_src"))
    first = len(L)
    L.append(conv_layer(rng, cin, 16, 3, s1, 1, act=act1, inp=NET_INPUT, name="stem1"))
    L.append(conv_layer(rng, 16, cout, 3, s2, 1, act=act2, inp=first, res_mode=res_mode,
                        res=0 if res_mode != RES_NONE else NO_RES, name="stem2"))
    return Workload(f"stem_pair_{seed}", x, L)


def random_conv_case(seed: int, n: int, cin: int, h: int, w: int, cout: int, k: int,
                     stride: int, pad: int, groups: int = 1, act: int = ACT_SILU,
                     res_mode: int = RES_NONE, x_lo: float = -1.0) -> Tuple[np.ndarray, Layer]:
    """A single-layer case for parity sweeps: x ~ U(x_lo, 1) of shape [n,cin,h,w]
    and one seeded conv layer.  A residual, when the case has one, is drawn
    separately by ``residual_for`` once the caller knows the output's shape."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(x_lo, 1.0, (n, cin, h, w)).astype(np.float32)
    layer = conv_layer(rng, cin, cout, k, stride, pad, groups=groups, act=act, res_mode=res_mode)
    return x, layer


def residual_for(seed: int, shape: Tuple[int, ...]) -> np.ndarray:
    """Independent U(-1,1) residual tensor for a parity case."""
    return np.random.default_rng(seed + 7777).uniform(-1.0, 1.0, shape).astype(np.float32)


def frame(seed: int, n: int, h: int, w: int) -> np.ndarray:
    """u8 HWC RGB frames, uniform over 0..255."""
    return np.random.default_rng(seed).integers(0, 256, (n, h, w, 3), dtype=np.uint8)
