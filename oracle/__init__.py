"""CPU oracle for the fused convolution + BatchNorm + activation layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package; the product library never
does, and this package imports nothing from the product.

The arithmetic lives in ``cvx_oracle.c`` (plain C, fp64, compiled with gcc);
this module marshals numpy arrays into it and walks layer lists.  All inputs
are the same fp32 arrays the GPU sees, promoted to float64; all results stay
float64.

Parity status of each function (what pins it is in ``tests/test_oracle_pins.py``):
  conv2d, conv_bn_act, fold_bn, activation, gap, fc, preprocess, forward: pinned.
  The FLOP count the MNIST page prints (16.9 M per pass) is parity unpinned: a
  2*MAC count of the transcribed network gives 15.90 M and the page does not say
  how it counted BatchNorm, ReLU and the adds.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cvx_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ACT_NONE, ACT_RELU, ACT_SILU = 0, 1, 2
RES_NONE, RES_BEFORE_ACT, RES_AFTER_ACT = 0, 1, 2
KIND_CONV, KIND_GAP, KIND_FC, KIND_PREPROC = 0, 1, 2, 3
NET_INPUT, NO_RES = -1, -2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no HIP, no shared sources)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib: Optional[ctypes.CDLL] = None


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        L = ctypes.c_long
        lib.oracle_out_extent.argtypes = [I, I, I, I]
        lib.oracle_out_extent.restype = I
        lib.oracle_conv2d.argtypes = [P, I, I, I, I, P, I, I, I, I, I, I, P]
        lib.oracle_conv2d.restype = None
        lib.oracle_conv_bn_act.argtypes = [P, I, I, I, I, P, I, I, I, I, I, I,
                                           P, P, P, P, D, I, I, P, P]
        lib.oracle_conv_bn_act.restype = None
        lib.oracle_fold_bn.argtypes = [P, P, P, P, D, I, P, P]
        lib.oracle_fold_bn.restype = None
        lib.oracle_activation.argtypes = [P, L, I]
        lib.oracle_activation.restype = None
        lib.oracle_gap.argtypes = [P, I, I, I, I, P]
        lib.oracle_gap.restype = None
        lib.oracle_fc.argtypes = [P, I, I, P, P, I, P]
        lib.oracle_fc.restype = None
        lib.oracle_preprocess.argtypes = [P, I, I, I, L, I, I, P, P, P]
        lib.oracle_preprocess.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        _lib = lib
    return _lib


def _d(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().oracle_num_threads()


def out_extent(n: int, k: int, stride: int, pad: int) -> int:
    return _load().oracle_out_extent(n, k, stride, pad)


def conv2d(x, w, stride: int = 1, pad: int = 0, groups: int = 1) -> np.ndarray:
    """Grouped cross-correlation in fp64, NCHW x OIHW -> NCHW."""
    x = _d(x)
    w = _d(w)
    n, cin, h, wd = x.shape
    cout, cin_g, kh, kw = w.shape
    assert cin_g * groups == cin and cout % groups == 0
    oh, ow = out_extent(h, kh, stride, pad), out_extent(wd, kw, stride, pad)
    out = np.zeros((n, cout, oh, ow), np.float64)
    _load().oracle_conv2d(_p(x), n, cin, h, wd, _p(w), cout, kh, kw, stride, pad, groups, _p(out))
    return out


def conv_bn_act(x, w, gamma, beta, mean, var, eps: float, stride: int, pad: int, groups: int,
                act: int, res_mode: int = RES_NONE, residual=None) -> np.ndarray:
    """Convolution, unfolded inference BatchNorm, residual and activation, fp64."""
    x = _d(x)
    w = _d(w)
    n, cin, h, wd = x.shape
    cout, cin_g, kh, kw = w.shape
    assert cin_g * groups == cin and cout % groups == 0
    oh, ow = out_extent(h, kh, stride, pad), out_extent(wd, kw, stride, pad)
    y = np.zeros((n, cout, oh, ow), np.float64)
    g, b, m, v = (_d(a) for a in (gamma, beta, mean, var))
    if res_mode != RES_NONE:
        r = _d(residual)
        assert r.shape == y.shape, (r.shape, y.shape)
        rp = _p(r)
    else:
        r = None
        rp = None
    _load().oracle_conv_bn_act(_p(x), n, cin, h, wd, _p(w), cout, kh, kw, stride, pad, groups,
                               _p(g), _p(b), _p(m), _p(v), float(eps), act, res_mode, rp, _p(y))
    return y


def fold_bn(gamma, beta, mean, var, eps: float):
    g, b, m, v = (_d(a) for a in (gamma, beta, mean, var))
    c = g.shape[0]
    scale = np.zeros(c, np.float64)
    bias = np.zeros(c, np.float64)
    _load().oracle_fold_bn(_p(g), _p(b), _p(m), _p(v), float(eps), c, _p(scale), _p(bias))
    return scale, bias


def activation(v, act: int) -> np.ndarray:
    a = _d(v).copy()
    _load().oracle_activation(_p(a), a.size, act)
    return a


def gap(x) -> np.ndarray:
    x = _d(x)
    n, c, h, w = x.shape
    out = np.zeros((n, c), np.float64)
    _load().oracle_gap(_p(x), n, c, h, w, _p(out))
    return out


def fc(v, w, b) -> np.ndarray:
    v = _d(v)
    w = _d(w)
    b = _d(b)
    n, in_f = v.shape
    out_f = w.shape[0]
    out = np.zeros((n, out_f), np.float64)
    _load().oracle_fc(_p(v), n, in_f, _p(w), _p(b), out_f, _p(out))
    return out


def preprocess(src: np.ndarray, dst_h: int, dst_w: int, mean: Sequence[float],
               std: Sequence[float]) -> np.ndarray:
    """u8 [N,H,W,3] -> f64 [N,3,dst_h,dst_w]: half-pixel bilinear, /255, (v-mean)/std."""
    src = np.ascontiguousarray(src, dtype=np.uint8)
    n, sh, sw, c3 = src.shape
    assert c3 == 3
    out = np.zeros((n, 3, dst_h, dst_w), np.float64)
    m = _d(mean)
    s = _d(std)
    _load().oracle_preprocess(_p(src), n, sh, sw, sw * 3, dst_h, dst_w, _p(m), _p(s), _p(out))
    return out


def run_layer(layer, x: np.ndarray, residual: Optional[np.ndarray]) -> np.ndarray:
    """Apply one layer (a ``workloads.Layer``) to ``x``."""
    if layer.kind == KIND_CONV:
        p = layer.params
        return conv_bn_act(x, p["w"], p["gamma"], p["beta"], p["mean"], p["var"], 1e-5,
                           layer.stride, layer.pad, layer.groups, layer.act, layer.res_mode,
                           residual)
    if layer.kind == KIND_GAP:
        v = gap(x)
        return v.reshape(v.shape[0], v.shape[1], 1, 1)
    if layer.kind == KIND_FC:
        v = _d(x).reshape(x.shape[0], -1)
        o = fc(v, layer.params["w"], layer.params["b"])
        return o.reshape(o.shape[0], o.shape[1], 1, 1)
    if layer.kind == KIND_PREPROC:
        return preprocess(x, layer.dst_h, layer.dst_w, layer.pre_mean, layer.pre_std)
    raise ValueError("unknown layer kind %r" % (layer.kind,))


def forward(layers: List, x: np.ndarray, keep_all: bool = False):
    """Walk an ordered layer list: layer i reads the output of layer ``inp``
    (-1 = network input) and, if it has one, the residual from layer ``res``."""
    outs: List[np.ndarray] = []

    def fetch(i: int) -> np.ndarray:
        return x if i == NET_INPUT else outs[i]

    for layer in layers:
        r = fetch(layer.res) if (layer.kind == KIND_CONV and layer.res_mode != RES_NONE) else None
        outs.append(run_layer(layer, fetch(layer.inp), r))
    return outs if keep_all else outs[-1]


def timed_forward(layers: List, x: np.ndarray, repeats: int = 1) -> Dict[str, float]:
    """Wall-clock seconds of ``forward`` (for the CPU baseline)."""
    t0 = time.perf_counter()
    for _ in range(repeats):
        forward(layers, x)
    return {"seconds": (time.perf_counter() - t0) / repeats, "threads": num_threads()}
