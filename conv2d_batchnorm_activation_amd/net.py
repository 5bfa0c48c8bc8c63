"""Device-resident layer lists for ``cvx_forward``.

``Net`` uploads a layer list's parameters once (weights, BatchNorm statistics),
folds every BatchNorm with ``cvx_fold_bn`` on the GPU, and keeps the
``cvx_layer`` array, the workspace and the output buffer, so one forward is a
single ``cvx_forward`` call on the caller's stream.

A layer list is a sequence of objects with the attributes kind, inp, res, cin,
cout, k, stride, pad, groups, act, res_mode, params (numpy arrays ``w``,
``gamma``, ``beta``, ``mean``, ``var`` for convolutions; ``w``, ``b`` for fc),
and dst_h, dst_w, pre_mean, pre_std for the prologue.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import cvx

EPS = 1e-5
_F3 = ctypes.c_float * 3


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class Net:
    def __init__(self, layers: Sequence, input_shape: Sequence[int], device="cuda", eps: float = EPS,
                 w_layout: int = 1):
        self.device = torch.device(device)
        self.keep: List[torch.Tensor] = []
        self.input_shape = tuple(input_shape)
        shapes: List[tuple] = []
        cl: List[cvx.cvx_layer] = []
        self.descs: List[Optional[cvx.cvx_conv_desc]] = []
        self.layer_io: List[tuple] = []

        def shape_of(i):
            return self.input_shape if i == cvx.CVX_INPUT else shapes[i]

        for L in layers:
            s_in = shape_of(L.inp)
            lay = cvx.cvx_layer()
            lay.kind = L.kind
            lay.in_ = L.inp
            lay.res = L.res if L.res_mode != 0 else cvx.CVX_NO_RES
            if L.kind == cvx.CVX_L_PREPROC:
                n, h, w, _ = s_in
                lay.conv = cvx.cvx_conv_desc(n, 3, h, w, 3, 1, 1, 1, 0, 1, 0, 0)
                lay.dst_h, lay.dst_w = L.dst_h, L.dst_w
                lay.mean = _F3(*L.pre_mean)
                lay.std = _F3(*L.pre_std)
                out = (n, 3, L.dst_h, L.dst_w)
                self.descs.append(None)
            elif L.kind == cvx.CVX_L_CONV:
                n, c, h, w = s_in
                d = cvx.make_desc(n, c, h, w, L.cout, L.k, L.stride, L.pad, L.groups, L.act,
                                  L.res_mode, w_layout)
                oh, ow = cvx.cvx_conv_out_shape(d)
                p = L.params
                wt = _dev(p["w"], self.device)
                if w_layout == cvx.CVX_W_PACKED:
                    wpk = torch.empty(cvx.cvx_packed_weights_bytes(d) // 4, dtype=torch.float32,
                                      device=self.device)
                    cvx.cvx_pack_weights(d, wt, wpk)
                    self.keep.append(wt)
                    wt = wpk
                g, b, m, v = (_dev(p[k], self.device) for k in ("gamma", "beta", "mean", "var"))
                scale = torch.empty(L.cout, dtype=torch.float32, device=self.device)
                bias = torch.empty_like(scale)
                cvx.cvx_fold_bn(g, b, m, v, eps, scale, bias)
                self.keep += [wt, scale, bias]
                lay.conv = d
                lay.w, lay.scale, lay.bias = wt.data_ptr(), scale.data_ptr(), bias.data_ptr()
                out = (n, L.cout, oh, ow)
                self.descs.append(d)
            elif L.kind == cvx.CVX_L_GAP:
                n, c, h, w = s_in
                lay.conv = cvx.cvx_conv_desc(n, c, h, w, c, 1, 1, 1, 0, 1, 0, 0)
                out = (n, c, 1, 1)
                self.descs.append(None)
            elif L.kind == cvx.CVX_L_FC:
                n, c = s_in[:2]
                wt = _dev(L.params["w"], self.device)
                bb = _dev(L.params["b"], self.device)
                self.keep += [wt, bb]
                lay.conv = cvx.cvx_conv_desc(n, c, 1, 1, L.cout, 1, 1, 1, 0, 1, 0, 0)
                lay.w, lay.bias = wt.data_ptr(), bb.data_ptr()
                out = (n, L.cout, 1, 1)
                self.descs.append(None)
            else:
                raise ValueError(f"unknown layer kind {L.kind}")
            shapes.append(out)
            self.layer_io.append((s_in, out))
            cl.append(lay)
        self.layers = cl
        self.arr = cvx.layer_array(cl)
        self.out_shape = cvx.cvx_forward_out_shape(self.arr)
        self.ws_bytes = cvx.cvx_forward_workspace_bytes(self.arr)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        self.output = torch.empty(self.out_shape, dtype=torch.float32, device=self.device)

    def __call__(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        o = self.output if out is None else out
        cvx.cvx_forward(self.arr, x, o, self.workspace, self.ws_bytes, stream=stream)
        return o
