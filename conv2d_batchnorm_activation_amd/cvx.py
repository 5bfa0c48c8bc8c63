"""Thin ctypes binding of libcvx (include/cvx.h): argument marshalling only.

Every function here has the name of the C entry point it wraps and does nothing
but turn tensors into device pointers, pick the caller's current HIP stream and
turn status codes into exceptions.  All computation happens in libcvx's HIP
kernels.  PyTorch provides device memory and streams.

Importing this module raises ImportError when libcvx.so has not been built:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch  # loaded first: the process then has one HIP runtime, torch's

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcvx.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"libcvx.so not found at {_LIB_PATH}: build it with "
        "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
lib = ctypes.CDLL(_LIB_PATH)

CVX_OK = 0
CVX_ACT_NONE, CVX_ACT_RELU, CVX_ACT_SILU = 0, 1, 2
CVX_RES_NONE, CVX_RES_BEFORE_ACT, CVX_RES_AFTER_ACT = 0, 1, 2
CVX_L_CONV, CVX_L_GAP, CVX_L_FC, CVX_L_PREPROC = 0, 1, 2, 3
CVX_INPUT, CVX_NO_RES = -1, -2
CVX_W_OIHW, CVX_W_PACKED = 0, 1
CVX_DT_F32, CVX_DT_F16, CVX_DT_BF16 = 0, 1, 2
STATUS_NAMES = {0: "CVX_OK", -1: "CVX_ERR_NULL", -2: "CVX_ERR_SHAPE", -3: "CVX_ERR_UNSUPPORTED",
                -4: "CVX_ERR_ALIGN", -5: "CVX_ERR_ALIAS", -6: "CVX_ERR_WORKSPACE",
                -7: "CVX_ERR_HIP", -8: "CVX_ERR_ARG", -9: "CVX_ERR_SCRATCH"}


class cvx_conv_desc(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int) for f in
                ("n", "c_in", "h", "w", "c_out", "kh", "kw", "stride", "pad", "groups", "act",
                 "res_mode", "w_layout")]


class cvx_layer(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("in_", ctypes.c_int), ("res", ctypes.c_int),
                ("conv", cvx_conv_desc),
                ("w", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("dst_h", ctypes.c_int), ("dst_w", ctypes.c_int),
                ("mean", ctypes.c_float * 3), ("std", ctypes.c_float * 3)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_DP = ctypes.POINTER(cvx_conv_desc)
_LP = ctypes.POINTER(cvx_layer)

lib.cvx_status_str.argtypes = [_I]
lib.cvx_status_str.restype = ctypes.c_char_p
lib.cvx_version.argtypes = []
lib.cvx_version.restype = ctypes.c_char_p
lib.cvx_conv_out_shape.argtypes = [_DP, ctypes.POINTER(_I), ctypes.POINTER(_I)]
lib.cvx_conv_out_shape.restype = _I
lib.cvx_conv_plan.argtypes = [_DP, ctypes.c_char_p, _I]
lib.cvx_conv_plan.restype = _I
lib.cvx_conv_workspace_bytes.argtypes = [_DP]
lib.cvx_conv_workspace_bytes.restype = _Z
lib.cvx_packed_weights_bytes.argtypes = [_DP]
lib.cvx_packed_weights_bytes.restype = _Z
lib.cvx_pack_weights.argtypes = [_DP, _P, _P, _P]
lib.cvx_pack_weights.restype = _I
lib.cvx_fold_bn.argtypes = [_P, _P, _P, _P, ctypes.c_float, _I, _P, _P, _P]
lib.cvx_fold_bn.restype = _I
lib.cvx_conv_bn_act.argtypes = [_DP, _P, _P, _P, _P, _P, _P, _P, _Z, _P]
lib.cvx_conv_bn_act.restype = _I
lib.cvx_preprocess_u8.argtypes = [_P, _I, _I, _I, ctypes.c_long, _P, _I, _I,
                                  ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float), _P]
lib.cvx_preprocess_u8.restype = _I
lib.cvx_gap_fc.argtypes = [_P, _I, _I, _I, _I, _P, _P, _I, _P, _P]
lib.cvx_gap_fc.restype = _I
lib.cvx_forward_out_shape.argtypes = [_LP, _I, ctypes.POINTER(_I)]
lib.cvx_forward_out_shape.restype = _I
lib.cvx_forward_workspace_bytes.argtypes = [_LP, _I, ctypes.POINTER(_I)]
lib.cvx_forward_workspace_bytes.restype = _Z
lib.cvx_forward_plan.argtypes = [_LP, _I, ctypes.c_char_p, _I]
lib.cvx_forward_plan.restype = _I
lib.cvx_forward.argtypes = [_LP, _I, _P, _P, _P, _Z, _P]
lib.cvx_forward.restype = _I
lib.cvx_nhwc_packed_weights_bytes.argtypes = [_DP, _I]
lib.cvx_nhwc_packed_weights_bytes.restype = _Z
lib.cvx_nhwc_plan.argtypes = [_DP, _I, ctypes.c_char_p, _I]
lib.cvx_nhwc_plan.restype = _I
lib.cvx_nhwc_pack_weights.argtypes = [_DP, _I, _P, _P, _P]
lib.cvx_nhwc_pack_weights.restype = _I
lib.cvx_conv_bn_act_nhwc.argtypes = [_DP, _I, _P, _P, _P, _P, _P, _P, _P]
lib.cvx_conv_bn_act_nhwc.restype = _I
lib.cvx_static_scratch_bytes.argtypes = []
lib.cvx_static_scratch_bytes.restype = _Z
lib.cvx_forward_noalloc.argtypes = [_LP, _I, _P, _P, _P]
lib.cvx_forward_noalloc.restype = _I
lib.cvx_workgroup_xcds.argtypes = [_P, _I, _P]
lib.cvx_workgroup_xcds.restype = _I

#: every entry point include/cvx.h declares
EXPORTS = ("cvx_status_str", "cvx_version", "cvx_conv_out_shape", "cvx_conv_plan",
           "cvx_conv_workspace_bytes", "cvx_packed_weights_bytes", "cvx_pack_weights", "cvx_fold_bn", "cvx_conv_bn_act", "cvx_preprocess_u8",
           "cvx_gap_fc", "cvx_forward_out_shape", "cvx_forward_workspace_bytes", "cvx_forward_plan",
           "cvx_forward", "cvx_nhwc_packed_weights_bytes", "cvx_nhwc_plan", "cvx_nhwc_pack_weights",
           "cvx_conv_bn_act_nhwc", "cvx_static_scratch_bytes", "cvx_forward_noalloc",
           "cvx_workgroup_xcds")


class CvxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({lib.cvx_status_str(status).decode()})")


def _check(st: int, where: str) -> None:
    if st != CVX_OK:
        raise CvxError(st, where)


def _ptr(t) -> Optional[int]:
    """Device (or raw) pointer of a tensor / int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(n, c_in, h, w, c_out, k, stride, pad, groups=1, act=CVX_ACT_NONE,
              res_mode=CVX_RES_NONE, w_layout=CVX_W_OIHW) -> cvx_conv_desc:
    return cvx_conv_desc(n, c_in, h, w, c_out, k, k, stride, pad, groups, act, res_mode, w_layout)


def cvx_status_str(status: int) -> str:
    return lib.cvx_status_str(status).decode()


def cvx_version() -> str:
    return lib.cvx_version().decode()


def cvx_conv_out_shape(desc: cvx_conv_desc):
    oh, ow = _I(), _I()
    _check(lib.cvx_conv_out_shape(ctypes.byref(desc), ctypes.byref(oh), ctypes.byref(ow)),
           "cvx_conv_out_shape")
    return oh.value, ow.value


def cvx_conv_plan(desc: cvx_conv_desc) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib.cvx_conv_plan(ctypes.byref(desc), buf, 256), "cvx_conv_plan")
    return buf.value.decode()


def cvx_conv_workspace_bytes(desc: cvx_conv_desc) -> int:
    return lib.cvx_conv_workspace_bytes(ctypes.byref(desc))


def cvx_packed_weights_bytes(desc: cvx_conv_desc) -> int:
    return lib.cvx_packed_weights_bytes(ctypes.byref(desc))


def cvx_pack_weights(desc: cvx_conv_desc, w_oihw, w_packed, stream=None) -> None:
    _check(lib.cvx_pack_weights(ctypes.byref(desc), _ptr(w_oihw), _ptr(w_packed), _stream(stream)),
           "cvx_pack_weights")


def cvx_fold_bn(gamma, beta, mean, var, eps: float, scale, bias, stream=None) -> None:
    _check(lib.cvx_fold_bn(_ptr(gamma), _ptr(beta), _ptr(mean), _ptr(var), eps, gamma.numel(),
                           _ptr(scale), _ptr(bias), _stream(stream)), "cvx_fold_bn")


def cvx_conv_bn_act(desc: cvx_conv_desc, x, w, scale, bias, residual, y, workspace=None,
                    ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    _check(lib.cvx_conv_bn_act(ctypes.byref(desc), _ptr(x), _ptr(w), _ptr(scale), _ptr(bias),
                               _ptr(residual), _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)),
           "cvx_conv_bn_act")


def cvx_preprocess_u8(src, dst, mean: Sequence[float], std: Sequence[float], stream=None,
                      src_row_bytes: Optional[int] = None) -> None:
    n, src_h, src_w, _ = src.shape
    _, _, dst_h, dst_w = dst.shape
    m = (ctypes.c_float * 3)(*mean)
    s = (ctypes.c_float * 3)(*std)
    rb = 3 * src_w if src_row_bytes is None else src_row_bytes
    _check(lib.cvx_preprocess_u8(_ptr(src), n, src_h, src_w, rb, _ptr(dst), dst_h, dst_w, m, s,
                                 _stream(stream)), "cvx_preprocess_u8")


def cvx_gap_fc(x, fc_w, fc_b, out, stream=None) -> None:
    n, c, h, w = x.shape
    _check(lib.cvx_gap_fc(_ptr(x), n, c, h, w, _ptr(fc_w), _ptr(fc_b), fc_w.shape[0], _ptr(out),
                          _stream(stream)), "cvx_gap_fc")


def layer_array(layers: Sequence[cvx_layer]):
    arr = (cvx_layer * len(layers))(*layers)
    return arr, len(layers)


def cvx_forward_out_shape(layers) -> tuple:
    arr, n = layers if isinstance(layers, tuple) else layer_array(layers)
    out = (_I * 4)()
    _check(lib.cvx_forward_out_shape(arr, n, out), "cvx_forward_out_shape")
    return tuple(out)


def cvx_forward_plan(layers) -> list:
    """Per-layer launch plan of a list: one string per layer (see cvx_forward_plan)."""
    arr, n = layers if isinstance(layers, tuple) else layer_array(layers)
    size = 320 * n + 1
    buf = ctypes.create_string_buffer(size)
    _check(lib.cvx_forward_plan(arr, n, buf, size), "cvx_forward_plan")
    return [line.split(" ", 1)[1] for line in buf.value.decode().split("\n")]


def cvx_forward_workspace_bytes(layers) -> int:
    arr, n = layers if isinstance(layers, tuple) else layer_array(layers)
    st = _I(0)
    b = lib.cvx_forward_workspace_bytes(arr, n, ctypes.byref(st))
    _check(st.value, "cvx_forward_workspace_bytes")
    return b


def cvx_forward(layers, inp, out, workspace, ws_bytes: Optional[int] = None, stream=None) -> None:
    arr, n = layers if isinstance(layers, tuple) else layer_array(layers)
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    _check(lib.cvx_forward(arr, n, _ptr(inp), _ptr(out), _ptr(workspace), ws_bytes,
                           _stream(stream)), "cvx_forward")


def cvx_workgroup_xcds(out, stream=None) -> None:
    """XCD index of each of out.numel() workgroups of one launch (int32 device tensor)."""
    _check(lib.cvx_workgroup_xcds(_ptr(out), out.numel(), _stream(stream)), "cvx_workgroup_xcds")


def cvx_static_scratch_bytes() -> int:
    return lib.cvx_static_scratch_bytes()


def cvx_forward_noalloc(layers, inp, out, stream=None) -> None:
    arr, n = layers if isinstance(layers, tuple) else layer_array(layers)
    _check(lib.cvx_forward_noalloc(arr, n, _ptr(inp), _ptr(out), _stream(stream)),
           "cvx_forward_noalloc")


def cvx_nhwc_packed_weights_bytes(desc: cvx_conv_desc, dtype: int) -> int:
    return lib.cvx_nhwc_packed_weights_bytes(ctypes.byref(desc), dtype)


def cvx_nhwc_plan(desc: cvx_conv_desc, dtype: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib.cvx_nhwc_plan(ctypes.byref(desc), dtype, buf, 256), "cvx_nhwc_plan")
    return buf.value.decode()


def cvx_nhwc_pack_weights(desc: cvx_conv_desc, dtype: int, w_oihw, w_packed, stream=None) -> None:
    _check(lib.cvx_nhwc_pack_weights(ctypes.byref(desc), dtype, _ptr(w_oihw), _ptr(w_packed),
                                     _stream(stream)), "cvx_nhwc_pack_weights")


def cvx_conv_bn_act_nhwc(desc: cvx_conv_desc, dtype: int, x, w_packed, scale, bias, residual, y,
                         stream=None) -> None:
    _check(lib.cvx_conv_bn_act_nhwc(ctypes.byref(desc), dtype, _ptr(x), _ptr(w_packed), _ptr(scale),
                                    _ptr(bias), _ptr(residual), _ptr(y), _stream(stream)),
           "cvx_conv_bn_act_nhwc")
