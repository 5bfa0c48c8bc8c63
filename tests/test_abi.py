"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/cvx.h declares, and rejects bad arguments on the host before launching
anything (the error paths return before any HIP call, so they run here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads as wl
from conv2d_batchnorm_activation_amd import cvx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cvx.h")

# fake, never dereferenced device addresses (validation fails before any launch)
X = 0x10000000
W = 0x20000000
S = 0x30000000
B = 0x30001000
Y = 0x40000000
R = 0x50000000
WS = 0x60000000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"CVX_API\s+[\w\s\*]*?\b(cvx_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    decl = declared_functions()
    assert len(decl) >= 12
    assert sorted(cvx.EXPORTS) == decl


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(cvx._LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert "gfx950" in cvx.cvx_version()
    for code in range(-8, 1):
        assert cvx.cvx_status_str(code)
    assert cvx.cvx_status_str(-99) == "unknown status"


def _desc(**kw):
    base = dict(n=1, c_in=64, h=80, w=80, c_out=64, k=3, stride=1, pad=1, groups=1,
                act=cvx.CVX_ACT_SILU, res_mode=cvx.CVX_RES_NONE)
    base.update(kw)
    return cvx.make_desc(**base)


def _call(d, x=X, w=W, s=S, b=B, r=None, y=Y, ws=None, ws_bytes=0):
    return cvx.lib.cvx_conv_bn_act(ctypes.byref(d), x, w, s, b, r, y, ws, ws_bytes, None)


@pytest.mark.parametrize("h,k,s,p,expect", [
    (80, 3, 1, 1, 80), (80, 3, 2, 1, 40), (40, 3, 2, 1, 20), (13, 3, 1, 1, 13), (28, 1, 2, 0, 14),
    (7, 3, 2, 1, 4), (640, 3, 2, 1, 320), (5, 5, 2, 2, 3), (9, 7, 3, 3, 3), (4, 3, 1, 0, 2),
])
def test_out_shape(h, k, s, p, expect):
    assert cvx.cvx_conv_out_shape(_desc(h=h, w=h + 1 if h > 4 else h, k=k, stride=s, pad=p)) == \
        (expect, (h + 1 + 2 * p - k) // s + 1 if h > 4 else expect)


@pytest.mark.parametrize("bad,code", [
    (dict(n=0), -2), (dict(c_in=0), -2), (dict(h=-1), -2), (dict(c_out=0), -2),
    (dict(stride=0), -2), (dict(pad=-1), -2), (dict(groups=0), -2),
    (dict(groups=3), -2),                         # 64 % 3 != 0
    (dict(k=9), -3), (dict(stride=5), -3), (dict(pad=3), -3),
    (dict(h=1, w=1, pad=0), -2),                  # window larger than the image
    (dict(act=3), -8), (dict(res_mode=7), -8), (dict(act=-1), -8), (dict(w_layout=2), -8),
    (dict(n=70000), -2),
    (dict(n=4096, c_in=1024, h=1024, w=1024), -2),  # > 2^31 elements
])
def test_invalid_descriptors_rejected(bad, code):
    d = _desc(**bad)
    oh, ow = ctypes.c_int(), ctypes.c_int()
    assert cvx.lib.cvx_conv_out_shape(ctypes.byref(d), ctypes.byref(oh), ctypes.byref(ow)) == code
    assert _call(d) == code


def test_non_square_kernel_rejected():
    d = _desc()
    d.kw = 1
    assert _call(d) == -3


def test_null_pointers_rejected():
    d = _desc()
    assert cvx.lib.cvx_conv_bn_act(None, X, W, S, B, None, Y, None, 0, None) == -1
    for kw in (dict(x=None), dict(w=None), dict(s=None), dict(b=None), dict(y=None)):
        assert _call(d, **kw) == -1
    # residual required iff a residual mode is set
    assert _call(_desc(res_mode=cvx.CVX_RES_AFTER_ACT)) == -1


def test_misaligned_pointers_rejected():
    d = _desc()
    assert _call(d, x=X + 2) == -4
    assert _call(d, y=Y + 1) == -4
    assert _call(_desc(res_mode=cvx.CVX_RES_BEFORE_ACT), r=R + 2) == -4


def test_aliasing_rejected():
    d = _desc()
    assert _call(d, y=X) == -5                      # y == x
    assert _call(d, y=X + 4 * 64 * 80 * 80 - 4) == -5  # y starts in x's last element
    assert _call(d, y=W + 8) == -5
    assert _call(d, y=S - 4) == -5                  # y's tail covers scale
    r = _desc(res_mode=cvx.CVX_RES_AFTER_ACT)
    assert _call(r, r=Y + 4) == -5
    # residual may equal x (read only), so that is not an aliasing error; on a
    # shape whose plan splits the reduction, the missing workspace is the next
    # error reported (nothing is launched)
    r = _split_desc(res_mode=cvx.CVX_RES_AFTER_ACT)
    assert _call(r, r=X) == -6


def _split_desc(**kw):
    """A layer whose plan splits the reduction over workgroups (needs a workspace)."""
    for cin, hw in ((256, 20), (512, 20), (1024, 10), (2048, 7), (4096, 4)):
        d = _desc(c_in=cin, h=hw, w=hw, c_out=256, **kw)
        if cvx.cvx_conv_workspace_bytes(d) > 0:
            return d
    raise AssertionError("no split-reduction plan among the candidate shapes")


def test_workspace_checks():
    d = _split_desc()
    need = cvx.cvx_conv_workspace_bytes(d)
    assert need > 0
    assert _call(d) == -6
    assert _call(d, ws=WS, ws_bytes=need - 4) == -6
    assert _call(d, ws=Y, ws_bytes=need) == -5      # workspace overlapping the output
    assert _call(d, ws=WS + 8, ws_bytes=need) == -4  # split workspaces are 16-byte aligned
    assert cvx.cvx_conv_workspace_bytes(_desc(groups=64, c_in=64, c_out=64)) == 0


def test_fold_bn_validation():
    f = cvx.lib.cvx_fold_bn
    assert f(None, X, X + 4096, X + 8192, 1e-5, 16, Y, Y + 4096, None) == -1
    assert f(X, X + 4096, X + 8192, X + 12288, 1e-5, 0, Y, Y + 4096, None) == -2
    assert f(X, X + 4096, X + 8192, X + 12288, 0.0, 16, Y, Y + 4096, None) == -8
    assert f(X, X + 4096, X + 8192, X + 12288, 1e-5, 16, Y, Y + 32, None) == -5
    assert f(X, X + 4096, X + 8192, X + 12288, 1e-5, 16, X + 4096, Y, None) == -5
    assert f(X + 1, X + 4096, X + 8192, X + 12288, 1e-5, 16, Y, Y + 4096, None) == -4


def test_preprocess_validation():
    f = cvx.lib.cvx_preprocess_u8
    m = (ctypes.c_float * 3)(0.5, 0.5, 0.5)
    s = (ctypes.c_float * 3)(0.2, 0.2, 0.2)
    z = (ctypes.c_float * 3)(0.2, 0.0, 0.2)
    assert f(None, 1, 720, 1280, 3840, Y, 640, 640, m, s, None) == -1
    assert f(X, 1, 720, 1280, 3840, Y, 640, 640, None, s, None) == -1
    assert f(X, 0, 720, 1280, 3840, Y, 640, 640, m, s, None) == -2
    assert f(X, 1, 720, 1280, 3839, Y, 640, 640, m, s, None) == -2
    assert f(X, 1, 720, 1280, 3840, Y + 2, 640, 640, m, s, None) == -4
    assert f(X, 1, 720, 1280, 3840, Y, 640, 640, m, z, None) == -8
    assert f(X, 1, 720, 1280, 3840, X + 100, 640, 640, m, s, None) == -5


def test_gap_fc_validation():
    f = cvx.lib.cvx_gap_fc
    assert f(X, 1, 192, 7, 7, None, B, 10, Y, None) == -1
    assert f(X, 1, 5000, 7, 7, W, B, 10, Y, None) == -2
    assert f(X, 1, 192, 7, 7, W, B, 10, X + 8, None) == -5


def test_workgroup_xcds_validation():
    f = cvx.lib.cvx_workgroup_xcds
    assert f(None, 8, None) == -1
    assert f(Y, 0, None) == -2
    assert f(Y, (1 << 20) + 1, None) == -2
    assert f(Y + 2, 8, None) == -4


def _net_layers(wk, w_layout=cvx.CVX_W_OIHW):
    """cvx_layer array for a workload, with fake parameter pointers (planning only)."""
    shapes = []
    out = []
    for i, L in enumerate(wk.layers):
        lay = cvx.cvx_layer()
        lay.kind, lay.in_, lay.res = L.kind, L.inp, (L.res if L.res_mode else cvx.CVX_NO_RES)
        s_in = wk.x.shape if L.inp == -1 else shapes[L.inp]
        if L.kind == wl.KIND_PREPROC:
            n, h, w, _ = s_in
            lay.conv = cvx.cvx_conv_desc(n, 3, h, w, 3, 1, 1, 1, 0, 1, 0, 0)
            lay.dst_h, lay.dst_w = L.dst_h, L.dst_w
            lay.mean = (ctypes.c_float * 3)(*L.pre_mean)
            lay.std = (ctypes.c_float * 3)(*L.pre_std)
            o = (n, 3, L.dst_h, L.dst_w)
        elif L.kind == wl.KIND_CONV:
            n, c, h, w = s_in
            d = cvx.make_desc(n, c, h, w, L.cout, L.k, L.stride, L.pad, L.groups, L.act, L.res_mode,
                              w_layout)
            oh, ow = cvx.cvx_conv_out_shape(d)
            lay.conv = d
            lay.w, lay.scale, lay.bias = W + 0x100000 * i, S + 0x1000 * i, B + 0x1000 * i + 0x800
            o = (n, L.cout, oh, ow)
        elif L.kind == wl.KIND_GAP:
            n, c, h, w = s_in
            lay.conv = cvx.cvx_conv_desc(n, c, h, w, c, 1, 1, 1, 0, 1, 0, 0)
            o = (n, c, 1, 1)
        else:
            n, c = s_in[:2]
            lay.conv = cvx.cvx_conv_desc(n, c, 1, 1, L.cout, 1, 1, 1, 0, 1, 0, 0)
            lay.w, lay.bias = W + 0x100000 * i, B + 0x1000 * i
            o = (n, L.cout, 1, 1)
        shapes.append(o)
        out.append(lay)
    return out, shapes


@pytest.mark.parametrize("wk_fn,expect", [
    (lambda: wl.mnist_cnn(1), (1, 10, 1, 1)),
    (lambda: wl.mnist_cnn(256), (256, 10, 1, 1)),
    (lambda: wl.detector_stem(), (1, 32, 160, 160)),
    (lambda: wl.detector_pipeline(1), (1, 256, 20, 20)),
    (lambda: wl.detector_pipeline(8), (8, 256, 20, 20)),
])
def test_forward_shapes_and_workspace(wk_fn, expect, monkeypatch):
    monkeypatch.setenv("CVX_CHAIN", "0")  # placement only (the chain's own words: test_chain_plan_on_the_host)
    wk = wk_fn()
    layers, shapes = _net_layers(wk)
    assert cvx.cvx_forward_out_shape(layers) == expect
    ws = cvx.cvx_forward_workspace_bytes(layers)
    inter = [s for s in shapes[:-1]]
    largest = max(4 * s[0] * s[1] * s[2] * s[3] for s in inter)
    total = sum(4 * s[0] * s[1] * s[2] * s[3] for s in inter)
    # liveness-based reuse: at least the largest intermediate, at most all of them
    # (plus alignment) and any split-K partials
    assert ws >= largest
    assert ws <= total + 256 * len(inter) + max(
        cvx.cvx_conv_workspace_bytes(l.conv) if l.kind == 0 else 0 for l in layers)


def _block_list(n, act_skip, layout=cvx.CVX_W_PACKED):
    """conv 1x1 -> dw 3x3 -> pw 1x1 + shortcut 1x1 (added before the ReLU) -> GAP,
    all at 8x8, with fake parameter pointers (planning only)."""
    def conv(inp, res, c_in, c_out, k, groups, act, res_mode, i):
        lay = cvx.cvx_layer()
        lay.kind, lay.in_, lay.res = cvx.CVX_L_CONV, inp, res
        lay.conv = cvx.make_desc(n, c_in, 8, 8, c_out, k, 1, k // 2, groups, act, res_mode, layout)
        lay.w, lay.scale, lay.bias = W + 0x100000 * i, S + 0x1000 * i, B + 0x1000 * i + 0x800
        return lay
    R, N = cvx.CVX_ACT_RELU, cvx.CVX_ACT_NONE
    out = [conv(cvx.CVX_INPUT, cvx.CVX_NO_RES, 32, 32, 1, 1, R, cvx.CVX_RES_NONE, 0),
           conv(0, cvx.CVX_NO_RES, 32, 32, 3, 32, R, cvx.CVX_RES_NONE, 1),
           conv(0, cvx.CVX_NO_RES, 32, 64, 1, 1, act_skip, cvx.CVX_RES_NONE, 2),
           conv(1, 2, 32, 64, 1, 1, R, cvx.CVX_RES_BEFORE_ACT, 3)]
    gap = cvx.cvx_layer()
    gap.kind, gap.in_, gap.res = cvx.CVX_L_GAP, 3, cvx.CVX_NO_RES
    gap.conv = cvx.cvx_conv_desc(n, 64, 8, 8, 64, 1, 1, 1, 0, 1, 0, 0)
    return out + [gap]


@pytest.mark.parametrize("n,merged", [(64, True), (8, False)])
def test_forward_merges_1x1_shortcut(n, merged, monkeypatch):
    """A 1x1 shortcut (BN, no activation) read only by a packed pointwise layer
    that adds it before its activation runs inside that layer's kernel: its
    output takes no workspace, while its input stays live one layer longer.
    First-fit places A, B, C (the shortcut's output) at 0, |A|, 2|A| and then D
    after C, as B and C are live while D is written; merged, D goes where C was.
    Below 64 workgroups the pointwise kernel does not take the layers and
    nothing is merged; an activation on the shortcut also keeps it.  (One
    launch per layer: a chain launch would add its control words.)"""
    monkeypatch.setenv("CVX_CHAIN", "0")
    a = 4 * n * 32 * 64            # A = conv 1x1 output, B = dw output: 32 x 8 x 8
    c = 4 * n * 64 * 64            # C = shortcut output, D = pw output: 64 x 8 x 8
    kept = 2 * a + 2 * c
    ws = cvx.cvx_forward_workspace_bytes(_block_list(n, cvx.CVX_ACT_NONE))
    assert cvx.cvx_forward_workspace_bytes(_block_list(n, cvx.CVX_ACT_RELU)) == kept
    assert ws == (2 * a + c if merged else kept)
    plan = cvx.cvx_forward_plan(_block_list(n, cvx.CVX_ACT_NONE))
    assert len(plan) == 5
    if merged:
        assert plan[2] == "merged into 3"
        assert plan[3].startswith("pointwise k1 s1 + shortcut k1 s1 ") and plan[3].endswith(" shortcut=2")
        assert "kernel=cvx::k_pointwise<" in plan[3]
    else:
        assert "merged" not in plan[2] and "shortcut" not in plan[3]
    assert plan[4] == "gap kernel=cvx::k_gap_fc"
    # OIHW weights never take the pointwise kernel
    assert cvx.cvx_forward_workspace_bytes(_block_list(n, cvx.CVX_ACT_NONE, cvx.CVX_W_OIHW)) == kept


def test_forward_workspace_placement():
    """Intermediates that total at most 256 MiB each get their own region (a
    kernel writing memory that another kernel has just read runs slower); a
    larger list reuses regions.  MNIST b=256 (about 140 MB of intermediates)
    is laid out end to end, b=512 (about 280 MB) is not."""
    def inter_total(wk):
        layers, shapes = _net_layers(wk, cvx.CVX_W_PACKED)
        plan = cvx.cvx_forward_plan(layers)
        tot = 0
        for i, sh in enumerate(shapes[:-1]):
            if plan[i].startswith("merged") or plan[i].startswith("gap+fc"):
                continue
            tot += (4 * int(np.prod(sh)) + 255) // 256 * 256
        return layers, tot
    layers, tot = inter_total(wl.mnist_cnn(256))
    assert tot <= 256 << 20
    assert cvx.cvx_forward_workspace_bytes(layers) == tot
    layers, tot = inter_total(wl.mnist_cnn(512))
    assert tot > 256 << 20
    ws = cvx.cvx_forward_workspace_bytes(layers)
    assert ws < tot
    # the largest intermediate plus its input must still fit
    assert ws >= 2 * 4 * 512 * 48 * 28 * 28


def test_forward_list_validation():
    wk = wl.mnist_cnn(1)
    layers, _ = _net_layers(wk)
    arr, n = cvx.layer_array(layers)
    out = (ctypes.c_int * 4)()
    # forward reference
    bad = cvx.layer_array(layers)[0]
    bad[3].in_ = 5
    assert cvx.lib.cvx_forward_out_shape(bad, n, out) == -8
    # residual of the wrong shape (block 0's pw reading conv1's output as shortcut)
    bad = cvx.layer_array(layers)[0]
    bad[3].res = 0
    assert cvx.lib.cvx_forward_out_shape(bad, n, out) == -2
    # shape chain broken
    bad = cvx.layer_array(layers)[0]
    bad[1].conv.c_in = 47
    assert cvx.lib.cvx_forward_out_shape(bad, n, out) == -2
    # unknown kind
    bad = cvx.layer_array(layers)[0]
    bad[2].kind = 9
    assert cvx.lib.cvx_forward_out_shape(bad, n, out) == -8
    # prologue anywhere but first
    bad = cvx.layer_array(layers)[0]
    bad[4].kind = cvx.CVX_L_PREPROC
    assert cvx.lib.cvx_forward_out_shape(bad, n, out) == -8
    # runtime checks
    ws = cvx.cvx_forward_workspace_bytes(layers)
    f = cvx.lib.cvx_forward
    assert f(arr, n, X, Y, WS, ws - 4, None) == -6
    assert f(arr, n, X, Y, WS + 16, ws, None) == -4   # workspace must be 256-byte aligned
    assert f(arr, n, X, X, WS, ws, None) == -5        # output == input
    assert f(arr, n, None, Y, WS, ws, None) == -1
    assert f(arr, 0, X, Y, WS, ws, None) == -2


def test_forward_noalloc_rejects_lists_beyond_the_scratch():
    """The allocation-free forward takes its workspace from a static array of
    CVX_STATIC_SCRATCH_BYTES; a list that needs more is refused on the host
    with CVX_ERR_SCRATCH before anything is launched, and list errors come
    back as they do from cvx_forward."""
    assert cvx.cvx_static_scratch_bytes() == 32 << 20
    big, _ = _net_layers(wl.mnist_cnn(256), cvx.CVX_W_PACKED)
    assert cvx.cvx_forward_workspace_bytes(big) > cvx.cvx_static_scratch_bytes()
    arr, n = cvx.layer_array(big)
    assert cvx.lib.cvx_forward_noalloc(arr, n, X, Y, None) == -9
    assert cvx.cvx_status_str(-9) != "unknown status"
    small, _ = _net_layers(wl.mnist_cnn(1))
    arr, n = cvx.layer_array(small)
    arr[3].in_ = 5  # forward reference
    assert cvx.lib.cvx_forward_noalloc(arr, n, X, Y, None) == -8
    assert cvx.lib.cvx_forward_noalloc(arr, 0, X, Y, None) == -2


def test_chain_plan_on_the_host(monkeypatch):
    """With CVX_CHAIN=1 the detector's nine dense packed layers (stem2 .. g)
    plan as one chain launch; by default, and with the forced reuse placement
    (a chain's layers run concurrently, so no region may be reused inside it),
    every layer keeps a launch of its own; OIHW weights never chain."""
    monkeypatch.setenv("CVX_STEM_PAIR", "0")  # stem2 chains instead of pairing with stem1
    layers, _ = _net_layers(wl.detector_pipeline(1), cvx.CVX_W_PACKED)
    plan = cvx.cvx_forward_plan(layers)
    assert not any(p.startswith("chain") for p in plan)
    ws_plain = cvx.cvx_forward_workspace_bytes(layers)
    monkeypatch.setenv("CVX_CHAIN", "1")
    plan = cvx.cvx_forward_plan(layers)
    assert all(p.startswith("chain 2-10 ") and p.endswith("kernel=cvx::k_chain") for p in plan[2:]), plan
    assert cvx.cvx_forward_workspace_bytes(layers) >= ws_plain
    monkeypatch.setenv("CVX_FORWARD_REUSE", "1")
    assert not any(p.startswith("chain") for p in cvx.cvx_forward_plan(layers))
    monkeypatch.delenv("CVX_FORWARD_REUSE")
    layers, _ = _net_layers(wl.detector_pipeline(1), cvx.CVX_W_OIHW)
    assert not any(p.startswith("chain") for p in cvx.cvx_forward_plan(layers))


def test_nhwc_host_validation():
    """The channels-last entry points reject unsupported layers and bad
    arguments on the host, before any launch."""
    F32, F16 = cvx.CVX_DT_F32, cvx.CVX_DT_F16
    f = cvx.lib.cvx_conv_bn_act_nhwc
    d = _desc(c_in=12, c_out=32)  # 12 channels: not whole 16-byte fp16 pieces
    assert cvx.cvx_nhwc_packed_weights_bytes(d, F16) == 0
    assert cvx.cvx_nhwc_packed_weights_bytes(d, F32) > 0
    assert f(ctypes.byref(d), F16, X, W, S, B, None, Y, None) == -3
    d = _desc(c_in=16, c_out=32, h=8, w=8)
    assert f(ctypes.byref(d), 7, X, W, S, B, None, Y, None) == -8          # dtype
    assert f(ctypes.byref(d), F16, X + 4, W, S, B, None, Y, None) == -4    # 16-byte alignment
    assert f(ctypes.byref(d), F16, None, W, S, B, None, Y, None) == -1
    assert f(ctypes.byref(d), F16, X, W, S, B, None, X, None) == -5        # y overlaps x
    dr = _desc(c_in=16, c_out=16, h=8, w=8, res_mode=cvx.CVX_RES_AFTER_ACT)
    assert f(ctypes.byref(dr), F16, X, W, S, B, None, Y, None) == -1       # residual missing
    dg = _desc(c_in=16, c_out=16, h=8, w=8, groups=16)
    assert f(ctypes.byref(dg), F32, X, W, S, B, None, Y, None) == -3       # grouped
    # sizes: 32-row blocks x 16 (fp32) or 32 (fp16) input channels x taps
    d = _desc(c_in=64, c_out=64, h=8, w=8)
    assert cvx.cvx_nhwc_packed_weights_bytes(d, F32) == 2 * 4 * 9 * 32 * 16 * 4
    assert cvx.cvx_nhwc_packed_weights_bytes(d, F16) == 2 * 2 * 9 * 32 * 32 * 2
    assert "k_conv_nhwc<_Float16, 3" in cvx.cvx_nhwc_plan(d, F16)
    # bf16 shares fp16's 16-bit layout: same sizes, limits and checks
    BF16 = cvx.CVX_DT_BF16
    assert cvx.cvx_nhwc_packed_weights_bytes(d, BF16) == cvx.cvx_nhwc_packed_weights_bytes(d, F16)
    assert "k_conv_nhwc<__bf16, 3" in cvx.cvx_nhwc_plan(d, BF16)
    assert cvx.cvx_nhwc_packed_weights_bytes(_desc(c_in=12, c_out=32), BF16) == 0
    assert f(ctypes.byref(d), BF16, X + 4, W, S, B, None, Y, None) == -4
    assert f(ctypes.byref(d), 3, X, W, S, B, None, Y, None) == -8
    assert cvx.lib.cvx_nhwc_pack_weights(ctypes.byref(d), 3, W, X, None) == -8


def test_bf16_rounding_of_the_test_inputs_is_nearest_even():
    """The channels-last bf16 tests round their fp32 inputs and weights to
    bf16 with torch's CPU conversion, and the packing kernel rounds weights to
    nearest even; the two must agree on ties.  bf16 keeps 7 significand bits:
    between 1 and 2 its step is 2^-7, so 1 + 2^-8 is a tie."""
    import torch
    v = torch.tensor([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20,
                      1 + 2.0 ** -8 - 2.0 ** -20, 3.0e38], dtype=torch.float32)
    got = v.to(torch.bfloat16).to(torch.float32).tolist()
    assert got[:5] == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7, 1.0]
    assert np.isfinite(got[5]) and abs(got[5] - 3.0e38) <= 3.0e38 * 2.0 ** -8  # fp32's range


def test_gemm1x1_plan_on_the_host(monkeypatch):
    """A 1x1 stride-1 layer with packed weights takes the 1x1 GEMM kernel when
    it has at least 768 32 x 32 output blocks (the detector's c and f at batch
    8, not at batch 1), always with CVX_GEMM1X1=1 and never with =0; the packed
    weights are the same size either way (one layout for both kernels)."""
    P = cvx.CVX_W_PACKED
    c8 = _desc(n=8, c_in=128, h=40, w=40, c_out=128, k=1, pad=0, w_layout=P)
    c1 = _desc(n=1, c_in=128, h=40, w=40, c_out=128, k=1, pad=0, w_layout=P)
    monkeypatch.delenv("CVX_GEMM1X1", raising=False)
    assert cvx.cvx_conv_plan(c8).startswith("gemm1x1 k1 s1 waves=1600 ")
    assert cvx.cvx_conv_plan(c1).startswith("igemm_packed")
    f8 = _desc(n=8, c_in=256, h=20, w=20, c_out=256, k=1, pad=0, w_layout=P)
    assert cvx.cvx_conv_plan(f8).startswith("gemm1x1 k1 s1 waves=832 ")
    nb = cvx.cvx_packed_weights_bytes(c8)
    monkeypatch.setenv("CVX_GEMM1X1", "1")
    assert cvx.cvx_conv_plan(c1).startswith("gemm1x1")
    assert cvx.cvx_packed_weights_bytes(c1) == nb
    # 3x3, strided and OIHW layers never take it
    assert not cvx.cvx_conv_plan(_desc(n=8, w_layout=P)).startswith("gemm1x1")
    assert not cvx.cvx_conv_plan(_desc(n=8, c_in=128, h=40, w=40, c_out=128, k=1, pad=0, stride=2,
                                       w_layout=P)).startswith("gemm1x1")
    assert not cvx.cvx_conv_plan(_desc(n=8, c_in=128, h=40, w=40, c_out=128, k=1, pad=0)).startswith("gemm1x1")
    monkeypatch.setenv("CVX_GEMM1X1", "0")
    assert cvx.cvx_conv_plan(c8).startswith("igemm_packed")
    assert cvx.cvx_packed_weights_bytes(c8) == nb


def test_sixteen_pixel_tile_plan_on_the_host(monkeypatch):
    """The 16-pixel tile (packed kind 3, v_mfma_f32_16x16x4_f32): the
    detector's e, f and g at batch 1 take it, e and g without a split (their
    32 x 32 tiles number fewer than the compute units), the other layers keep
    32-channel x 32-pixel tiles; it can be forced on 1x1 layers too.  Packed
    weights hold two copies (the 32 x 32 tiles' lane order, then the 16-pixel
    tile's)."""
    P = cvx.CVX_W_PACKED
    monkeypatch.delenv("CVX_IGEMM_TILE", raising=False)
    e1 = _desc(n=1, c_in=128, h=40, w=40, c_out=256, stride=2, w_layout=P)
    g1 = _desc(n=1, c_in=256, h=20, w=20, c_out=256, w_layout=P)
    d1 = _desc(n=1, c_in=128, h=40, w=40, c_out=128, w_layout=P)
    assert " tile=3 bm=32 bn=16 tc=8 splitk=1 kernel=cvx::k_igemm_packed<3, 0, 2, 1>" in cvx.cvx_conv_plan(e1)
    assert " tile=3 bm=32 bn=16 tc=0 splitk=1 " in cvx.cvx_conv_plan(g1)
    f1 = _desc(n=1, c_in=256, h=20, w=20, c_out=256, k=1, pad=0, w_layout=P)
    assert " tile=3 bm=32 bn=16 tc=0 splitk=1 kernel=cvx::k_igemm_packed<1, 0, 4, 1>" in cvx.cvx_conv_plan(f1)
    assert " tile=0 bm=32 bn=32 " in cvx.cvx_conv_plan(d1)
    assert " tile=3 " not in cvx.cvx_conv_plan(_desc(n=8, c_in=256, h=20, w=20, c_out=256, w_layout=P))
    # one copy: ceil(c_out/32) blocks x ceil(c_in/16) chunks x 20 KB (3x3) or 2 KB (1x1)
    assert cvx.cvx_packed_weights_bytes(g1) == 2 * 8 * 16 * 5120 * 4
    assert cvx.cvx_packed_weights_bytes(f1) == 2 * 8 * 16 * 512 * 4
    monkeypatch.setenv("CVX_IGEMM_TILE", "3,4,1")
    assert " tile=3 bm=32 bn=16 tc=4 splitk=1 " in cvx.cvx_conv_plan(d1)
    assert " tile=3 bm=32 bn=16 tc=4 splitk=1 kernel=cvx::k_igemm_packed<1, 0, 4, 1>" in cvx.cvx_conv_plan(f1)
    monkeypatch.setenv("CVX_IGEMM_TILE", "3,32,1")  # wider than the tile: not a configuration
    assert " tile=3 " not in cvx.cvx_conv_plan(d1)


def test_dsblock_plan_on_the_host(monkeypatch):
    """At small batches a depthwise layer, the 1x1 layer that alone reads it and
    that layer's 1x1 shortcut run as one kernel: neither the depthwise output
    nor the shortcut's takes workspace.  Large batches keep the separate
    kernels (and the two-source pointwise merge).  The block kernel is opt-in
    (CVX_DSBLOCK=1): measured slower than the separate kernels."""
    monkeypatch.setenv("CVX_CHAIN", "0")
    plan = cvx.cvx_forward_plan(_block_list(8, cvx.CVX_ACT_NONE))
    assert not any("k_dsblock" in p for p in plan), plan
    monkeypatch.setenv("CVX_DSBLOCK", "1")
    n = 8
    a = 4 * n * 32 * 64            # conv 1x1 output, dw output: 32 x 8 x 8
    c = 4 * n * 64 * 64            # shortcut output, pw output: 64 x 8 x 8
    plan = cvx.cvx_forward_plan(_block_list(n, cvx.CVX_ACT_NONE))
    assert plan[1] == "merged into 3" and plan[2] == "merged into 3", plan
    assert plan[3].startswith("dsblock dw s1 + pw k1 + shortcut k1 ") and plan[3].endswith(" dw=1 shortcut=2")
    assert "kernel=cvx::k_dsblock" in plan[3]
    assert cvx.cvx_forward_workspace_bytes(_block_list(n, cvx.CVX_ACT_NONE)) == a + c
    # an activation on the shortcut: the depthwise and pointwise layers still
    # merge, the shortcut runs on its own and is added as a residual tensor
    plan = cvx.cvx_forward_plan(_block_list(n, cvx.CVX_ACT_RELU))
    assert plan[1] == "merged into 3" and "merged" not in plan[2], plan
    assert "kernel=cvx::k_dsblock" in plan[3] and plan[3].endswith(" dw=1"), plan
    # large batch: more workgroups than the block kernel takes
    plan = cvx.cvx_forward_plan(_block_list(256, cvx.CVX_ACT_NONE))
    assert not any("k_dsblock" in p for p in plan), plan
