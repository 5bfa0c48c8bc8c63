"""Host-side checks of bench.py that need no GPU."""
import os
import sys

import workloads as wl
from conv2d_batchnorm_activation_amd import cvx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _conv_shapes(wk):
    """(layer, input shape, output shape) of every convolution, following the
    list's input indices (the same arithmetic as the C planner's out-extent)."""
    out = {}
    rows = []
    for i, L in enumerate(wk.layers):
        if L.kind == cvx.CVX_L_PREPROC:
            out[i] = (wk.x.shape[0], 3, L.dst_h, L.dst_w)
            continue
        if L.kind != cvx.CVX_L_CONV:
            continue
        src = tuple(wk.x.shape) if L.inp == -1 else out[L.inp]
        oh = (src[2] + 2 * L.pad - L.k) // L.stride + 1
        ow = (src[3] + 2 * L.pad - L.k) // L.stride + 1
        out[i] = (src[0], L.cout, oh, ow)
        rows.append((L, src, out[i]))
    return rows


def test_timed_layers_get_a_residual_of_the_output_shape():
    """A layer timed alone must get a residual the kernel can read with the
    output's shape: the MNIST blocks that widen the channels (48->96, 96->192)
    must not be handed their narrower input."""
    seen_own = 0
    for wk in (wl.mnist_cnn(2), wl.detector_pipeline(1), wl.depthwise_single()):
        for L, s_in, s_out in _conv_shapes(wk):
            src = bench.residual_source(s_in, s_out, L.res_mode)
            if not L.res_mode:
                assert src == "none"
            elif src == "input":
                assert tuple(s_in) == tuple(s_out), (wk.name, L.name)
            else:
                assert src == "own"
                seen_own += 1
    assert seen_own == 2  # b0.pw and b2.pw of the MNIST net


def test_batch_scaling_is_t1_over_tb():
    """thr(B) / (B * thr(1)) = t(1) / t(B): a batch of 8 that takes four times
    one image's time runs at efficiency 0.25 and twice the batch-1 throughput."""
    r = bench.batch_scaling(70.0, 280.0, 8)
    assert r["efficiency"] == 0.25 and r["throughput_ratio"] == 2.0
    res = {"ms_per_forward_graph10": 0.07,
           "other_workloads": {"detector_b8": {"batch": 8, "us_per_forward_graph10": 280.0},
                               "mnist_b1": {"batch": 1, "us_per_forward_graph10": 50.0},
                               "mnist_b256": {"batch": 256, "us_per_forward_graph10": 100.0}}}
    out = bench.batch_scalings(res)
    assert out["detector_b8"]["efficiency"] == 0.25
    assert out["mnist_b256"]["efficiency"] == 0.5 and out["mnist_b256"]["throughput_ratio"] == 128.0
    assert bench.batch_scalings({}) == {}
