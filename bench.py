#!/usr/bin/env python3
"""Benchmark of the fused conv + folded-BN + activation path on one MI355X.

One step = one whole forward of the detector pipeline at batch 1: a u8
720x1280 RGB frame -> fused resize/normalise/CHW to 3x640x640 -> stem
(3->16 s2, 16->32 s2) -> bridge (32->64 s2) -> the seven nano-detector layers
(64@80^2 ... 256@20^2), every conv with folded BN + SiLU and the residual add
on the stride-1 equal-width layers, as one cvx_forward on one stream.  The
frame, the weights and all buffers are resident in HBM before timing starts.

Printed: one JSON line (rank 0) with the whole-forward throughput in GFLOP/s
(algorithmic 2*MAC FLOPs of the convolutions / time), ms per forward, the
roofline position of the dominant kernel (per-launch average from HIP events
over back-to-back launches), a per-layer table, and the CPU oracle timed on a
bounded sample of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch B]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix
RIDGE = MFMA_F32_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def time_launches(fn, reps: int, warm: int = 3) -> float:
    """Average milliseconds per call of `fn` over `reps` back-to-back calls on the
    current stream, bracketed by HIP events (includes the host's per-call cost
    whenever that exceeds the GPU's)."""
    import torch
    for _ in range(warm):
        fn()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / reps


def capture(fn, inner: int):
    """A HIP graph of `inner` back-to-back calls of `fn` (kernel launches only;
    the library records no memsets or host synchronisation)."""
    import torch
    fn()  # plans are made (and cached) outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(inner):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, inner: int, replays: int, warm: int = 2) -> float:
    """Average milliseconds per captured call: `replays` replays of a graph of
    `inner` calls, bracketed by HIP events on the replay stream."""
    import torch
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / (replays * inner)


def residual_source(s_in, s_out, res_mode) -> str:
    """Which tensor a layer timed alone gets as its residual: its own input when
    that has the output's shape (the detector's stride-1 equal-width layers),
    else a tensor of the output's shape ("own"), or none.  The kernels read the
    residual with the output's shape, so a smaller buffer would be read past its
    end."""
    if not res_mode:
        return "none"
    return "input" if tuple(s_in) == tuple(s_out) else "own"


def layer_residual(xin, s_out, res_mode, alloc=None):
    import torch
    src = residual_source(xin.shape, s_out, res_mode)
    if src == "none":
        return None
    if src == "input":
        return xin
    return alloc(s_out) if alloc is not None else torch.rand(s_out, device=xin.device)


COLD_BYTES = 512 << 20   # a cold leg rotates at least this many bytes of distinct buffers
MAX_COLD_SETS = 2048


class Pool:
    """Views into one large device buffer of random fp32 values (256-byte aligned),
    for the cold leg's rotating buffer sets."""

    def __init__(self, nbytes: int):
        import torch
        self.buf = torch.empty(nbytes // 4 + 64, device="cuda").uniform_()
        self.off = 0

    def take(self, shape, dtype=None):
        import numpy as np
        import torch
        n = int(np.prod(shape))
        if dtype == torch.uint8:
            nf = (n + 3) // 4
            t = self.buf[self.off:self.off + nf].view(torch.uint8)[:n].view(*shape)
        else:
            nf = n
            t = self.buf[self.off:self.off + nf].view(*shape)
        self.off += (nf + 63) // 64 * 64
        assert self.off <= self.buf.numel(), "cold pool exhausted"
        return t


def layer_setup(wk, net, i, alloc):
    """Layer i alone on buffers from `alloc(shape, dtype=None)`: (call, plan, kernel,
    splitk).  The weights, scales and biases are the network's own."""
    import torch
    from conv2d_batchnorm_activation_amd import cvx
    L = wk.layers[i]
    s_in, s_out = net.layer_io[i]
    if L.kind == cvx.CVX_L_PREPROC:
        src = alloc(s_in, torch.uint8)
        dst = alloc(s_out)
        fn = lambda src=src, dst=dst, L=L: cvx.cvx_preprocess_u8(src, dst, L.pre_mean, L.pre_std)
        return fn, "preprocess", "cvx::k_preprocess", 1
    lay = net.layers[i]
    d = lay.conv
    xin = alloc(s_in)
    y = alloc(s_out)
    res = layer_residual(xin, s_out, L.res_mode, alloc)
    nws = cvx.cvx_conv_workspace_bytes(d)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
    fn = (lambda d=d, xin=xin, lay=lay, res=res, y=y, ws=ws, nws=nws:
          cvx.cvx_conv_bn_act(d, xin, lay.w, lay.scale, lay.bias, res, y, ws, nws))
    plan = cvx.cvx_conv_plan(d)
    kernel = plan.split("kernel=")[1] if "kernel=" in plan else plan
    splitk = int(plan.split("splitk=")[1].split()[0]) if "splitk=" in plan else 1
    return fn, plan, kernel, splitk


def hot_alloc(shape, dtype=None):
    import torch
    if dtype == torch.uint8:
        return torch.randint(0, 256, tuple(shape), dtype=torch.uint8, device="cuda")
    return torch.rand(tuple(shape), device="cuda")


def time_rotating(fns, reps: int) -> float:
    """Average milliseconds per launch over a graph that calls each of `fns` (each
    on its own buffers) in turn, at least 20 launches, replayed until about `reps`
    launches have been timed."""
    inner = max(len(fns), 20)
    seq = [fns[j % len(fns)] for j in range(inner)]
    g = capture(lambda: [f() for f in seq], 1)
    return time_graph(g, inner, max(2, reps // inner))


def layer_buffer_bytes(wk, net, i) -> int:
    """Bytes of the buffers one timed launch of layer i gets: its whole input
    tensor (a strided 1x1 layer reads only part of it), its output and, when
    the residual is a tensor of its own, that too; each rounded to 256 bytes."""
    import numpy as np
    from conv2d_batchnorm_activation_amd import cvx
    L = wk.layers[i]
    s_in, s_out = net.layer_io[i]
    r = lambda b: (int(b) + 255) // 256 * 256
    if L.kind == cvx.CVX_L_PREPROC:
        return r(np.prod(s_in)) + r(4 * np.prod(s_out))
    own = residual_source(s_in, s_out, L.res_mode) == "own"
    return r(4 * np.prod(s_in)) + r(4 * np.prod(s_out)) * (2 if own else 1)


def cold_layer_us(wk, net, i, reps: int) -> "tuple[float, int, int]":
    """Layer i timed over rotating buffer sets totalling at least COLD_BYTES (at
    most MAX_COLD_SETS sets), so that neither the L2 caches nor the 256 MB MALL
    hold its input or output from one launch to the next: (us per launch,
    sets, bytes per set)."""
    import math
    import torch
    set_bytes = layer_buffer_bytes(wk, net, i)
    sets = int(min(MAX_COLD_SETS, max(2, math.ceil(COLD_BYTES / set_bytes))))
    pool = Pool(sets * (set_bytes + 1024) + (4 << 20))
    fns = [layer_setup(wk, net, i, pool.take)[0] for _ in range(sets)]
    ms = time_rotating(fns, max(reps, sets))
    del fns, pool
    torch.cuda.empty_cache()
    return ms * 1e3, sets, set_bytes


def copy_floor_us(nbytes: int, reps: int) -> "tuple[float, float]":
    """A plain device copy (torch copy_, the runtime's copy) that reads and
    writes nbytes in total, hot (same buffers) and cold (rotating over at least
    COLD_BYTES): the rate a bandwidth-bound kernel of that size can reach on
    this GPU, beside the HBM peak.  (us hot, us cold)."""
    import math
    import torch
    n = max(64, int(nbytes) // 8)  # floats per side
    a = torch.rand(n, device="cuda")
    b = torch.empty_like(a)
    fn = lambda: b.copy_(a)
    inner = 20
    hot = time_graph(capture(fn, inner), inner, max(1, reps // inner)) * 1e3
    sets = int(min(MAX_COLD_SETS, max(2, math.ceil(COLD_BYTES / (8 * n)))))
    bufs = [(torch.rand(n, device="cuda"), torch.empty(n, device="cuda")) for _ in range(sets)]
    fns = [lambda x=x, y=y: y.copy_(x) for x, y in bufs]
    cold = time_rotating(fns, max(reps, sets)) * 1e3
    del bufs, fns, a, b
    torch.cuda.empty_cache()
    return hot, cold


def per_layer(wk, net, counts, reps: int, cold: bool = True):
    """Each layer alone, on inputs of its own shape, timed with events: `us` over
    the same buffers every launch (cache-resident: hot), `us_cold` over rotating
    buffer sets of at least 512 MB (cold).  Fractions of the HBM peak come from
    the cold time; fractions of the MFMA peak from the hot time."""
    from conv2d_batchnorm_activation_amd import cvx
    rows = []
    fplan = cvx.cvx_forward_plan(net.arr)
    for i, L in enumerate(wk.layers):
        c = counts[i]
        if L.kind not in (cvx.CVX_L_PREPROC, cvx.CVX_L_CONV):
            continue
        fn, plan, kernel, splitk = layer_setup(wk, net, i, hot_alloc)
        marker()
        ms_eager = time_launches(fn, reps)
        inner = 20
        ms = time_graph(capture(fn, inner), inner, max(1, reps // inner))
        us = ms * 1e3
        gflops = c["flop"] / (ms * 1e-3) / 1e9
        gbs = c["bytes"] / (ms * 1e-3) / 1e9
        bound = "mfma" if c["ai"] >= RIDGE else "hbm"
        us_cold, sets, set_bytes = (None, 0, 0)
        if cold:
            us_cold, sets, set_bytes = cold_layer_us(wk, net, i, reps)
        gbs_cold = c["bytes"] / (us_cold * 1e-6) / 1e9 if us_cold else None
        if bound == "mfma":
            frac = gflops / (MFMA_F32_PEAK_TFLOPS * 1e3)
        else:
            frac = (gbs_cold if gbs_cold is not None else gbs) / HBM_PEAK_GBS
        attainable = min(MFMA_F32_PEAK_TFLOPS * 1e3, c["ai"] * HBM_PEAK_GBS) if c["flop"] else None
        copy_hot = copy_cold = None
        if bound == "hbm" and cold:
            copy_hot, copy_cold = copy_floor_us(c["bytes"], reps)
        rows.append({"layer": L.name, "plan": plan, "kernel": kernel, "splitk": splitk,
                     "us": round(us, 3), "us_eager": round(ms_eager * 1e3, 3),
                     "us_cold": round(us_cold, 3) if us_cold else None, "cold_sets": sets,
                     "cold_rotated_mbytes": round(sets * set_bytes / 1e6, 1),
                     "gflop": c["flop"] / 1e9, "mbytes": c["bytes"] / 1e6, "ai": round(c["ai"], 2),
                     "gflops": round(gflops, 1), "gbs_hot": round(gbs, 1),
                     "gbs_cold": round(gbs_cold, 1) if gbs_cold else None, "bound": bound,
                     "frac_of_peak": round(frac, 4),
                     "frac_of_peak_hot": round((gflops / (MFMA_F32_PEAK_TFLOPS * 1e3)) if bound == "mfma"
                                               else gbs / HBM_PEAK_GBS, 4),
                     "frac_of_attainable": (round(gflops / attainable, 4) if attainable else
                                            round((gbs_cold or gbs) / HBM_PEAK_GBS, 4)),
                     "copy_us": round(copy_hot, 3) if copy_hot else None,
                     "copy_us_cold": round(copy_cold, 3) if copy_cold else None,
                     "of_copy_cold": round(copy_cold / us_cold, 3) if copy_cold and us_cold else None,
                     # a layer the forward runs inside another kernel (a stem pair) is timed
                     # here alone for reference; the pair has a row of its own below
                     "in_forward": not (fplan[i].startswith("merged into") or fplan[i].startswith("stem_pair")),
                     "forward_plan": fplan[i]})
        cold_txt = f" cold {us_cold:7.2f} us {gbs_cold:7.1f} GB/s" if us_cold else ""
        if copy_cold:
            cold_txt += f" (a copy of its bytes: {copy_cold:.2f} us cold)"
        log(f"  {L.name:16s} {us:8.2f} us hot (eager {ms_eager * 1e3:6.2f}){cold_txt}  "
            f"{gflops:9.1f} GFLOP/s  {gbs:8.1f} GB/s hot  {bound} frac {frac:.3f}  [{plan}]")
    for i, line in enumerate(fplan):
        if line.startswith("stem_pair") and not wk.layers[i].res_mode:
            marker()
            rows.append(stem_pair_row(wk, counts, i - 1, line, reps, cold))
    marker()
    return rows


def stem_pair_row(wk, counts, i, line, reps: int, cold: bool):
    """Layers i (a stem) and i+1, which the forward runs as one kernel
    (k_stem_pair), timed as that kernel: a two-layer list on an input of the
    stem's input shape (with "from=u8", the prologue before them too, on the
    u8 frames), hot (a graph of 20 forwards on the same buffers) and cold
    (rotating sets of at least COLD_BYTES).  Algorithmic counts: the layers'
    FLOPs; the first layer's input, the second layer's output and residual and
    the weights (what the kernel passes between the layers never leaves the
    chip)."""
    import dataclasses
    import math
    import numpy as np
    import torch
    import workloads as wl
    from conv2d_batchnorm_activation_amd.net import Net
    L1, L2 = wk.layers[i], wk.layers[i + 1]
    u8 = "from=u8" in line
    if u8:
        first = i - 1
        sub = [dataclasses.replace(wk.layers[first], inp=wl.NET_INPUT), dataclasses.replace(L1, inp=0),
               dataclasses.replace(L2, inp=1)]
        shape = tuple(wk.x.shape)
        in_b = float(np.prod(shape))  # u8 frames
    else:
        first = i
        sub = [dataclasses.replace(L1, inp=wl.NET_INPUT), dataclasses.replace(L2, inp=0)]
        shape = _layer_input_shape(wk, i)
        in_b = 4.0 * float(np.prod(shape))
    net = Net(sub, shape)
    flop = sum(counts[j]["flop"] for j in range(first, i + 2))
    out_b = 4.0 * float(np.prod(net.out_shape))
    byts = in_b + out_b * (2 if L2.res_mode else 1) + \
        4.0 * (L1.params["w"].size + L2.params["w"].size + 2 * L1.cout + 2 * L2.cout)
    rand_in = (lambda: torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda")) if u8 else \
        (lambda: torch.rand(shape, device="cuda"))
    x = rand_in()
    fn = lambda: net(x)
    inner = 20
    us = time_graph(capture(fn, inner), inner, max(1, reps // inner)) * 1e3
    us_cold = None
    sets = 0
    if cold:
        set_bytes = int(in_b) + int(out_b) + net.ws_bytes
        sets = int(min(MAX_COLD_SETS, max(2, math.ceil(COLD_BYTES / set_bytes))))
        bufs = [(rand_in(), torch.empty(net.out_shape, device="cuda"),
                 torch.empty(max(net.ws_bytes, 256), dtype=torch.uint8, device="cuda")) for _ in range(sets)]
        from conv2d_batchnorm_activation_amd import cvx
        fns = [lambda b=b: cvx.cvx_forward(net.arr, b[0], b[1], b[2], net.ws_bytes) for b in bufs]
        us_cold = time_rotating(fns, max(reps, sets)) * 1e3
        del bufs, fns
        torch.cuda.empty_cache()
    gflops = flop / (us * 1e-6) / 1e9
    ai = flop / byts
    bound = "mfma" if ai >= RIDGE else "hbm"
    gbs_cold = byts / (us_cold * 1e-6) / 1e9 if us_cold else None
    frac = gflops / (MFMA_F32_PEAK_TFLOPS * 1e3) if bound == "mfma" else (gbs_cold or byts / (us * 1e-6) / 1e9) / HBM_PEAK_GBS
    kernel = line.split("kernel=")[1].split()[0] if "kernel=" in line else line
    name = "+".join(wk.layers[j].name for j in range(first, i + 2))
    log(f"  {name:16s} {us:8.2f} us hot" + (f" cold {us_cold:7.2f} us" if us_cold else "") +
        f"  {gflops:9.1f} GFLOP/s  {bound} frac {frac:.3f}  [{line}]")
    return {"layer": name, "plan": line, "kernel": kernel, "splitk": 1,
            "us": round(us, 3), "us_cold": round(us_cold, 3) if us_cold else None, "cold_sets": sets,
            "gflop": flop / 1e9, "mbytes": byts / 1e6, "ai": round(ai, 2), "gflops": round(gflops, 1),
            "gbs_hot": round(byts / (us * 1e-6) / 1e9, 1), "gbs_cold": round(gbs_cold, 1) if gbs_cold else None,
            "bound": bound, "frac_of_peak": round(frac, 4), "in_forward": True, "forward_plan": line}


def _layer_input_shape(wk, i):
    """The input shape of layer i of a workload (its producer's output shape)."""
    from conv2d_batchnorm_activation_amd.net import Net  # noqa: F401
    import workloads as wl
    shapes = []
    for L in wk.layers[:i + 1]:
        s_in = wk.x.shape if L.inp == wl.NET_INPUT else shapes[L.inp]
        if L.kind == wl.KIND_PREPROC:
            n = s_in[0]
            out = (n, 3, L.dst_h, L.dst_w)
        elif L.kind == wl.KIND_CONV:
            n, _, h, w = s_in
            oh = (h + 2 * L.pad - L.k) // L.stride + 1
            ow = (w + 2 * L.pad - L.k) // L.stride + 1
            out = (n, L.cout, oh, ow)
        else:
            out = (s_in[0], L.cout if L.kind == wl.KIND_FC else s_in[1], 1, 1)
        shapes.append(out)
    L = wk.layers[i]
    return tuple(wk.x.shape if L.inp == wl.NET_INPUT else shapes[L.inp])


MARKER_KERNEL = "spin_kernel"


def forward_launches(wk, plan) -> list:
    """The forward's launches in order: (layers they compute, joined with '+',
    kernel), one per plan line that is not merged into a later one."""
    import re
    out = []
    for i, line in enumerate(plan):
        if line.startswith("merged into"):
            continue
        names = [wk.layers[j].name for j in range(len(plan)) if plan[j] == f"merged into {i}"] + [wk.layers[i].name]
        m = re.search(r"kernel=(cvx::\w+(?:<[^>]*>)?)", line)
        out.append(("+".join(names), m.group(1) if m else ""))
    return out


def forward_probe(wk, net, x, forwards: int = 20) -> dict:
    """`forwards` back-to-back forwards right after the per-layer timing's last
    marker, closed by a marker of their own: in a kernel trace they give each
    layer's duration inside the forward, beside its duration alone."""
    import torch
    from conv2d_batchnorm_activation_amd import cvx
    for _ in range(forwards):
        net(x)
    marker()
    torch.cuda.synchronize()
    return {"forwards": forwards, "launches": forward_launches(wk, cvx.cvx_forward_plan(net.arr))}


def marker() -> None:
    """A tiny torch spin kernel on the stream: in a kernel trace it separates the
    launches of one layer's timing from the next (see --rocprof-summary)."""
    import torch
    torch.cuda._sleep(1)


def dominant(rows, with_traffic: bool = True):
    """The kernel (exact template instantiation, as profilers name it) with the
    largest total time over the forward's layers, and its roofline position:
    algorithmic FLOPs (or bytes) per launch over its average launch time.

    A split-K layer's launch also carries the partial sums' round trip through
    memory, so the average is taken over the kernel's layers without a split
    (all of its layers when it has none of those)."""
    by = {}
    for r in rows:
        if not r.get("in_forward", True):
            continue  # timed alone for reference; the forward runs it inside another kernel
        k = by.setdefault(r["kernel"], [])
        k.append(r)
    name, group = max(by.items(), key=lambda kv: sum(r["us"] for r in kv[1]))
    single = [r for r in group if r["splitk"] == 1]
    use = single or group
    n = len(use)
    avg_us = sum(r["us"] for r in use) / n
    flop = sum(r["gflop"] * 1e9 for r in use) / n
    byts = sum(r["mbytes"] * 1e6 for r in use) / n
    ai = flop / byts if byts else 0.0
    if flop > 0 and ai >= RIDGE:
        achieved = flop / (avg_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_F32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F32_PEAK_TFLOPS, 4)}
    else:
        achieved = byts / (avg_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    plans = {r["layer"]: r["plan"] for r in use}
    roof.update({"traffic": traffic_for(name, [r["layer"] for r in use], plans) if with_traffic else None,
                 "kernel": name, "avg_launch_us": round(avg_us, 3),
                 "measured_layers": [r["layer"] for r in use],
                 "all_layers": [r["layer"] for r in group],
                 "flop_per_launch": flop, "bytes_per_launch": byts})
    return roof


# ---------------------------------------------------------------- HBM traffic
# Measured HBM bytes per launch come from two rocprofv3 counter passes
# (FETCH_SIZE, WRITE_SIZE) over `bench.py --pmc-probe`, scaled by what the same
# counters read for a plain device copy of known size, and are kept as a small
# text record under profiles/ together with a hash of the kernel's sources.  A
# record whose hash no longer matches the sources is stale and gives null.
CSRC = os.path.join(ROOT, "conv2d_batchnorm_activation_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_sources_hash(kernel: str) -> str:
    import hashlib
    base = kernel.split("<")[0].split("::")[-1]
    srcfile = {"k_igemm_packed": "k_igemm_packed.hip", "k_igemm": "k_igemm.hip",
               "k_direct": "k_direct.hip", "k_stem": "k_direct.hip", "k_depthwise3x3": "k_depthwise.hip",
               "k_dw_planes": "k_depthwise.hip", "k_dw_rows": "k_depthwise.hip", "k_pointwise": "k_pointwise.hip",
               "k_preprocess": "k_preprocess.hip", "k_preprocess_rows": "k_preprocess.hip",
               "k_stem_pair": "k_stem_pair.hip", "k_conv_nhwc": "k_nhwc.hip", "k_chain": "k_chain.hip",
               "k_gemm1x1": "k_gemm1x1.hip"}.get(base)
    h = hashlib.sha256()
    for f in ([srcfile] if srcfile else []) + ["bufio.h", "epilogue.h", "cvx_internal.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_record(path: str) -> dict:
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(("#", "|", " ")):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    return rec


TRAFFIC_FILE = os.path.join(PROFILES, "counters_detector640_b1.md")


def traffic_for(kernel: str, layers, plans=None) -> "float | None":
    """Mean measured HBM bytes per launch of `kernel` over `layers`, from the
    committed counter record, or None (no record, the sources changed, or a
    layer's plan is no longer the one the counters were taken with)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = kernel_sources_hash(kernel)
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if not line.startswith("record: "):
                continue
            rec = json.loads(line[len("record: "):])
            if rec["kernel"] != kernel or rec["source_hash"] != want:
                continue
            per = rec["traffic_bytes_per_layer"]
            rp = rec.get("plan_per_layer", {})
            if plans and any(rp.get(l) != plans.get(l) for l in layers):
                continue
            if layers and all(l in per for l in layers):
                return round(sum(per[l] for l in layers) / len(layers), 1)
    return None


COPY_BYTES = 64 << 20  # the calibration copy: 64 MiB read, 64 MiB written

PMC_WORKLOADS = {
    "detector_b1": ("detector pipeline 640x640 b=1", lambda wl: wl.detector_pipeline(1)),
    "detector_b8": ("detector pipeline 640x640 b=8", lambda wl: wl.detector_pipeline(8)),
    "mnist_b256": ("MNIST depthwise-separable CNN b=256", lambda wl: wl.mnist_cnn(256)),
}


def pmc_probe(args) -> int:
    """Short run for counter passes: one 64 MiB device copy (the calibration),
    then each layer of the workload's forward alone, `reps` times, in order, on
    the same buffers.  Prints a manifest line (JSON) that --pmc-summary uses to
    map dispatches to layers."""
    import torch
    import workloads as wl
    from conv2d_batchnorm_activation_amd import accounting, cvx
    from conv2d_batchnorm_activation_amd.net import Net
    wk = PMC_WORKLOADS[args.workload][1](wl)
    net = Net(wk.layers, wk.x.shape)
    counts = accounting.layer_counts(wk.layers, wk.x.shape)
    calls = []
    for i, L in enumerate(wk.layers):
        if L.kind not in (cvx.CVX_L_PREPROC, cvx.CVX_L_CONV):
            continue
        fn, plan, kernel, splitk = layer_setup(wk, net, i, hot_alloc)
        calls.append((L.name, kernel, splitk, counts[i]["bytes"], counts[i]["flop"], fn, plan))
    a = torch.empty(COPY_BYTES // 4, device="cuda").uniform_()
    b = torch.empty_like(a)
    for c in calls:
        c[5]()  # plans made and code loaded before the probed dispatches
    torch.cuda.synchronize()
    b.copy_(a)  # calibration: marks the start of the probed dispatches
    for c in calls:
        for _ in range(args.reps):
            c[5]()
    torch.cuda.synchronize()
    print(json.dumps({"workload": args.workload,
                      "manifest": [{"layer": n, "kernel": k, "splitk": s, "reps": args.reps,
                                    "algorithmic_bytes": by, "algorithmic_flop": fl, "plan": pl}
                                   for n, k, s, by, fl, _, pl in calls]}))
    return 0


def _dispatches(d: str):
    """{counter: [(dispatch id, kernel name, value)]} from rocprofv3 counter CSVs
    under d: instances summed, except GRBM counters (one per XCD, all counting
    the same cycles), whose largest instance is taken."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                c = r["Counter_Name"]
                k = int(r["Dispatch_Id"])
                v = float(r["Counter_Value"])
                name, old = per.setdefault(c, {}).get(k, (r["Kernel_Name"], None))
                if old is None:
                    new = v
                elif c.startswith("GRBM_"):
                    new = max(old, v)
                else:
                    new = old + v
                per[c][k] = (name, new)
    return {c: [(k, n, v) for k, (n, v) in sorted(m.items())] for c, m in per.items()}


def _trace_dispatches(d: str):
    """[(dispatch id, kernel name, duration ns)] from a rocprofv3 kernel trace under d."""
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                            float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))))
    return sorted(out)


def _probe_map(disp, manifest):
    """Counter value per probed layer: the calibration copy is the last copy
    dispatch before the layers; the cvx dispatches after it follow the
    manifest, one dispatch per call (a split-K layer finishes its tiles inside
    the same launch)."""
    cal = [i for i, (_, n, v) in enumerate(disp) if "copy" in n.lower() and "cvx::" not in n]
    i0 = cal[-1]
    cal_v = disp[i0][2]
    rest = [(n, v) for _, n, v in disp[i0 + 1:] if "cvx::" in n]
    per, names, j = {}, {}, 0
    for m in manifest:
        vals = []
        for _ in range(m["reps"]):
            n, v = rest[j]
            assert m["kernel"].split("<")[0] in n, (m, n)
            vals.append(v)
            j += 1
        per[m["layer"]] = sum(vals) / len(vals)
        names[m["layer"]] = n.split("(")[0].replace("void ", "").strip()  # the variant that ran
    return cal_v, per, names


SIMDS = 1024  # 256 compute units x 4
CLOCK_GHZ = 2.4  # MI355X peak engine clock (the peaks above assume it)


def pmc_summary(args) -> int:
    with open(args.manifest) as fh:
        info = json.loads(fh.read().strip().splitlines()[-1])
    manifest = info["manifest"]
    title = PMC_WORKLOADS.get(info.get("workload", ""), ("", None))[0] or info.get("workload", "")
    ctr, cal, names = {}, {}, {}
    for d in args.pmc_summary:
        for c, disp in _dispatches(d).items():
            cal[c], ctr[c], nm = _probe_map(disp, manifest)
            names.update(nm)
        tr = _trace_dispatches(d)
        if tr:
            _, ctr["duration_ns"], nm = _probe_map(tr, manifest)
            names.update(nm)
    has = lambda *cs: all(c in ctr for c in cs)
    lines = [f"# Counters per launch, {title}, each layer alone",
             "",
             f"Counter passes (rocprofv3 --pmc, one counter group per run): {args.cmd}",
             ""]
    ff = fw = None
    if has("FETCH_SIZE", "WRITE_SIZE"):
        ff = COPY_BYTES / (cal["FETCH_SIZE"] * 1024.0)
        fw = COPY_BYTES / (cal["WRITE_SIZE"] * 1024.0)
        lines += [f"Calibration: a {COPY_BYTES >> 20} MiB device copy read FETCH_SIZE {cal['FETCH_SIZE']:.0f} KiB "
                  f"(scale {ff:.4f}) and WRITE_SIZE {cal['WRITE_SIZE']:.0f} KiB (scale {fw:.4f}).",
                  "traffic = FETCH_SIZE*1024*scale_f + WRITE_SIZE*1024*scale_w (L2 egress and writes: "
                  "includes MALL hits, so it is an upper bound on HBM bytes), averaged over the calls."]
    if has("SQ_VALU_MFMA_BUSY_CYCLES", "duration_ns"):
        lines += [f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (kernel duration x {CLOCK_GHZ} GHz x 1024 SIMDs): "
                  "the share of the launch's peak matrix-pipe cycles it kept busy, with the duration from a "
                  "kernel trace of the same probe (GRBM_GUI_ACTIVE under --pmc also counts the profiler's "
                  "serialisation of each dispatch, so the profiler's MfmaUtil is not used)."]
    if has("SQ_INSTS_VALU_MFMA_MOPS_F32"):
        lines += ["MFMA FLOP = SQ_INSTS_VALU_MFMA_MOPS_F32 x 512 (fp32 matrix operations issued, padding "
                  "included) against the layer's algorithmic 2*MAC count."]
    lines += [""]
    head = ["layer", "kernel"]
    if ff is not None:
        head += ["FETCH KiB", "WRITE KiB", "traffic bytes", "algorithmic bytes", "traffic/alg"]
    if has("duration_ns"):
        head += ["trace us"]
        if ff is not None:
            head += ["traffic GB/s", "of HBM peak"]
    if has("SQ_VALU_MFMA_BUSY_CYCLES", "duration_ns"):
        head += ["MFMA busy"]
    if has("SQ_INSTS_VALU_MFMA_MOPS_F32"):
        head += ["MFMA FLOP / alg"]
    for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES"):
        if c in ctr:
            head.append(c)
    lines += ["| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    recs = {}
    for m in manifest:
        L = m["layer"]
        k = names.get(L, m["kernel"])
        row = [L, f"`{k}`"]
        if ff is not None:
            t = ctr["FETCH_SIZE"][L] * 1024 * ff + ctr["WRITE_SIZE"][L] * 1024 * fw
            row += [f"{ctr['FETCH_SIZE'][L]:.0f}", f"{ctr['WRITE_SIZE'][L]:.0f}", f"{t:.0f}",
                    f"{m['algorithmic_bytes']:.0f}", f"{t / m['algorithmic_bytes']:.2f}"]
            r = recs.setdefault(k, {"kernel": k, "source_hash": kernel_sources_hash(k),
                                    "traffic_bytes_per_layer": {}, "plan_per_layer": {}})
            r["traffic_bytes_per_layer"][L] = round(t, 1)
            r["plan_per_layer"][L] = m.get("plan")
        if has("duration_ns"):
            dur = ctr["duration_ns"][L]
            row += [f"{dur / 1e3:.2f}"]
            if ff is not None:
                row += [f"{t / dur:.0f}", f"{t / dur / HBM_PEAK_GBS:.3f}"]
        if has("SQ_VALU_MFMA_BUSY_CYCLES", "duration_ns"):
            dur = ctr["duration_ns"][L]
            row += [f"{ctr['SQ_VALU_MFMA_BUSY_CYCLES'][L] / (dur * CLOCK_GHZ * SIMDS):.3f}"]
        if has("SQ_INSTS_VALU_MFMA_MOPS_F32"):
            fl = m.get("algorithmic_flop", 0.0)
            row += [f"{ctr['SQ_INSTS_VALU_MFMA_MOPS_F32'][L] * 512 / fl:.2f}" if fl else "-"]
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES"):
            if c in ctr:
                row.append(f"{ctr[c][L]:.0f}")
        lines.append("| " + " | ".join(row) + " |")
    if recs:
        lines.append("")
        for r in recs.values():
            lines.append("record: " + json.dumps(r))
    print("\n".join(lines))
    return 0


def tile_sweep(args) -> int:
    """Every packed tile configuration (kind x tc x split, and the persistent
    form at 256 and 512 workgroups, forced through CVX_IGEMM_TILE) of every
    dense packed layer of a workload, and for a 1x1 stride-1 layer the 1x1
    GEMM kernel (CVX_GEMM1X1=1), each timed alone
    like the per-layer rows (a graph of 20 launches, hot), against the
    planner's own choice.  Prints a markdown table (the per-shape tile choice's
    evidence) and one JSON line per layer."""
    import torch
    import workloads as wl
    from conv2d_batchnorm_activation_amd import cvx
    from conv2d_batchnorm_activation_amd.net import Net
    wk = PMC_WORKLOADS[args.workload][1](wl)
    net = Net(wk.layers, wk.x.shape)
    rows = []
    print(f"# Tile sweep, {PMC_WORKLOADS[args.workload][0]}: every packed configuration of each dense layer "
          "(and the 1x1 GEMM kernel for 1x1 stride-1 layers)\n")
    print(f"Command: {args.cmd}\n")
    print("Each configuration timed alone as a graph of 20 launches on the same buffers (hot), "
          f"{args.layer_reps} launches; `default` is the planner's choice.\n")
    print("| layer | default plan | default us | best plan | best us | default / best | configurations |")
    print("|---|---|---|---|---|---|---|")
    for i, L in enumerate(wk.layers):
        if L.kind != cvx.CVX_L_CONV:
            continue
        d = net.layers[i].conv
        plan0 = cvx.cvx_conv_plan(d)
        if "igemm_packed" not in plan0 and not plan0.startswith("gemm1x1"):
            continue
        def timed():
            fn, plan, _, _ = layer_setup(wk, net, i, hot_alloc)
            inner = 20
            ms = time_graph(capture(fn, inner), inner, max(1, args.layer_reps // inner))
            return ms * 1e3, plan.split(" kernel")[0]
        os.environ.pop("CVX_IGEMM_TILE", None)
        us0, p0 = timed()
        res = [(us0, p0)]
        seen = {p0}
        if p0.startswith("igemm_packed k1 s1 "):  # the 1x1 GEMM kernel as an alternative
            prev = os.environ.get("CVX_GEMM1X1")
            os.environ["CVX_GEMM1X1"] = "1"
            p = cvx.cvx_conv_plan(d).split(" kernel")[0]
            if p.startswith("gemm1x1") and p not in seen:
                seen.add(p)
                res.append(timed())
            if prev is None:
                os.environ.pop("CVX_GEMM1X1", None)
            else:
                os.environ["CVX_GEMM1X1"] = prev
        for kind in range(4):  # 32 x 32, 64, 128 pixels, and the 16-pixel tile
            for tc in (0, 4, 8, 16, 32, 64, 128):
                for sk, pe in [(1, 0), (1, 256), (1, 512), (2, 0), (3, 0), (4, 0), (6, 0), (8, 0)]:
                    os.environ["CVX_IGEMM_TILE"] = f"{kind},{tc},{sk},{pe}"
                    p = cvx.cvx_conv_plan(d).split(" kernel")[0]
                    if p in seen or f"tile={kind} " not in p or f"tc={tc} " not in p or f"splitk={sk}" not in p:
                        continue
                    if pe and f"persist={pe}" not in p:
                        continue
                    seen.add(p)
                    res.append(timed())
        os.environ.pop("CVX_IGEMM_TILE", None)
        best = min(res)
        print(f"| {L.name} | {p0} | {us0:.2f} | {best[1]} | {best[0]:.2f} | {us0 / best[0]:.3f} | {len(res)} |",
              flush=True)
        rows.append({"layer": L.name, "default": p0, "default_us": round(us0, 3), "best": best[1],
                     "best_us": round(best[0], 3), "all": [[p, round(u, 3)] for u, p in sorted(res)]})
        torch.cuda.synchronize()
    print()
    for r in rows:
        print("sweep: " + json.dumps(r))
    return 0


def rocprof_summary(args) -> int:
    """Markdown table of a rocprofv3 --kernel-trace --stats run."""
    import csv
    import glob
    f = glob.glob(os.path.join(args.rocprof_summary, "**", "*kernel_stats.csv"), recursive=True)[0]
    with open(f) as fh:
        rows = list(csv.DictReader(fh))
    print(f"# Kernel durations, {args.title}")
    print()
    print(f"Command: {args.cmd}")
    print()
    print("| kernel | calls | avg us | min us | max us | total % |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = r["Name"].split("(")[0].replace("void ", "")
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.1f} |")
    traces = glob.glob(os.path.join(args.rocprof_summary, "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        with open(traces[0]) as fh:
            tr = list(csv.DictReader(fh))
        groups = {}
        for r in tr:
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            if not name.startswith("cvx::"):
                continue
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            grid = (int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])) // max(wg, 1)
            key = (name, r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"], grid,
                   r["VGPR_Count"], r["Accum_VGPR_Count"], r["LDS_Block_Size"], r["Scratch_Size"])
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        print()
        print("Per launch shape (one row per layer shape):")
        print()
        print("| kernel | grid x,y,z (threads) | workgroups | vgpr | agpr | lds B | scratch | calls | avg us | median us |")
        print("|---|---|---|---|---|---|---|---|---|---|")
        for key, v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            v = sorted(v)
            print(f"| `{key[0]}` | {key[1]},{key[2]},{key[3]} | {key[4]} | {key[5]} | {key[6]} | "
                  f"{key[7]} | {key[8]} | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | "
                  f"{v[len(v) // 2] / 1e3:.2f} |")
        if args.bench_json:
            layer_agreement(tr, args.bench_json, args.ref_json)
    return 0


def in_forward_table(probe: dict, seg, alone: dict) -> None:
    """Each launch of the forward probe (its forwards back to back) against the
    same layer's hot launches timed alone."""
    launches = probe["launches"]
    n = probe["forwards"]
    print()
    if len(seg) != n * len(launches) or any(seg[k][0] != launches[k % len(launches)][1] for k in range(len(seg))):
        print(f"(in-forward table skipped: {len(seg)} launches in the probe, {n} x {len(launches)} expected)")
        return
    print(f"Per layer inside the forward ({n} back-to-back forwards, trace durations) against the same "
          "launch alone (hot graph launches above):")
    print()
    print("| layer | kernel | in forward avg us | alone avg us | in forward / alone |")
    print("|---|---|---|---|---|")
    tot_in = tot_alone = 0.0
    for p, (name, kernel) in enumerate(launches):
        d = [seg[k][1] for k in range(p, len(seg), len(launches))]
        t = sum(d) / len(d) / 1e3
        a = alone.get(name)
        tot_in += t
        tot_alone += a or 0.0
        print(f"| {name} | `{kernel}` | {t:.2f} | {a:.2f} | {t / a:.2f} |" if a else
              f"| {name} | `{kernel}` | {t:.2f} | - | - |")
    print(f"| sum | | {tot_in:.2f} | {tot_alone:.2f} | {tot_in / tot_alone:.2f} |" if tot_alone else "")


def layer_agreement(tr, bench_json: str, ref_json: str = "") -> None:
    """Per layer of the bench's layer timing (launches between two markers), the
    trace's average kernel duration beside the bench's event time, and the
    dominant kernel's average over the layers of its roofline figure."""
    with open(bench_json) as fh:
        res = json.loads([ln for ln in fh.read().splitlines() if ln.startswith("{")][-1])
    layers = res.get("layers", [])
    tr = sorted(tr, key=lambda r: int(r["Start_Timestamp"]))
    segs, cur = [], None
    for r in tr:
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        if MARKER_KERNEL in r["Kernel_Name"]:
            cur = []
            segs.append(cur)
        elif cur is not None and name.startswith("cvx::"):
            cur.append((name, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    segs = [sg for sg in segs if sg]
    probe = res.get("forward_probe")
    want = len(layers) + (1 if probe else 0)
    if len(segs) != want:
        print(f"\n(layer agreement skipped: {len(segs)} marked segments, {want} expected)")
        return
    probe_seg = segs[len(layers)] if probe else None
    segs = segs[:len(layers)]
    print()
    print("Per layer of the bench's layer timing (the launches between two markers):")
    print()
    # a layer's launches in order: warm-up and `reps` eager calls, then the
    # graph replays on the same buffers (hot, what `us` times), then the cold sets
    reps = int(res.get("layer_reps", 200))
    # the bench's own hot figure, from the untraced run when there is one (the
    # traced run's event times carry the tracer's per-launch cost)
    ref_us = {}
    if ref_json:
        with open(ref_json) as fh:
            ref0 = json.loads([ln for ln in fh.read().splitlines() if ln.startswith("{")][-1])
        ref_us = {r["layer"]: r["us"] for r in ref0.get("layers", [])}
    hot0 = 3 + reps
    hot1 = hot0 + 20 * (2 + max(1, reps // 20))
    col = "untraced bench us (graph of 20, hot)" if ref_us else "bench us (graph of 20, hot)"
    print(f"| layer | kernel (the segment's most frequent) | launches | trace avg us, all | trace avg us, hot graph launches | {col} |")
    print("|---|---|---|---|---|---|")
    avg = {}
    for L, sg in zip(layers, segs):
        counts = {}
        for n, _ in sg:
            counts[n] = counts.get(n, 0) + 1
        k = max(counts, key=counts.get)
        d = [t for n, t in sg if n == k]
        hot = d[hot0:hot1] if len(d) >= hot1 else d
        avg[L["layer"]] = sum(hot) / len(hot) / 1e3
        print(f"| {L['layer']} | `{k}` | {len(d)} | {sum(d) / len(d) / 1e3:.2f} | {avg[L['layer']]:.2f} | "
              f"{ref_us.get(L['layer'], L['us']):.2f} |")
    roof = res.get("roofline") or {}
    use = roof.get("measured_layers") or []
    if use and all(u in avg for u in use):
        t = sum(avg[u] for u in use) / len(use)
        print()
        print(f"Dominant kernel `{roof.get('kernel')}` over {', '.join(use)}: trace average over the hot "
              f"graph launches {t:.2f} us per launch (kernel start to end); the traced run's own `avg_launch_us` "
              f"{roof.get('avg_launch_us')} us (its event times carry the tracer's per-launch cost).")
        if ref_json:
            with open(ref_json) as fh:
                ref = json.loads([ln for ln in fh.read().splitlines() if ln.startswith("{")][-1])
            rr = ref.get("roofline") or {}
            print(f"The untraced bench run of the same build: `avg_launch_us` {rr.get('avg_launch_us')} us "
                  f"for `{rr.get('kernel')}` (frac {rr.get('frac')}).")
    if probe_seg:
        in_forward_table(probe, probe_seg, avg)


def gpu_clocks() -> dict:
    """Current shader and memory clocks as rocm-smi reports them (for a record
    against throttling), or an empty dict when the tool is unavailable."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
    except Exception:  # noqa: BLE001 -- a record only; absent tool or format
        return {}
    out = {}
    for card, v in d.items():
        if isinstance(v, dict):
            out[card] = {k: v[k] for k in v if "sclk" in k.lower() or "mclk" in k.lower()
                         or "fclk" in k.lower()}
    return out


def host_info() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_model": model, "nproc": affinity, "os_cpu_count": os.cpu_count()}


def stats(per_step_ms) -> dict:
    import numpy as np
    a = np.asarray(per_step_ms, dtype=np.float64) * 1e3
    return {"mean_us": round(float(a.mean()), 3), "p50_us": round(float(np.percentile(a, 50)), 3),
            "p99_us": round(float(np.percentile(a, 99)), 3), "min_us": round(float(a.min()), 3),
            "cv": round(float(a.std() / a.mean()), 4) if a.mean() > 0 else None, "n": int(a.size)}


def plain_steps(fn, steps: int) -> float:
    """`steps` back-to-back calls of `fn` on one stream between two events and
    nothing else: the ms between them.  The host enqueues a forward in about
    half the time the GPU takes to run it, so this is GPU time."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    e1.synchronize()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def timed_steps(fn, steps: int):
    """`steps` back-to-back calls of `fn` on one stream with an event before and
    after each: (total ms between the first and last event, per-call ms list).
    The GPU runs the calls back to back (the host enqueues faster than they
    run), so a per-call time is that forward's own duration plus the cost of
    the event between calls (about 4 us on the detector forward): the spread
    comes from such a pass, the means from `plain_steps`."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for k in range(steps):
        fn()
        ev[k + 1].record()
    ev[-1].synchronize()
    torch.cuda.synchronize()
    per = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
    return ev[0].elapsed_time(ev[-1]), per


def cold_forward_us(net, wk, steps: int) -> dict:
    """Whole forwards over rotating (frame, workspace, output) sets totalling at
    least 512 MB (at most 2048 sets: a tiny list rotates less, which the record
    states), so every intermediate a forward writes and reads is absent from
    the caches when it starts (the weights, a few MB, are shared)."""
    import math
    import torch
    from conv2d_batchnorm_activation_amd import cvx
    out_elems = 1
    for v in net.out_shape:
        out_elems *= v
    ws_b = (max(net.ws_bytes, 256) + 255) // 256 * 256
    set_bytes = wk.x.nbytes + ws_b + out_elems * 4
    sets = int(min(MAX_COLD_SETS, max(2, math.ceil(COLD_BYTES / set_bytes))))
    pool = Pool(sets * (set_bytes + 1024) + (4 << 20))
    u8 = wk.x.dtype.name == "uint8"
    bufs = [(pool.take(wk.x.shape, torch.uint8 if u8 else None), pool.take(net.out_shape),
             pool.take((ws_b // 4,))) for _ in range(sets)]
    k = [0]

    def one():
        xj, oj, wj = bufs[k[0] % sets]
        k[0] += 1
        cvx.cvx_forward(net.arr, xj, oj, wj, net.ws_bytes)
    for _ in range(sets):
        one()
    n = max(steps, 2 * sets)
    plain_us = plain_steps(one, n) / n * 1e3
    _, per = timed_steps(one, n)
    st = stats(per)
    # mean without per-forward events (comparable with the hot figure); the
    # other statistics from the pass with an event after each forward
    st["events_mean_us"] = st["mean_us"]
    st["mean_us"] = round(plain_us, 3)
    st["sets"] = sets
    st["rotated_mbytes"] = round(sets * set_bytes / 1e6, 1)
    del bufs, pool
    torch.cuda.empty_cache()
    return st


def forward_time_ms(net, x, steps: int, per_graph: int = 1) -> float:
    """Milliseconds per forward: `per_graph` forwards captured as one graph,
    replayed until `steps` forwards ran, between two events.  With one forward
    per graph each replay adds the graph launch's own cost (about 5 us); with
    ten, a tiny forward's figure is the GPU's time, not the host's enqueue."""
    import torch
    g = capture(lambda: net(x), per_graph)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / (reps * per_graph)


def other_workloads(layer_reps: int, steps: int):
    """The other configurations, reported beside the headline (not part of
    `value`), timed like it (back-to-back calls, and a graph replay per
    forward): the MNIST depthwise-separable net at batch 256 (with per-layer
    rows: its depthwise and pointwise layers are large enough to show bandwidth
    rather than launch latency) and at batch 1, the single depthwise layer, and
    the detector pipeline at batch 8 (per layer too, with the roofline position
    of its dominant kernel).  Per-layer inputs are reused across the timed
    launches, so they are cache-resident (hot) figures."""
    import torch
    import workloads as wl
    from conv2d_batchnorm_activation_amd import accounting
    from conv2d_batchnorm_activation_amd.net import Net
    out = {}
    for name, wk, layers in [("mnist_b256", wl.mnist_cnn(256), True),
                             ("mnist_b1", wl.mnist_cnn(1), False),
                             ("depthwise_48x28x28", wl.depthwise_single(), True),
                             ("dw3x3_64x13x13_res", wl.sweep_layer("h_64x13_dw3x3"), True),
                             ("detector_b8", wl.detector_pipeline(8), True)]:
        log(f"{name}: timing the forward")
        counts = accounting.layer_counts(wk.layers, wk.x.shape)
        flop = sum(c["flop"] for c in counts)
        byts = sum(c["bytes"] for c in counts)
        net = Net(wk.layers, wk.x.shape)
        x = torch.from_numpy(wk.x).cuda()
        for _ in range(3):
            net(x)
        ms = plain_steps(lambda: net(x), steps) / steps
        _t, per = timed_steps(lambda: net(x), steps)
        ms_graph = forward_time_ms(net, x, steps)
        ms_graph10 = forward_time_ms(net, x, steps, per_graph=10)
        log(f"{name}: {ms * 1e3:.1f} us/forward, {ms_graph * 1e3:.1f} us as a graph replay, "
            f"{ms_graph10 * 1e3:.1f} us per forward in graphs of ten "
            f"({flop / 1e9:.3f} GFLOP, {byts / 1e6:.1f} MB)")
        entry = {"workload": wk.name, "batch": int(wk.x.shape[0]), "us_per_forward": round(ms * 1e3, 2),
                 "us_per_forward_graph": round(ms_graph * 1e3, 2),
                 "us_per_forward_graph10": round(ms_graph10 * 1e3, 2),
                 "gflops": round(flop / (ms * 1e-3) / 1e9, 1),
                 "gbs": round(byts / (ms * 1e-3) / 1e9, 1), "spread": stats(per),
                 "cold": cold_forward_us(net, wk, steps)}
        if name == "mnist_b1":
            # the whole-block kernel (opt-in, CVX_DSBLOCK=1) timed the same way
            os.environ["CVX_DSBLOCK"] = "1"
            try:
                net_b = Net(wk.layers, wk.x.shape)
                for _ in range(3):
                    net_b(x)
                entry["us_per_forward_dsblock"] = round(plain_steps(lambda: net_b(x), steps) / steps * 1e3, 2)
                entry["us_per_forward_graph10_dsblock"] = round(
                    forward_time_ms(net_b, x, steps, per_graph=10) * 1e3, 2)
                log(f"{name}: {entry['us_per_forward_dsblock']:.1f} us/forward with each block as one kernel")
                del net_b
            finally:
                os.environ.pop("CVX_DSBLOCK", None)
        if layers:
            entry["layers"] = per_layer(wk, net, counts, layer_reps)
            # the same roofline position as the headline's, for this workload's
            # dominant kernel (the traffic record covers the headline only)
            entry["roofline"] = dominant(entry["layers"], with_traffic=False)
        out[name] = entry
        del net
        torch.cuda.empty_cache()
    return out


F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 and bf16 matrix (the same rate)


def layout_comparison(reps: int):
    """The detector's dense layers a..g alone at batch 1 and 8, each as the NCHW
    fp32 layer (packed weights, the production path), the NHWC fp32 layer and
    the NHWC fp16 and bf16 layers (fp32 accumulation), timed like the per-layer rows
    (graphs of 20 launches on the same buffers, hot).  The NHWC variants'
    inputs are synthetic tensors of the same shapes (timing does not depend on
    the values)."""
    import torch
    import workloads as wl
    from conv2d_batchnorm_activation_amd import accounting, cvx
    out = []
    for batch in (1, 8):
        for name in [s[0] for s in wl.SWEEP[:7]]:
            wk = wl.sweep_layer(name, batch=batch)
            L = wk.layers[0]
            n, c, h, w = wk.x.shape
            cnt = accounting.conv_count(n, c, h, w, L.cout, L.k, L.stride, L.pad, L.groups,
                                        residual=L.res_mode != 0)
            row = {"layer": name, "batch": batch, "gflop": round(cnt.flop / 1e9, 4)}
            dev = "cuda"
            g_, b_, m_, v_ = (torch.from_numpy(L.params[k]).to(dev) for k in ("gamma", "beta", "mean", "var"))
            scale = torch.empty(L.cout, device=dev)
            bias = torch.empty(L.cout, device=dev)
            cvx.cvx_fold_bn(g_, b_, m_, v_, wl.EPS, scale, bias)
            wt = torch.from_numpy(L.params["w"]).to(dev)
            # NCHW fp32, packed weights
            d = cvx.make_desc(n, c, h, w, L.cout, L.k, L.stride, L.pad, L.groups, L.act, L.res_mode,
                              cvx.CVX_W_PACKED)
            oh, ow = cvx.cvx_conv_out_shape(d)
            wp = torch.empty(cvx.cvx_packed_weights_bytes(d) // 4, device=dev)
            cvx.cvx_pack_weights(d, wt, wp)
            x = torch.rand((n, c, h, w), device=dev)
            y = torch.empty((n, L.cout, oh, ow), device=dev)
            res = x if L.res_mode else None
            nws = cvx.cvx_conv_workspace_bytes(d)
            ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
            fn = lambda: cvx.cvx_conv_bn_act(d, x, wp, scale, bias, res, y, ws, nws)
            ms = time_graph(capture(fn, 20), 20, max(1, reps // 20))
            row["nchw_f32_us"] = round(ms * 1e3, 3)
            row["nchw_plan"] = cvx.cvx_conv_plan(d).split(" kernel")[0]
            for dt, tag, tdt in ((cvx.CVX_DT_F32, "nhwc_f32", torch.float32),
                                 (cvx.CVX_DT_F16, "nhwc_f16", torch.float16),
                                 (cvx.CVX_DT_BF16, "nhwc_bf16", torch.bfloat16)):
                wq = torch.empty(cvx.cvx_nhwc_packed_weights_bytes(d, dt), dtype=torch.uint8, device=dev)
                cvx.cvx_nhwc_pack_weights(d, dt, wt, wq)
                xq = torch.rand((n, h, w, c), device=dev).to(tdt)
                yq = torch.empty((n, oh, ow, L.cout), dtype=tdt, device=dev)
                rq = xq if L.res_mode else None
                fq = (lambda d=d, dt=dt, xq=xq, wq=wq, rq=rq, yq=yq:
                      cvx.cvx_conv_bn_act_nhwc(d, dt, xq, wq, scale, bias, rq, yq))
                ms = time_graph(capture(fq, 20), 20, max(1, reps // 20))
                row[tag + "_us"] = round(ms * 1e3, 3)
                row[tag + "_plan"] = cvx.cvx_nhwc_plan(d, dt).split(" kernel")[0]
            f = cnt.flop
            row["nchw_f32_frac_mfma"] = round(f / (row["nchw_f32_us"] * 1e-6) / 1e12 / MFMA_F32_PEAK_TFLOPS, 4)
            row["nhwc_f32_frac_mfma"] = round(f / (row["nhwc_f32_us"] * 1e-6) / 1e12 / MFMA_F32_PEAK_TFLOPS, 4)
            row["nhwc_f16_frac_mfma_f16"] = round(f / (row["nhwc_f16_us"] * 1e-6) / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)
            row["nhwc_bf16_frac_mfma_bf16"] = round(f / (row["nhwc_bf16_us"] * 1e-6) / 1e12 / F16_MFMA_PEAK_TFLOPS,
                                                    4)
            log(f"  b={batch} {name:16s} NCHW f32 {row['nchw_f32_us']:7.2f} us  NHWC f32 {row['nhwc_f32_us']:7.2f} us  "
                f"NHWC f16 {row['nhwc_f16_us']:7.2f} us  NHWC bf16 {row['nhwc_bf16_us']:7.2f} us")
            out.append(row)
    return out


def batch_scaling(t1_us: float, tb_us: float, batch: int) -> dict:
    """Throughput-scaling of a batch against batch 1: images per second at
    batch B over B times the batch-1 rate, thr(B) / (B * thr(1)), which is
    t(1) / t(B) (1.0 when a batch of B takes no longer than one image), and
    the plain throughput ratio thr(B) / thr(1)."""
    eff = t1_us / tb_us
    return {"batch": batch, "us_b1": t1_us, "us_batch": tb_us, "efficiency": round(eff, 4),
            "throughput_ratio": round(batch * eff, 3)}


def batch_scalings(result: dict) -> dict:
    """The detector at b=8 and the MNIST net at b=256 against their batch-1
    forwards, from the graphs-of-ten figures (GPU time: the back-to-back figure
    of a tiny forward is the host's enqueue rate)."""
    ow = result.get("other_workloads", {})
    out = {}
    d8 = ow.get("detector_b8")
    if d8 and result.get("ms_per_forward_graph10"):
        out["detector_b8"] = batch_scaling(round(result["ms_per_forward_graph10"] * 1e3, 2),
                                           d8["us_per_forward_graph10"], d8["batch"])
    m1, m256 = ow.get("mnist_b1"), ow.get("mnist_b256")
    if m1 and m256:
        out["mnist_b256"] = batch_scaling(m1["us_per_forward_graph10"], m256["us_per_forward_graph10"],
                                          m256["batch"])
    return out


def cpu_baseline(wk, flop_per_forward: float, budget_s: float):
    import oracle
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(wk.layers, wk.x)
        reps += 1
        if time.perf_counter() - t0 >= budget_s or reps >= 200:
            break
    dt = (time.perf_counter() - t0) / reps
    return {"value": round(flop_per_forward / dt / 1e9, 3), "unit": "GFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", **host_info(),
            "sample": f"{reps} full forwards of the batch-1 detector pipeline "
                      f"(fp64 direct 7-loop oracle, OpenMP), {dt * 1e3:.1f} ms each",
            "ms_per_forward": round(dt * 1e3, 2)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layer-reps", type=int, default=200)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layers", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the other configurations")
    ap.add_argument("--others-only", action="store_true",
                    help="time only the other configurations and print them (for profiling)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="short run for rocprofv3 counter passes (prints a manifest line)")
    ap.add_argument("--reps", type=int, default=3, help="calls per layer in --pmc-probe")
    ap.add_argument("--workload", default="detector_b1", choices=sorted(PMC_WORKLOADS),
                    help="workload of --pmc-probe")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="turn counter passes (one output directory each) into a table and, with "
                         "FETCH_SIZE and WRITE_SIZE, the traffic record (stdout)")
    ap.add_argument("--manifest", help="stdout of the --pmc-probe run (for --pmc-summary)")
    ap.add_argument("--layouts-only", action="store_true",
                    help="time only the NCHW / NHWC fp32 / NHWC fp16 comparison of the dense layers")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="time every packed tile configuration of each dense layer of --workload")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="markdown table of a rocprofv3 --kernel-trace --stats output directory")
    ap.add_argument("--cmd", default="", help="command line recorded in a summary")
    ap.add_argument("--bench-json", default="",
                    help="stdout of the traced bench run (for --rocprof-summary's per-layer agreement)")
    ap.add_argument("--ref-json", default="",
                    help="stdout of an untraced bench run of the same build, quoted beside it")
    ap.add_argument("--title", default="detector pipeline 640x640 b=1 (bench.py)",
                    help="workload named in a --rocprof-summary heading")
    args = ap.parse_args()
    if args.rocprof_summary:
        return rocprof_summary(args)
    if args.pmc_summary:
        return pmc_summary(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): this build has no "
              f"multi-GPU path; run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import workloads as wl
    from conv2d_batchnorm_activation_amd import accounting
    from conv2d_batchnorm_activation_amd.net import Net

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.pmc_probe:
        return pmc_probe(args)
    if args.tile_sweep:
        return tile_sweep(args)
    if args.others_only:
        print(json.dumps({"other_workloads": other_workloads(args.layer_reps, args.steps)}))
        return 0
    if args.layouts_only:
        print(json.dumps({"layout_comparison": layout_comparison(args.layer_reps)}))
        return 0
    wk = wl.detector_pipeline(args.batch)
    counts = accounting.layer_counts(wk.layers, wk.x.shape)
    flop = sum(c["flop"] for c in counts)
    bytes_ = sum(c["bytes"] for c in counts)
    net = Net(wk.layers, wk.x.shape)
    x = torch.from_numpy(wk.x).cuda()
    log(f"workload {wk.name}: {len(wk.layers)} layers, {flop / 1e9:.3f} GFLOP, "
        f"{bytes_ / 1e6:.1f} MB algorithmic per forward; workspace {net.ws_bytes / 1e6:.1f} MB")

    clocks_start = gpu_clocks()
    # eager: one cvx_forward call per step (host planning is cached after the first)
    for _ in range(args.warmup):
        net(x)
    torch.cuda.synchronize()
    # the timed region: exactly `steps` forwards between two events
    t_wall = time.perf_counter()
    total_ms = plain_steps(lambda: net(x), args.steps)
    wall = time.perf_counter() - t_wall
    ms_eager = total_ms / args.steps
    # two more reruns of the same timed region (run-to-run spread)
    reruns = [round(ms_eager * 1e3, 3)]
    for _ in range(2):
        reruns.append(round(plain_steps(lambda: net(x), args.steps) / args.steps * 1e3, 3))
    # the per-forward spread: a separate pass with an event after each forward
    # (each event adds its own cost, reported as the difference of the means)
    _t, per = timed_steps(lambda: net(x), args.steps)
    spread = stats(per)
    spread["event_cost_us"] = round(spread["mean_us"] - ms_eager * 1e3, 3)
    # graph: the forward captured once, replayed once per step
    ms = forward_time_ms(net, x, args.steps)
    ms10 = forward_time_ms(net, x, args.steps, per_graph=10)
    cold = cold_forward_us(net, wk, args.steps)
    log(f"forward: {ms_eager * 1e3:.1f} us/forward ({args.steps} cvx_forward calls; p50 "
        f"{spread['p50_us']} p99 {spread['p99_us']} cv {spread['cv']}; reruns {reruns}), "
        f"{ms * 1e3:.1f} us as a graph replay per forward, {ms10 * 1e3:.1f} us per forward in graphs "
        f"of ten, cold {cold['mean_us']} us (wall {wall:.3f} s)")

    rows = [] if args.no_layers else per_layer(wk, net, counts, args.layer_reps)
    probe = forward_probe(wk, net, x) if rows else None
    roof = dominant(rows) if rows else None

    result = {
        "metric": "fused conv+BN+act GB/s & GFLOP/s vs roofline; ms/forward 640x640 b=1",
        "value": round(flop / (ms_eager * 1e-3) / 1e9, 2),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_eager, 5),
        "ms_per_forward": round(ms_eager, 5),
        "ms_per_forward_graph": round(ms, 5),
        "ms_per_forward_graph10": round(ms10, 5),
        "forward_spread": spread,
        "forward_reruns_us": reruns,
        "forward_cold": cold,
        "layer_reps": args.layer_reps,
        "forward_probe": probe,
        "gpu_clocks": {"start": clocks_start, "end": None},
        "timing": "steps back-to-back cvx_forward calls on one stream between two HIP events "
                  "and nothing else; forward_spread (mean, p50, p99, cv of the per-forward "
                  "times) comes from a separate pass with an event after each forward, whose "
                  "mean exceeds the timed region's by event_cost_us (the events' own cost); "
                  "forward_reruns_us repeats the timed region twice more; ms_per_forward_graph replays a HIP graph of one forward per step, "
                  "whose launch boundary adds about 5 us (ms_per_forward_graph10: graphs of ten "
                  "forwards, which also removes most of the gaps between kernels); forward_cold "
                  "rotates frame, workspace "
                  "and output over sets totalling >= 512 MB. Per-layer `us` from graphs of 20 "
                  "back-to-back launches on the same buffers (cache-resident: hot), `us_cold` "
                  "over rotating buffer sets of >= 512 MB; HBM fractions use the cold time; "
                  "bandwidth-bound rows also carry copy_us/copy_us_cold, a plain device copy "
                  "of the same bytes, and of_copy_cold = copy_us_cold / us_cold",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"detector pipeline b={args.batch}: u8 720x1280 frame -> "
                               "resize/normalise 640x640 -> stem 3->16->32 s2 -> bridge 32->64 s2 "
                               "-> nano-detector layers a..g (SiLU, residual on s1 layers)",
                   "batch": args.batch, "gflop_per_forward": round(flop / 1e9, 4),
                   "mbytes_per_forward": round(bytes_ / 1e6, 3)},
        "gbs_per_forward": round(bytes_ / (ms_eager * 1e-3) / 1e9, 1),
        "roofline": roof,
        "layers": rows,
        "cpu_baseline": None,
    }
    if not args.no_others and not args.no_layers:
        result["other_workloads"] = other_workloads(args.layer_reps, args.steps)
        result["batch_scaling"] = batch_scalings(result)
        result["layout_comparison"] = layout_comparison(args.layer_reps)
    result["gpu_clocks"]["end"] = gpu_clocks()
    if not args.no_cpu_baseline and args.batch == 1:
        result["cpu_baseline"] = cpu_baseline(wk, flop, args.cpu_budget)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
