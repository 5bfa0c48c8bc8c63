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
    current stream, bracketed by HIP events."""
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


def per_layer(wk, net, counts, reps: int):
    """Each layer alone, on inputs of its own shape, timed with events."""
    import torch
    from conv2d_batchnorm_activation_amd import cvx
    rows = []
    for i, L in enumerate(wk.layers):
        s_in, s_out = net.layer_io[i]
        c = counts[i]
        if L.kind == cvx.CVX_L_PREPROC:
            src = torch.from_numpy(wk.x).cuda()
            dst = torch.empty(s_out, device="cuda")
            fn = lambda src=src, dst=dst, L=L: cvx.cvx_preprocess_u8(src, dst, L.pre_mean, L.pre_std)
            kernel = "cvx::k_preprocess"
            plan = "preprocess"
        elif L.kind == cvx.CVX_L_CONV:
            lay = net.layers[i]
            d = lay.conv
            xin = torch.rand(s_in, device="cuda")
            y = torch.empty(s_out, device="cuda")
            res = xin if L.res_mode else None
            nws = cvx.cvx_conv_workspace_bytes(d)
            ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
            fn = (lambda d=d, xin=xin, lay=lay, res=res, y=y, ws=ws, nws=nws:
                  cvx.cvx_conv_bn_act(d, xin, lay.w, lay.scale, lay.bias, res, y, ws, nws))
            plan = cvx.cvx_conv_plan(d)
            kernel = plan.split("kernel=")[1] if "kernel=" in plan else plan
        else:
            continue
        ms = time_launches(fn, reps)
        us = ms * 1e3
        gflops = c["flop"] / (ms * 1e-3) / 1e9
        gbs = c["bytes"] / (ms * 1e-3) / 1e9
        bound = "mfma" if c["ai"] >= RIDGE else "hbm"
        frac = (gflops / (MFMA_F32_PEAK_TFLOPS * 1e3)) if bound == "mfma" else gbs / HBM_PEAK_GBS
        attainable = min(MFMA_F32_PEAK_TFLOPS * 1e3, c["ai"] * HBM_PEAK_GBS) if c["flop"] else None
        rows.append({"layer": L.name, "plan": plan, "kernel": kernel, "us": round(us, 3),
                     "gflop": c["flop"] / 1e9, "mbytes": c["bytes"] / 1e6, "ai": round(c["ai"], 2),
                     "gflops": round(gflops, 1), "gbs": round(gbs, 1), "bound": bound,
                     "frac_of_peak": round(frac, 4),
                     "frac_of_attainable": (round(gflops / attainable, 4) if attainable else
                                            round(gbs / HBM_PEAK_GBS, 4))})
        log(f"  {L.name:16s} {us:9.2f} us  {gflops:9.1f} GFLOP/s  {gbs:8.1f} GB/s  "
            f"{bound} frac {frac:.3f}  [{plan}]")
    return rows


def dominant(rows):
    """Kernel with the largest total time over the forward's layers: its
    algorithmic FLOPs (or bytes) per launch over its average launch time."""
    by = {}
    for r in rows:
        k = by.setdefault(r["kernel"], {"us": 0.0, "flop": 0.0, "bytes": 0.0, "n": 0, "layers": []})
        k["us"] += r["us"]
        k["flop"] += r["gflop"] * 1e9
        k["bytes"] += r["mbytes"] * 1e6
        k["n"] += 1
        k["layers"].append(r["layer"])
    name, k = max(by.items(), key=lambda kv: kv[1]["us"])
    avg_s = k["us"] / k["n"] * 1e-6
    ai = k["flop"] / k["bytes"] if k["bytes"] else 0.0
    if k["flop"] > 0 and ai >= RIDGE:
        achieved = k["flop"] / k["n"] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_F32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_F32_PEAK_TFLOPS, 4)}
    else:
        achieved = k["bytes"] / k["n"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": None, "kernel": name, "launches_per_forward": k["n"],
                 "avg_launch_us": round(k["us"] / k["n"], 3), "layers": k["layers"],
                 "flop_per_launch": k["flop"] / k["n"], "bytes_per_launch": k["bytes"] / k["n"]})
    return roof


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
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} full forwards of the batch-1 detector pipeline "
                      f"(fp64 direct 7-loop oracle, OpenMP), {dt * 1e3:.1f} ms each",
            "ms_per_forward": round(dt * 1e3, 2)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layer-reps", type=int, default=200)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layers", action="store_true")
    args = ap.parse_args()
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
    wk = wl.detector_pipeline(args.batch)
    counts = accounting.layer_counts(wk.layers, wk.x.shape)
    flop = sum(c["flop"] for c in counts)
    bytes_ = sum(c["bytes"] for c in counts)
    net = Net(wk.layers, wk.x.shape)
    x = torch.from_numpy(wk.x).cuda()
    log(f"workload {wk.name}: {len(wk.layers)} layers, {flop / 1e9:.3f} GFLOP, "
        f"{bytes_ / 1e6:.1f} MB algorithmic per forward; workspace {net.ws_bytes / 1e6:.1f} MB")

    for _ in range(args.warmup):
        net(x)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    s.record()
    for _ in range(args.steps):
        net(x)
    e.record()
    e.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = s.elapsed_time(e) / args.steps
    log(f"forward: {ms * 1e3:.1f} us/forward ({args.steps} steps, wall {wall:.3f} s)")

    rows = [] if args.no_layers else per_layer(wk, net, counts, args.layer_reps)
    roof = dominant(rows) if rows else None

    result = {
        "metric": "fused conv+BN+act GB/s & GFLOP/s vs roofline; ms/forward 640x640 b=1",
        "value": round(flop / (ms * 1e-3) / 1e9, 2),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_forward": round(ms, 5),
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
        "gbs_per_forward": round(bytes_ / (ms * 1e-3) / 1e9, 1),
        "roofline": roof,
        "layers": rows,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.batch == 1:
        result["cpu_baseline"] = cpu_baseline(wk, flop, args.cpu_budget)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
