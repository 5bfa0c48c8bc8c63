"""Algorithmic FLOP and byte counts used to report throughput and roofline fractions.

Conventions (restated from the pages, checked by the CPU tests against the
figures the pages print):
  * FLOP = 2 * multiply-adds of the convolution (or fc); the epilogue's few
    operations per output are not counted in the headline.
  * Bytes = every fp32 tensor the layer must touch, counted once: the input
    elements the window actually reads, the output, the residual (if any), the
    weights and the folded per-channel scale and bias.  With the scale/bias term
    left out this is the convention behind the depthwise arithmetic-intensity
    range of "Как я свертки ускорял" ("Ускоряем скорость", problem 3).
  * Prologue bytes = the u8 frame read once plus the fp32 planar tensor written
    once, the fused-pass ledger of "A fused Ampere preprocess kernel" ("The
    theory").
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Sequence

FP32 = 4


def out_extent(n: int, k: int, stride: int, pad: int) -> int:
    return (n + 2 * pad - k) // stride + 1


@dataclass
class Count:
    flop: float
    bytes: float

    @property
    def ai(self) -> float:
        return self.flop / self.bytes if self.bytes else 0.0


def conv_count(n: int, cin: int, h: int, w: int, cout: int, k: int, stride: int, pad: int,
               groups: int = 1, residual: bool = False, with_scale_bias: bool = True) -> Count:
    oh, ow = out_extent(h, k, stride, pad), out_extent(w, k, stride, pad)
    macs = n * cout * oh * ow * (cin // groups) * k * k
    if k == 1 and pad == 0:
        # a strided 1x1 window reads only every stride-th row and column
        in_elems = n * cin * oh * ow
    else:
        in_elems = n * cin * h * w
    out_elems = n * cout * oh * ow
    w_elems = cout * (cin // groups) * k * k
    b = FP32 * (in_elems + out_elems * (2 if residual else 1) + w_elems
                + (2 * cout if with_scale_bias else 0))
    return Count(2.0 * macs, float(b))


def gap_fc_count(n: int, c: int, h: int, w: int, out_f: int) -> Count:
    flop = n * c * h * w + 2.0 * n * c * out_f
    b = FP32 * (n * c * h * w + out_f * c + out_f + n * out_f)
    return Count(float(flop), float(b))


def preprocess_bytes(n: int, src_h: int, src_w: int, dst_h: int, dst_w: int) -> int:
    """u8 HWC frame read once + fp32 CHW tensor written once."""
    return n * (src_h * src_w * 3 + 3 * dst_h * dst_w * FP32)


def preprocess_three_pass_bytes(n: int, src_h: int, src_w: int, dst_h: int, dst_w: int) -> List[int]:
    """Ledger of the unfused resize -> normalise -> layout passes (per pass)."""
    src = src_h * src_w * 3
    small_u8 = dst_h * dst_w * 3
    f32 = dst_h * dst_w * 3 * FP32
    return [n * (src + small_u8), n * (small_u8 + f32), n * (f32 + f32)]


def layer_counts(layers: Sequence, x_shape: Sequence[int]) -> List[Dict]:
    """Per-layer counts for a ``workloads`` layer list applied to an input of x_shape."""
    shapes: List[tuple] = []

    def shape_of(i):
        return tuple(x_shape) if i == -1 else shapes[i]

    rows = []
    for L in layers:
        if L.kind == 3:  # prologue: input is u8 NHWC
            n, sh, sw, _ = shape_of(L.inp)
            out = (n, 3, L.dst_h, L.dst_w)
            c = Count(0.0, float(preprocess_bytes(n, sh, sw, L.dst_h, L.dst_w)))
        elif L.kind == 0:
            n, cin, h, w = shape_of(L.inp)
            oh, ow = out_extent(h, L.k, L.stride, L.pad), out_extent(w, L.k, L.stride, L.pad)
            out = (n, L.cout, oh, ow)
            c = conv_count(n, cin, h, w, L.cout, L.k, L.stride, L.pad, L.groups,
                           residual=(L.res_mode != 0))
        elif L.kind == 1:
            n, cin, h, w = shape_of(L.inp)
            out = (n, cin, 1, 1)
            c = Count(float(n * cin * h * w), float(FP32 * (n * cin * h * w + n * cin)))
        else:
            n, cin = shape_of(L.inp)[:2]
            out = (n, L.cout, 1, 1)
            c = Count(2.0 * n * cin * L.cout, float(FP32 * (n * cin + L.cout * cin + L.cout + n * L.cout)))
        shapes.append(out)
        rows.append({"name": L.name, "kind": L.kind, "out_shape": out, "flop": c.flop,
                     "bytes": c.bytes, "ai": c.ai})
    return rows
