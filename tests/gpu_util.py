"""Helpers for the GPU parity tests: run one layer or a layer list through the
C ABI and compare against the oracle with the parity bound
|gpu - oracle| <= 1e-4 * max(1, |oracle|), element by element."""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = 1e-4
DEV = "cuda:0"


def say(msg: str) -> None:
    """Name the case before the GPU step (a fault then points at it)."""
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def check(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - r) / np.maximum(1.0, np.abs(r))
    worst = float(err.max()) if err.size else 0.0
    if worst > TOL:
        idx = np.unravel_index(int(err.argmax()), err.shape)
        raise AssertionError(f"{what}: max scaled error {worst:.3e} at {idx}: gpu={g[idx]!r} "
                             f"oracle={r[idx]!r}")
    return worst


class Guarded:
    """An output tensor with NaN-filled guard bands on both sides, to catch any
    write outside the output (the edge-tile overrun class of bug)."""

    def __init__(self, shape, guard: int = 4096, fill=float("nan")):
        self.n = int(np.prod(shape))
        self.guard = guard
        self.buf = torch.full((guard + self.n + guard,), fill, dtype=torch.float32, device=DEV)
        self.t = self.buf[guard:guard + self.n].view(*shape)

    def guards_intact(self) -> bool:
        b = self.buf.cpu().numpy()
        return bool(np.all(np.isnan(b[:self.guard])) and np.all(np.isnan(b[self.guard + self.n:])))


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
