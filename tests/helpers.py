"""Shared test helpers: host <-> device transfer of bf16 bit patterns and the
error metric used by the parity gates."""
from __future__ import annotations

import numpy as np

from canvas_attention_amd import synth

# Tolerances of the parity gates: per-row normalised max error
#   err = max over rows (b, i, h) of  max_d |gpu - oracle| / max_d |oracle|
# (elementwise relative error is ill-posed: a weighted sum of N(0,1) values has
# components arbitrarily close to zero).
TOL_BF16 = 2e-2
TOL_F32 = 1e-5


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host_bits(t) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_host_f64(t) -> np.ndarray:
    a = to_host_bits(t)
    return synth.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def row_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Per-row normalised max error over the last axis."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


def sample_rows(rng, B, Nc, Hq, n):
    """(b, i, h) triples: all corners plus n random rows."""
    rows = {(b, i, h) for b in (0, B - 1) for i in (0, Nc - 1) for h in (0, Hq - 1)}
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(Nc)), int(rng.integers(Hq))))
    return np.array(sorted(rows), np.int32)
