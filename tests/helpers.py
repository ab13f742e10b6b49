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

# fp8 (e4m3 inputs).  The kernel rounds each softmax weight p_j to e4m3 (round to
# nearest even, 3 mantissa bits), a relative error |d_j| <= 2^-4 (rms 2^-4/sqrt(6)
# ~ 0.026 for mantissas spread over a binade), and uses the rounded weights for
# both the weighted sum of values and the row sum.  With w = p / sum p and
# dbar = sum_j w_j d_j the output error is sum_j w_j d_j (v_j - out) / (1 + dbar).
# Hence:
#   * elementwise, for every output: |gpu - ref| <= 2^-4 / (1 - 2^-4) * (A + |ref|)
#     plus the bf16 rounding of the partial and final rows (2^-9 each), with
#     A = sum_j w_j |v_j| -- attention over |V|, which the oracle computes from the
#     value bytes with the sign bit cleared;
#   * statistically, the error has an rms of ~0.026 times that of the output for
#     values independent of the weights: TOL_FP8_RMS bounds the ratio of the two
#     over all checked elements, and TOL_FP8_ROW the per-row normalised error of
#     rows with at least 256 keys (a numpy model of the rounding gives a median of
#     0.027 and a maximum of 0.05 over 300 rows at 2k and 8k keys).
FP8_P_REL = 2.0 ** -4
TOL_FP8_RMS = 0.04
TOL_FP8_ROW = 0.1


# Measured parity errors of this session, printed in pytest's terminal summary
# (tests/conftest.py) so that each gate's margin is on record even under -q.
PARITY_RECORDS: list = []


def record(what: str, err: float, gate: float) -> float:
    """Log one measured error against its gate (under the current test's name)."""
    import os
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    PARITY_RECORDS.append((test, what, float(err), float(gate)))
    return float(err)


def to_dev(a: np.ndarray):
    """numpy -> GPU tensor: uint16 holds bf16 bits, uint8 holds e4m3 bytes."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda().view(torch.float8_e4m3fn)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host_bits(t) -> np.ndarray:
    import torch
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
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


def fp8_check(got: np.ndarray, ref: np.ndarray, ref_abs: np.ndarray, per_row: bool = True):
    """The fp8 gates above; ref_abs is the oracle's attention over |V|.  Returns
    (per-row normalised error, rms ratio)."""
    err = np.abs(got - ref)
    rel = FP8_P_REL / (1.0 - FP8_P_REL)
    bound = (rel + 2.0 ** -9 + 1e-4) * ref_abs + (rel + 2.0 ** -8) * np.abs(ref) + 1e-6
    worst = float((err - bound).max())
    assert worst <= 0, f"elementwise bound exceeded by {worst:.3e}"
    rms = float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300)))
    assert rms <= TOL_FP8_RMS, f"rms ratio {rms:.3e} > {TOL_FP8_RMS}"
    rerr = row_err(got, ref)
    if per_row:
        assert rerr <= TOL_FP8_ROW, f"per-row error {rerr:.3e} > {TOL_FP8_ROW}"
    return rerr, rms


def sample_rows(rng, B, Nc, Hq, n):
    """(b, i, h) triples: all corners plus n random rows."""
    rows = {(b, i, h) for b in (0, B - 1) for i in (0, Nc - 1) for h in (0, Hq - 1)}
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(Nc)), int(rng.integers(Hq))))
    return np.array(sorted(rows), np.int32)
