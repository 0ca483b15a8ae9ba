"""Helpers of the GPU parity tests: host <-> device copies and the parity tolerances.

Tolerances (from the stated bar of the row-softmax family):
  * fp32 outputs: max |gpu - oracle| <= 1e-5 over the compared tensor;
  * bf16-stored outputs: 2e-2 relative, elementwise, with the denominator floored at
    2^-7 times the row's largest |oracle| value (a relative test is meaningless near zero,
    where dx = y (dy - s) and (softmax - onehot) cross it) and at 5e-5 (so that an output
    that is exactly 0 in exact arithmetic, such as every entry of a one-column row, may
    carry the 1e-7-level residue of the fp32 arithmetic before its bf16 rounding);
  * mean loss: 1e-4 relative (+1e-5, and 1e-5 per row for a sum); row losses (fp32): 1e-4
    relative with a 1e-5 floor.
"""
from __future__ import annotations

import numpy as np
import torch

import synth

FP32_ABS = 1e-5
BF16_REL = 2e-2
BF16_FLOOR = 2.0 ** -7
BF16_ABS_FLOOR = 5e-5
MEAN_REL = 1e-4


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 (bf16 bits) -> bfloat16 tensor; float32 -> float32; int64 -> int64."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """bfloat16 -> uint16 bits; other dtypes as they are."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return synth.f32_from_bf16_bits(a).astype(np.float64)
    return a.astype(np.float64)


def check_fp32(gpu: np.ndarray, want: np.ndarray, what: str, tol: float = FP32_ABS) -> float:
    err = np.abs(widen(gpu) - want)
    worst = float(np.nanmax(err)) if err.size else 0.0
    assert np.all(np.isfinite(widen(gpu)) == np.isfinite(want)), f"{what}: finiteness differs"
    assert worst <= tol, f"{what}: max abs error {worst:.3e} > {tol:.1e}"
    return worst


def check_bf16(gpu: np.ndarray, want: np.ndarray, what: str) -> float:
    """Rows of bf16 bits against float64 rows; returns the worst scaled error."""
    g = widen(gpu)
    assert g.shape == want.shape, f"{what}: shape {g.shape} vs {want.shape}"
    floor = np.maximum(BF16_FLOOR * np.max(np.abs(want), axis=-1, keepdims=True), BF16_ABS_FLOOR)
    denom = np.maximum(np.abs(want), floor)
    with np.errstate(invalid="ignore", divide="ignore"):
        scaled = np.where(denom > 0, np.abs(g - want) / denom, np.abs(g - want))
    worst = float(np.max(scaled)) if scaled.size else 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert worst <= BF16_REL, f"{what}: worst scaled error {worst:.3e} > {BF16_REL:.0e}"
    return worst


def check_output(gpu: np.ndarray, want: np.ndarray, what: str) -> float:
    return check_bf16(gpu, want, what) if gpu.dtype == np.uint16 else check_fp32(gpu, want, what)


def check_losses(row_loss: np.ndarray, mean: float, want_rows: np.ndarray, want_mean: float,
                 what: str, mean_abs: float = 1e-5) -> None:
    """Row losses within 1e-4 relative (1e-5 floor); the reduced loss within 1e-4 relative
    plus `mean_abs` (a sum of row losses that are 0 in exact arithmetic, e.g. one-column
    rows, is a few fp32 roundings away from 0: the floor is 1e-5 per row it sums)."""
    err = np.abs(row_loss.astype(np.float64) - want_rows)
    tol = np.maximum(MEAN_REL * np.abs(want_rows), 1e-5)
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, f"{what}: row {bad[0]} loss {row_loss[bad[0]]} vs {want_rows[bad[0]]}"
    if np.isnan(want_mean):
        assert np.isnan(mean), f"{what}: mean {mean} should be NaN"
    else:
        assert abs(mean - want_mean) <= MEAN_REL * abs(want_mean) + mean_abs, \
            f"{what}: mean {mean} vs {want_mean}"
