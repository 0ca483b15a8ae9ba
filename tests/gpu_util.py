"""Helpers of the GPU parity tests: host <-> device copies and the parity tolerances.

The stated bar of the row-softmax family is max |error| <= 1e-5 on fp32 outputs, 2e-2
relative on bf16-stored outputs and 1e-4 relative on the mean loss. How each kind of output
is held to it:

* Outputs that never change sign and carry no cancellation -- softmax probabilities, and
  every non-target entry of a cross-entropy gradient row (s p_j / n_r) -- are compared
  element by element, relative to the oracle, with no floor but fp32 underflow:
  |g - o| <= r * max(|o|, 2^-100). r is 2^-7 for bf16 storage: one round-to-nearest-even to
  8 significant bits errs by at most 2^-8 relative, and the fp32 arithmetic before it by
  about 1e-5, so 2^-7 holds both with a factor two to spare and is tighter than 2e-2. For
  fp32 storage r is 1e-5 (on top of the 1e-5 absolute bound): the exponent argument
  x log2e - c, up to 2^7 in magnitude, is held in fp32 (half an ulp there is 2^-18, 2.6e-6
  in the result); the kernels round it twice at that magnitude and add the row sum's error,
  about 6.5e-6 at worst on the fp32 benchmark rows. 2^-100 is where fp32 results stop
  having relative precision to spare (results under 2^-126 are subnormal).
* The target entry of a cross-entropy gradient row, s (p_t - 1) / n_r, cancels when p_t is
  near 1, so it also gets an absolute allowance: p_t carries a relative error of about
  1e-6 in fp32 (the row sum, the exponential, the division), which (p_t - 1) keeps as an
  absolute error; 2^-18 |s| / n_r (3.8e-6 |s| / n_r) covers it. An entry that is exactly
  zero in exact arithmetic (a one-column row: p_t = 1) is held to that allowance too.
* Outputs that do cross zero (the softmax backward y (dy - s), layer norm, the block-sparse
  backward) follow the bar's 2e-2 relative with the denominator floored at 2^-7 of the
  row's largest |oracle| value (a relative test is meaningless where the result crosses
  zero); a caller may add an absolute allowance it derives from the fp32 arithmetic.
* Row losses (fp32) within 1e-4 relative with a 1e-5 floor; the reduced loss within 1e-4
  relative plus 1e-5 (1e-5 per row for a sum: a sum of losses that are 0 in exact
  arithmetic, e.g. one-column rows, is a few fp32 roundings away from 0).
"""
from __future__ import annotations

import numpy as np
import torch

import synth

FP32_ABS = 1e-5
FP32_REL = 1e-5
BF16_REL = 2e-2
BF16_ROUND = 2.0 ** -7
BF16_FLOOR = 2.0 ** -7
UNDERFLOW = 2.0 ** -100
TARGET_ABS = 2.0 ** -18
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


def check_bf16(gpu: np.ndarray, want: np.ndarray, what: str, abs_allow=0.0) -> float:
    """bf16 outputs that may cross zero, against float64 rows: |g - o| <= 2e-2 *
    max(|o|, 2^-7 max_j |o_ij|) + abs_allow. Returns the worst error over its bound."""
    g = widen(gpu)
    assert g.shape == want.shape, f"{what}: shape {g.shape} vs {want.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    floor = BF16_FLOOR * np.max(np.abs(want), axis=-1, keepdims=True)
    bound = BF16_REL * np.maximum(np.abs(want), floor) + abs_allow
    err = np.abs(g - want)
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: element {tuple(int(k) for k in i)} = {g[i]!r} vs "
                             f"{want[i]!r} (error {err[i]:.3e} > bound {bound[i]:.3e})")
    return worst


def check_output(gpu: np.ndarray, want: np.ndarray, what: str, allow=None) -> float:
    """allow: an absolute allowance per element for bf16 outputs (softmax_bwd_allow)."""
    if gpu.dtype == np.uint16:
        return check_bf16(gpu, want, what, abs_allow=0.0 if allow is None else allow)
    return check_fp32(gpu, want, what)


def softmax_bwd_allow(y: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """The absolute error fp32 arithmetic may leave in dx = y (dy - s), s = sum_j y_j dy_j:
    the dot product s carries at most d 2^-24 sum_j |y_j dy_j|, d the additions it is deep
    (at most 32 sequential per thread, then the reduction tree: d <= 32 + ceil(log2 N)), and
    y dy one rounding. Where dy_i is close to s that error is the whole result, however small
    the result is; elsewhere it is far below the relative bound."""
    yw, dw = widen(y), widen(dy)
    depth = 32 + int(np.ceil(np.log2(max(yw.shape[-1], 2))))
    mass = np.sum(np.abs(yw * dw), axis=-1, keepdims=True)
    return 2.0 ** -24 * np.abs(yw) * ((depth + 1) * mass + np.abs(dw))


def _check_rel(g: np.ndarray, want: np.ndarray, rel: float, extra, what: str) -> float:
    """|g - o| <= rel * max(|o|, 2^-100) + extra, element by element; worst error / bound."""
    err = np.abs(g - want)
    bound = rel * np.maximum(np.abs(want), UNDERFLOW)
    if extra is not None:
        bound = bound + extra
    ratio = err / bound
    worst = float(np.max(ratio)) if ratio.size else 0.0
    if not worst <= 1.0:  # (NaN fails too)
        i = np.unravel_index(int(np.argmax(np.where(np.isnan(ratio), np.inf, ratio))),
                             ratio.shape)
        raise AssertionError(f"{what}: element {tuple(int(k) for k in i)} = {g[i]!r} vs "
                             f"{want[i]!r} (error {err[i]:.3e} > bound {bound[i]:.3e})")
    return worst


def check_rel(gpu: np.ndarray, want: np.ndarray, what: str, roundings: int = 1,
              abs_tol: float = FP32_ABS) -> float:
    """Outputs with no cancellation (softmax probabilities, products such as element_mul):
    every element within 2^-7 per bf16 rounding on the way (or 1e-5 for fp32, plus the
    absolute bound abs_tol) of the oracle, relative; exact zeros (-inf inputs) must come
    back as zeros."""
    g = widen(gpu)
    assert g.shape == want.shape, f"{what}: shape {g.shape} vs {want.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    bf16 = gpu.dtype == np.uint16
    worst = _check_rel(g, want, roundings * BF16_ROUND if bf16 else FP32_REL, None, what)
    if not bf16:
        check_fp32(gpu, want, what, tol=abs_tol)
    return worst


def check_probs(gpu: np.ndarray, want: np.ndarray, what: str) -> float:
    """Softmax probabilities: check_rel with one rounding."""
    return check_rel(gpu, want, what)


def check_xent_grad(gpu: np.ndarray, want: np.ndarray, target: np.ndarray, V: int, n_r: float,
                    what: str, scale=None, ignore_index: int = -100, roundings: int = 1) -> float:
    """Cross-entropy gradient rows [k, V] against the oracle's float64 rows, every entry.

    target: the k rows' targets; n_r: the gradient's divisor (n for the mean reduction, 1
    for sum / none); scale: the upstream gradient (None, a number, or one value per row).
    Non-target entries: relative, 2^-7 (bf16) or 1e-5 (fp32), floored only at fp32
    underflow; the target entry: the same plus 2^-18 |s| / n_r for the cancellation in
    p_t - 1. Rows with no gradient (ignored or out-of-range targets) must be exactly zero.
    fp32 rows are also held to the 1e-5 absolute bound (scaled by max(1, |s|)). roundings:
    bf16 roundings on the way (2 when a second pass scales a stored gradient).
    Returns the worst error over its bound."""
    g = widen(gpu)
    k = want.shape[0]
    assert g.shape == want.shape == (k, V), f"{what}: shapes {g.shape} vs {want.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    t = np.asarray(target, dtype=np.int64)
    assert t.shape == (k,), f"{what}: {t.shape[0]} targets for {k} rows"
    s = np.ones(k) if scale is None else np.broadcast_to(
        np.abs(np.asarray(scale, dtype=np.float64)), (k,)).astype(np.float64)
    live = (t != ignore_index) & (t >= 0) & (t < V)
    dead = np.flatnonzero(~live)
    if dead.size:
        assert np.all(g[dead] == 0.0), f"{what}: rows without a gradient must be exactly zero"
        assert np.all(want[dead] == 0.0), f"{what}: oracle rows without a gradient"
    bf16 = gpu.dtype == np.uint16
    rel = roundings * BF16_ROUND if bf16 else FP32_REL
    extra = np.zeros_like(want)
    rows = np.flatnonzero(live)
    extra[rows, t[rows]] = TARGET_ABS * s[rows] / float(n_r)
    worst = _check_rel(g, want, rel, extra, what)
    if not bf16:
        check_fp32(gpu, want, what, tol=FP32_ABS * max(1.0, float(np.max(s)) if k else 1.0))
    return worst


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
