"""Pins for the float64 oracle: checks against facts the oracle cannot produce by itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises ``AssertionError``
when the oracle disagrees with the fact it checks. The facts are

* invariants of the definitions (rows sum to 1, gradients sum to 0, shift
  invariance, exact zeros for ignored rows and -inf logits);
* closed forms (uniform rows give 1/N and loss log V, two columns give the
  logistic function, hand-worked examples in ``golden/worked_examples.json``);
* central finite differences of the oracle's own forward quantities;
* independent library routines evaluated in float64 (``torch.softmax``,
  ``torch.nn.functional.cross_entropy`` and autograd, ``scipy.special``).

``tests/test_oracle_pins.py`` runs every pin against the real oracle;
``tests/test_oracle_mutants.py`` builds copies of the oracle with planted
mistakes and requires each copy to fail at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.json")
_MATH = {"log": math.log, "exp": math.exp, "sqrt": math.sqrt, "inf": math.inf,
         "nan": math.nan, "__builtins__": {}}


def closed_form(expr) -> float:
    """Evaluate a closed-form expression such as "(1/4-1)/2" or "log(1+exp(2))"."""
    if isinstance(expr, (int, float)):
        return float(expr)
    return float(eval(str(expr), dict(_MATH)))  # noqa: S307 - fixtures are repository text


def as_input(rows, dtype: str) -> np.ndarray:
    """Fixture rows (numbers or "-inf") as the bytes the library receives."""
    vals = np.array([[closed_form(v) for v in r] for r in rows], dtype=np.float32)
    return synth.bf16_bits_from_f32(vals) if dtype == "bf16" else vals


def decode(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits or float32 values, widened exactly to float64."""
    if a.dtype == np.uint16:
        return synth.f32_from_bf16_bits(a).astype(np.float64)
    return a.astype(np.float64)


def _grid_rows(seed: int, M: int, N: int, step: float, lo: float, hi: float) -> np.ndarray:
    """Rows of values on a coarse grid (exact in bf16 and fp32)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    k = rng.integers(int(lo / step), int(hi / step) + 1, size=(M, N))
    return (k * step).astype(np.float32)


# --------------------------------------------------------------------------- softmax forward
def pin_softmax_rows_sum_to_one(o):
    for seed, (M, N, dtype, scale) in enumerate([(7, 1, "f32", 1.0), (9, 2, "bf16", 3.0),
                                                 (16, 7, "f32", 8.0), (8, 1000, "f32", 3.0),
                                                 (4, 4096, "bf16", 1.0)]):
        x = synth.random_rows(100 + seed, M, N, dtype=dtype, scale=scale)
        y = o.softmax_fwd(x)
        assert np.all(y >= 0), "softmax output must be non-negative"
        assert np.max(np.abs(y.sum(axis=1) - 1.0)) <= 1e-12, "softmax rows must sum to 1"


def pin_softmax_shift_invariance(o):
    base = _grid_rows(11, 6, 33, 1.0 / 8, -4.0, 4.0)
    for dtype, shifts in (("bf16", (-2.0, 0.5, 4.0)), ("f32", (-48.0, 0.5, 1024.0))):
        conv = synth.bf16_bits_from_f32 if dtype == "bf16" else (lambda a: a)
        y0 = o.softmax_fwd(conv(base))
        for c in shifts:
            shifted = (base + np.float32(c)).astype(np.float32)
            assert np.array_equal(shifted - np.float32(c), base), "shift must be exact"
            y1 = o.softmax_fwd(conv(shifted))
            assert np.all(np.isfinite(y1)), f"shift {c} must not overflow"
            assert np.max(np.abs(y1 - y0) / y0) <= 1e-12, f"softmax not invariant to shift {c}"


def pin_large_magnitude_rows(o):
    """The definitions depend only on x - max. fp32 rows moved by +-2^20 (exact for inputs on
    a 1/8 grid under 16 in magnitude) give the same softmax, -log p, row losses and gradient;
    rows of one value at +-1e30 give 1/N, -log p = log N and the loss log N (a loss formed as
    (m + log d) - x_t would lose log N to cancellation in float64 there)."""
    V = 40
    base = _grid_rows(14, 5, V, 1.0 / 8, -8.0, 8.0)
    t = np.array([0, 3, 39, 17, 20], dtype=np.int64)
    y0 = o.softmax_fwd(base)
    out0, nl0 = o.nll_fwd(base, t)
    g0, l0, _, _ = o.xent(base, t, V)
    for c in (2.0 ** 20, -(2.0 ** 20)):
        sh = (base + np.float32(c)).astype(np.float32)
        assert np.array_equal(sh - np.float32(c), base), "shift must be exact"
        assert np.max(np.abs(o.softmax_fwd(sh) - y0) / y0) <= 1e-12, f"softmax, shift {c}"
        out1, nl1 = o.nll_fwd(sh, t)
        assert np.max(np.abs(out1 - out0)) <= 1e-12 * np.max(out0), f"-log p, shift {c}"
        g1, l1, _, _ = o.xent(sh, t, V)
        assert np.max(np.abs(l1 - l0)) <= 1e-12 * np.max(l0), f"row losses, shift {c}"
        assert np.max(np.abs(g1 - g0)) <= 1e-15, f"gradient, shift {c}"
    N = 5
    for c in (1e30, -1e30):
        x = np.full((2, N), c, dtype=np.float32)
        idx = np.array([1, 4], dtype=np.int64)
        assert np.max(np.abs(o.softmax_fwd(x) - 1.0 / N)) <= 1e-15, f"uniform row at {c}"
        out, _ = o.nll_fwd(x, idx)
        assert np.max(np.abs(out - math.log(N))) <= 1e-12, f"-log p of a uniform row at {c}"
        _, loss, _, _ = o.xent(x, idx, N)
        assert np.max(np.abs(loss - math.log(N))) <= 1e-12, f"loss of a uniform row at {c}"


def pin_softmax_uniform_row(o):
    for N in (1, 3, 1000, 4096):
        y = o.softmax_fwd(np.full((2, N), 7.25, dtype=np.float32))
        assert np.max(np.abs(y - 1.0 / N)) <= 1e-15 / N * 4, "a uniform row gives 1/N"


def pin_softmax_two_columns_logistic(o):
    x = _grid_rows(12, 50, 2, 1.0 / 16, -12.0, 12.0)
    y = o.softmax_fwd(x)
    xd = x.astype(np.float64)
    for i in range(x.shape[0]):
        a, b = xd[i]
        sig = 1.0 / (1.0 + math.exp(b - a))
        assert abs(y[i, 0] - sig) <= 1e-15 and abs(y[i, 1] - (1.0 - sig)) <= 1e-15


def pin_softmax_matches_libraries(o):
    import scipy.special
    import torch
    for seed, (M, N, dtype, scale) in enumerate([(5, 1000, "f32", 3.0), (6, 513, "bf16", 2.0),
                                                 (3, 4096, "bf16", 1.0)]):
        x = synth.random_rows(200 + seed, M, N, dtype=dtype, scale=scale)
        y = o.softmax_fwd(x)
        xd = decode(x)
        ref_t = torch.softmax(torch.from_numpy(xd), dim=1).numpy()
        ref_s = scipy.special.softmax(xd, axis=1)
        assert np.max(np.abs(y - ref_t)) <= 1e-15, "disagrees with torch.softmax (float64)"
        assert np.max(np.abs(y - ref_s)) <= 1e-15, "disagrees with scipy.special.softmax"


def pin_softmax_row_stride_and_padding(o):
    for dtype in ("f32", "bf16"):
        padded = synth.random_rows(300, 9, 100, ld=136, dtype=dtype, scale=2.0)
        dense = np.ascontiguousarray(padded[:, :100])
        y_p = o.softmax_fwd(padded, n_cols=100)
        y_d = o.softmax_fwd(dense)
        assert np.all(np.isfinite(y_p)), "padding (NaN) must never be read"
        assert np.array_equal(y_p, y_d), "strided rows must give the dense result"


def pin_softmax_neg_inf_entries(o):
    x = synth.random_rows(301, 4, 64, dtype="f32", scale=2.0)
    x[:, ::3] = -np.inf
    y = o.softmax_fwd(x)
    assert np.all(y[:, ::3] == 0.0), "-inf logits get probability exactly 0"
    assert np.max(np.abs(y.sum(axis=1) - 1.0)) <= 1e-12
    finite = np.ascontiguousarray(x[:, [j for j in range(64) if j % 3]])
    assert np.max(np.abs(o.softmax_fwd(finite) - y[:, [j for j in range(64) if j % 3]])) <= 1e-16


# --------------------------------------------------------------------------- softmax backward
def pin_softmax_bwd_rows_sum_to_zero(o):
    # Dyadic probability rows sum to exactly 1, so each dx row sums to 0 up to rounding.
    y = np.array([[0.5, 0.25, 0.125, 0.125], [0.25, 0.25, 0.25, 0.25], [1.0, 0.0, 0.0, 0.0]],
                 dtype=np.float32)
    dy = synth.random_rows(400, 3, 4, dtype="f32", scale=3.0)
    dx = o.softmax_bwd(y, dy)
    assert np.max(np.abs(dx.sum(axis=1))) <= 1e-14, "dx rows must sum to 0 when sum(y) = 1"


def pin_softmax_direct_formula_small_inputs(o):
    """For |x| < 10 the formula without the max shift, exp(x) / sum(exp(x)), is accurate in
    float64: the oracle's shifted form must agree with it to 1e-14 relative."""
    x = synth.random_rows(1050, 20, 300, dtype="f32", scale=3.0)
    x = np.clip(x, -9.5, 9.5).astype(np.float32)
    e = np.exp(decode(x))
    direct = e / e.sum(axis=1, keepdims=True)
    y = o.softmax_fwd(x)
    assert np.max(np.abs(y - direct) / direct) <= 1e-14


def pin_softmax_bwd_jacobian(o):
    """Brute force on tiny rows: dx = J^T dy with J = diag(y) - y y^T."""
    for N in (1, 2, 3, 5, 8):
        y = synth.random_rows(1060 + N, 4, N, dtype="f32", scale=1.0)
        y = np.abs(y) + np.float32(0.1)
        y = (y / y.sum(axis=1, keepdims=True)).astype(np.float32)
        dy = synth.random_rows(1070 + N, 4, N, dtype="f32", scale=1.0)
        dx = o.softmax_bwd(y, dy)
        yd, dyd = decode(y), decode(dy)
        for i in range(4):
            J = np.diag(yd[i]) - np.outer(yd[i], yd[i])
            assert np.max(np.abs(dx[i] - J.T @ dyd[i])) <= 1e-15, f"N={N} row {i}"


def pin_softmax_bwd_finite_differences(o):
    # phi(x) = sum_j softmax(x)_j dy_j; its gradient is the backward of softmax at y = softmax(x).
    x = _grid_rows(13, 3, 6, 1.0 / 4, -2.0, 2.0)
    dy = _grid_rows(14, 3, 6, 1.0 / 4, -2.0, 2.0)
    h = 2.0 ** -14
    y = o.softmax_fwd(x)
    dx = o.softmax_bwd(y.astype(np.float32), dy)
    for i in range(x.shape[0]):
        for k in range(x.shape[1]):
            xp = x[i:i + 1].copy()
            xm = x[i:i + 1].copy()
            xp[0, k] += np.float32(h)
            xm[0, k] -= np.float32(h)
            fd = ((o.softmax_fwd(xp) - o.softmax_fwd(xm)) @ dy[i].astype(np.float64))[0] / (2 * h)
            # y is rounded to fp32 before the backward: allow that rounding (~1e-7 relative).
            assert abs(fd - dx[i, k]) <= 2e-6 * max(1.0, np.max(np.abs(dx[i]))), \
                f"softmax backward disagrees with finite differences at ({i},{k})"


def pin_softmax_bwd_matches_torch(o):
    import torch
    for seed, (M, N, dtype) in enumerate([(4, 300, "f32"), (5, 4096, "bf16"), (3, 7, "bf16")]):
        y = synth.random_rows(500 + seed, M, N, dtype=dtype, scale=0.2)
        dy = synth.random_rows(600 + seed, M, N, dtype=dtype, scale=1.0)
        dx = o.softmax_bwd(y, dy)
        ref = torch._softmax_backward_data(torch.from_numpy(decode(dy)),
                                           torch.from_numpy(decode(y)), 1,
                                           torch.float64).numpy()
        assert np.max(np.abs(dx - ref)) <= 1e-13, "disagrees with torch softmax backward (float64)"


def pin_softmax_bwd_row_strides(o):
    y = synth.random_rows(700, 5, 50, ld=64, dtype="bf16", scale=0.3)
    dy = synth.random_rows(701, 5, 50, ld=80, dtype="bf16", scale=1.0)
    dx = o.softmax_bwd(y, dy, n_cols=50)
    dense = o.softmax_bwd(np.ascontiguousarray(y[:, :50]), np.ascontiguousarray(dy[:, :50]))
    assert np.all(np.isfinite(dx)) and np.array_equal(dx, dense), "row strides / padding"


# --------------------------------------------------------------------------- cross-entropy
def pin_xent_uniform_logits_loss_is_log_v(o):
    with open(GOLDEN) as f:
        lnv = json.load(f)["lnV"]["values"]
    for V_str, expect in lnv.items():
        V = int(V_str)
        assert abs(math.log(V) - expect) <= 1e-15 * expect
        x = np.full((3, V), -1.5, dtype=np.float32)
        t = np.array([0, V - 1, V // 2], dtype=np.int64)
        grad, loss, mean, (n, bad) = o.xent(x, t, V)
        assert n == 3 and bad == 0
        assert np.max(np.abs(loss - expect)) <= 1e-12 * expect, f"uniform logits: loss = log {V}"
        assert abs(mean - expect) <= 1e-12 * expect
        # all-equal rows: gradient (1/V - [j == t]) / n
        want = np.full(V, 1.0 / V / n)
        for r in range(3):
            w = want.copy()
            w[t[r]] = (1.0 / V - 1.0) / n
            assert np.max(np.abs(grad[r] - w)) <= 1e-15, "all-equal row gradient"


def pin_xent_loss_is_logsumexp_minus_target(o):
    import scipy.special
    x = synth.random_rows(800, 16, 3001, dtype="bf16", scale=4.0)
    t = synth.random_targets(801, 16, 3001, ignore_frac=0.25)
    n, _ = o.xent_count(t, 3001)
    _, loss = o.xent_rows(x, t, 3001, n, want_grad=False)
    xd = decode(x)
    for i in range(16):
        want = 0.0 if t[i] == -100 else scipy.special.logsumexp(xd[i]) - xd[i, t[i]]
        assert abs(loss[i] - want) <= 1e-12 * max(1.0, abs(want)), f"row {i} loss"


def pin_xent_matches_torch(o):
    import torch
    import torch.nn.functional as F
    for seed, (M, V, dtype, scale, ign, ii) in enumerate([
            (12, 1000, "f32", 3.0, 0.25, -100), (9, 513, "bf16", 2.0, 0.3, -100),
            (7, 64, "f32", 8.0, 0.3, 5)]):
        x = synth.random_rows(900 + seed, M, V, dtype=dtype, scale=scale)
        t = synth.random_targets(950 + seed, M, V, ignore_frac=ign, ignore_index=ii)
        grad, loss, mean, (n, bad) = o.xent(x, t, V, ignore_index=ii)
        xt = torch.from_numpy(decode(x)).requires_grad_(True)
        tt = torch.from_numpy(t)
        ref_mean = F.cross_entropy(xt, tt, ignore_index=ii, reduction="mean")
        ref_none = F.cross_entropy(xt.detach(), tt, ignore_index=ii, reduction="none").numpy()
        ref_mean.backward()
        assert n == int((t != ii).sum()) and bad == 0
        assert abs(mean - ref_mean.item()) <= 1e-13 * abs(ref_mean.item()), "mean loss vs torch"
        assert np.max(np.abs(loss - ref_none)) <= 1e-12, "row losses vs torch"
        assert np.max(np.abs(grad - xt.grad.numpy())) <= 1e-15, "gradient vs torch autograd"


def pin_xent_gradient_structure(o):
    x = synth.random_rows(1000, 10, 777, dtype="f32", scale=3.0)
    x[3, ::2] = -np.inf
    t = synth.random_targets(1001, 10, 777, ignore_frac=0.3)
    t[3] = 1  # a finite column of the half -inf row
    grad, loss, mean, (n, _) = o.xent(x, t, 777)
    for i in range(10):
        if t[i] == -100:
            assert np.all(grad[i] == 0.0) and not np.signbit(grad[i]).any(), "ignored row is +0"
            assert loss[i] == 0.0
        else:
            assert abs(grad[i].sum()) <= 1e-15 * 777, "gradient rows sum to 0"
            assert grad[i, t[i]] < 0 and np.all(np.delete(grad[i], t[i]) >= 0)
            assert loss[i] > 0
    assert np.all(grad[3, ::2] == 0.0), "-inf logits get exactly zero gradient"


def pin_xent_finite_differences(o):
    M, V = 5, 7
    x = _grid_rows(15, M, V, 1.0 / 4, -2.0, 2.0)
    t = np.array([3, -100, 0, 6, -100], dtype=np.int64)
    grad, _, _, (n, _) = o.xent(x, t, V)
    assert n == 3
    h = 2.0 ** -14
    for i in range(M):
        for j in range(V):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += np.float32(h)
            xm[i, j] -= np.float32(h)
            fd = (o.xent(xp, t, V, want_grad=False)[2] - o.xent(xm, t, V, want_grad=False)[2]) / (2 * h)
            assert abs(fd - grad[i, j]) <= 1e-8, f"gradient vs finite differences at ({i},{j})"


def pin_xent_count_and_mean(o):
    t = synth.random_targets(1100, 1000, 50, ignore_frac=0.37)
    t[5] = 50   # out of range, not ignored
    t[6] = -7   # out of range, not ignored
    n, bad = o.xent_count(t, 50)
    assert n == sum(1 for v in t.tolist() if v != -100) and bad == 2
    x = synth.random_rows(1101, 1000, 50, dtype="bf16", scale=2.0)
    grad, loss, mean, _ = o.xent(x, t, 50)
    assert abs(mean - math.fsum(loss.tolist()) / n) <= 1e-12 * abs(mean), "mean = fsum(loss)/n"
    for r in (5, 6):
        assert loss[r] == 0.0 and np.all(grad[r] == 0.0), "bad target rows are zero"
    all_ignored = np.full(4, -100, dtype=np.int64)
    g0, l0, m0, (n0, _) = o.xent(x[:4], all_ignored, 50)
    assert n0 == 0 and math.isnan(m0) and np.all(g0 == 0.0) and np.all(l0 == 0.0)


def pin_xent_row_subset_and_padding(o):
    x = synth.random_rows(1200, 20, 300, ld=333, dtype="f32", scale=4.0)
    t = synth.random_targets(1201, 20, 300, ignore_frac=0.2)
    g_all, l_all, _, (n, _) = o.xent(x, t, 300)
    assert np.all(np.isfinite(g_all)), "padding (NaN) must never be read"
    rows = np.array([19, 0, 7, 7, 13])
    g_sub, l_sub = o.xent_rows(x, t, 300, n, rows=rows)
    assert np.array_equal(g_sub, g_all[rows]) and np.array_equal(l_sub, l_all[rows])
    # a per-row upstream gradient belongs to the row, not to its place in the list
    s = np.arange(1.0, 21.0)
    g_none, _, _, _ = o.xent(x, t, 300, reduction="none", scale=s)
    g_sub, _ = o.xent_rows(x, t, 300, n, rows=rows, reduction="none", scale=s)
    assert np.array_equal(g_sub, g_none[rows])
    dense = np.ascontiguousarray(x[:, :300])
    g_d, l_d, _, _ = o.xent(dense, t, 300)
    assert np.array_equal(g_d, g_all) and np.array_equal(l_d, l_all)


# --------------------------------------------------------------------------- block-sparse backward
def _dense_from_blocks(a: np.ndarray, lay: dict, block: int) -> np.ndarray:
    """(Z, seq, seq) float64 matrix holding each listed block at its place, zeros elsewhere."""
    nb = lay["n_brows"]
    Z = a.shape[0]
    out = np.zeros((Z, nb * block, nb * block))
    lut = lay["lut"]
    for r in range(nb):
        size, off = lut[2 * r], lut[2 * r + 1]
        for k in range(size):
            bid, br, bc = lut[off + 4 * k: off + 4 * k + 3]
            blk = decode(a[:, bid * block * block:(bid + 1) * block * block]).reshape(Z, block, block)
            out[:, br * block:(br + 1) * block, bc * block:(bc + 1) * block] = blk
    return out


def pin_bsr_softmax_bwd_dense_equivalent(o):
    """A table listing every block of every block-row is the dense softmax backward (times
    scale) of the matrix those blocks tile."""
    for dtype, block in (("f32", 4), ("bf16", 8)):
        nb = 3
        rows, cols = np.nonzero(np.ones((nb, nb), dtype=bool))  # every block of the matrix
        lut = np.zeros(2 * nb + 4 * rows.size, dtype=np.int32)
        for k, (r, c) in enumerate(zip(rows, cols)):
            lut[2 * nb + 4 * k: 2 * nb + 4 * k + 4] = (k, r, c, 0)
        for r in range(nb):
            lut[2 * r] = nb
            lut[2 * r + 1] = 2 * nb + 4 * nb * r
        lay = {"lut": lut, "n_brows": nb, "n_blocks": rows.size}
        per_z = rows.size * block * block
        y = synth.random_rows(2000, 2, per_z, dtype=dtype, scale=1.0)
        dy = synth.random_rows(2001, 2, per_z, dtype=dtype, scale=1.0)
        for scale in (1.0, 2.5):
            out = o.bsr_softmax_bwd(y, dy, lut, nb, block, scale)
            # dense reference through the (separately pinned) softmax backward
            Yd = _dense_from_blocks(y, lay, block)
            Dd = _dense_from_blocks(dy, lay, block)
            for z in range(2):
                ref = o.softmax_bwd(Yd[z].astype(np.float32) if dtype == "f32" else
                                    synth.bf16_bits_from_f32(Yd[z].astype(np.float32)),
                                    Dd[z].astype(np.float32) if dtype == "f32" else
                                    synth.bf16_bits_from_f32(Dd[z].astype(np.float32))) * scale
                for k, (r, c) in enumerate(zip(rows, cols)):
                    blk = out[z, k * block * block:(k + 1) * block * block].reshape(block, block)
                    want = ref[r * block:(r + 1) * block, c * block:(c + 1) * block]
                    assert np.max(np.abs(blk - want)) <= 1e-14, f"{dtype} block ({r},{c}) scale {scale}"


def pin_bsr_softmax_bwd_matches_torch_masked(o):
    """A causal local + global layout: every listed row equals the masked dense formula
    y * (dy - sum(y dy)) * scale computed by torch (zeros outside the layout add nothing);
    unlisted storage is untouched; reordering a block-row's table entries changes nothing."""
    import torch
    import synth as sy
    block, nb = 4, 6
    lay = sy.bsr_layout(nb, local=2, stride=3)
    per_z = lay["n_blocks"] * block * block
    y = synth.random_rows(2010, 3, per_z + 16, dtype="f32", scale=1.0)  # 16 spare elements
    dy = synth.random_rows(2011, 3, per_z + 16, dtype="f32", scale=1.0)
    out = o.bsr_softmax_bwd(y, dy, lay["lut"], nb, block, 0.75)
    Y = torch.from_numpy(_dense_from_blocks(y, lay, block))
    D = torch.from_numpy(_dense_from_blocks(dy, lay, block))
    ref = (Y * (D - (Y * D).sum(-1, keepdim=True)) * 0.75).numpy()
    got = _dense_from_blocks(out, lay, block)
    mask = np.kron(lay["layout"], np.ones((block, block), dtype=bool))
    assert np.max(np.abs(got[:, mask] - ref[:, mask])) <= 1e-14, "listed rows vs torch"
    assert np.array_equal(out[:, per_z:], decode(dy)[:, per_z:]), "storage past the blocks"
    lut2 = lay["lut"].copy()
    for r in range(nb):  # reverse each block-row's entry order
        size, off = lut2[2 * r], lut2[2 * r + 1]
        ent = lut2[off: off + 4 * size].reshape(size, 4)[::-1].copy()
        lut2[off: off + 4 * size] = ent.reshape(-1)
    out2 = o.bsr_softmax_bwd(y, dy, lut2, nb, block, 0.75)
    assert np.max(np.abs(out2 - out)) <= 1e-13, "table order within a block-row (sum order only)"


# --------------------------------------------------------------------------- negative log-softmax
def _nearest_bf16(v: float) -> float:
    """The bf16 value nearest to v (ties to even), by exact rational arithmetic."""
    from fractions import Fraction
    if v == 0.0 or not math.isfinite(v):
        return v
    q = Fraction(v)
    e = math.frexp(v)[1]  # v = f 2^e, 0.5 <= |f| < 1: 8 significant bits are steps of 2^(e-8)
    step = Fraction(2) ** (e - 8)
    k = q / step
    lo = math.floor(k)
    rem = k - lo
    n = lo + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else lo
    return float(n * step)


def pin_nll_uniform_and_two_columns(o):
    for N in (4, 1000, 128256):
        x = np.full((2, N), 0.75, dtype=np.float32)
        out, loss = o.nll_fwd(x, np.array([0, N - 1]))
        assert np.max(np.abs(out - math.log(N))) <= 1e-12 * math.log(N), "uniform row: log N"
    a = 3.0
    x = np.array([[0.0, a], [a, 0.0]], dtype=np.float32)
    out, loss = o.nll_fwd(x, np.array([1, 1]))
    l1 = math.log1p(math.exp(a))
    want = np.array([[l1, l1 - a], [l1 - a, l1]])
    assert np.max(np.abs(out - want)) <= 1e-14, "two columns: softplus"
    assert loss[0] == float(np.float32(l1 - a)) and loss[1] == float(np.float32(l1))


def pin_nll_matches_torch(o):
    import torch
    for seed, (M, N, dtype, scale) in enumerate([(9, 1000, "f32", 4.0), (6, 777, "bf16", 3.0)]):
        x = synth.random_rows(1600 + seed, M, N, dtype=dtype, scale=scale)
        idx = synth.random_targets(1650 + seed, M, N)
        out, loss = o.nll_fwd(x, idx)
        ref = -torch.log_softmax(torch.from_numpy(decode(x)), dim=1).numpy()
        assert np.max(np.abs(out - ref)) <= 1e-12, "-log_softmax vs torch"
        assert np.all(out >= 0.0)
        p = np.exp(-out)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12, "exp(-out) rows sum to 1"


def pin_nll_loss_is_the_stored_element(o):
    """The loss is the output at the row's index rounded to the element type (checked with
    an independent exact rounding), NaN for an index outside the row; padding is never read."""
    M, N, ld = 40, 300, 320
    for dtype in ("f32", "bf16"):
        x = synth.random_rows(1700, M, N, ld=ld, dtype=dtype, scale=3.0, pad_nan=True)
        idx = synth.random_targets(1701, M, N)
        idx[0] = N
        idx[1] = -1
        out, loss = o.nll_fwd(x, idx, n_cols=N)
        assert np.all(np.isfinite(out)), "padding (NaN) must never be read"
        assert math.isnan(loss[0]) and math.isnan(loss[1]), "index outside the row: NaN"
        for i in range(2, M):
            v = out[i, idx[i]]
            want = float(np.float32(v)) if dtype == "f32" else _nearest_bf16(v)
            assert loss[i] == want, f"{dtype} row {i}: loss {loss[i]!r} vs stored {want!r}"
        dense = np.ascontiguousarray(x[:, :N])
        out_d, loss_d = o.nll_fwd(dense, idx)
        assert np.array_equal(out_d, out)


# --------------------------------------------------------------------------- layer norm
def _ln_inputs(seed, M, N, dtype, ld=None, scale=2.0):
    x = synth.random_rows(seed, M, N, ld=ld, dtype=dtype, scale=scale, pad_nan=ld is not None)
    wb = synth.random_rows(seed + 1, 2, N, dtype=dtype, scale=1.0)
    return x, np.ascontiguousarray(wb[0]), np.ascontiguousarray(wb[1])


def pin_layernorm_matches_torch(o):
    import torch
    import torch.nn.functional as F
    for seed, (M, N, dtype, eps, ld) in enumerate([(9, 1000, "f32", 1e-5, None),
                                                   (7, 513, "bf16", 1e-6, 520),
                                                   (5, 64, "f32", 0.5, 70)]):
        x, w, b = _ln_inputs(1800 + 10 * seed, M, N, dtype, ld)
        dy = synth.random_rows(1805 + 10 * seed, M, N, dtype=dtype, scale=1.0)
        y, mean, rstd = o.layernorm_fwd(x, w, b, eps, n_cols=N)
        dx, dw, db = o.layernorm_bwd(dy, x, w, eps, n_cols=N)
        xt = torch.from_numpy(decode(x)[:, :N]).requires_grad_(True)
        wt = torch.from_numpy(decode(w)).requires_grad_(True)
        bt = torch.from_numpy(decode(b)).requires_grad_(True)
        ref = F.layer_norm(xt, (N,), wt, bt, eps)
        ref.backward(torch.from_numpy(decode(dy)))
        assert np.max(np.abs(y - ref.detach().numpy())) <= 1e-12, "y vs torch layer_norm"
        assert np.max(np.abs(dx - xt.grad.numpy())) <= 1e-12, "dx vs torch autograd"
        assert np.max(np.abs(dw - wt.grad.numpy())) <= 1e-12, "dw vs torch autograd"
        assert np.max(np.abs(db - bt.grad.numpy())) <= 1e-12, "db vs torch autograd"
        xd = decode(x)[:, :N]
        assert np.max(np.abs(mean - xd.mean(axis=1))) <= 1e-12
        assert np.max(np.abs(rstd - 1 / np.sqrt(xd.var(axis=1) + eps))) <= 1e-9 * np.max(rstd)


def pin_layernorm_invariants(o):
    """With w = 1 and b = 0 every output row has mean 0 and mean square var / (var + eps);
    constant rows give y = b exactly and rstd = 1/sqrt(eps); the backward of w = 1 rows sums
    to 0 (and with eps = 0 is orthogonal to xhat); db is the exact column sum of dy."""
    M, N, eps = 6, 300, 1e-3
    x, _, b = _ln_inputs(1900, M, N, "f32", scale=3.0)
    ones = np.ones(N, dtype=np.float32)
    zeros = np.zeros(N, dtype=np.float32)
    y, mean, rstd = o.layernorm_fwd(x, ones, zeros, eps)
    var = decode(x).var(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) <= 1e-12
    assert np.max(np.abs((y ** 2).mean(axis=1) - var / (var + eps))) <= 1e-12
    c = np.full((2, N), 1.25, dtype=np.float32)
    yc, mc, rc = o.layernorm_fwd(c, ones, b, eps)
    assert np.all(yc == decode(b)[None, :]) and np.all(mc == 1.25)
    assert np.all(rc == 1.0 / math.sqrt(eps))
    dy = synth.random_rows(1901, M, N, dtype="f32", scale=1.0)
    dx, dw, db = o.layernorm_bwd(dy, x, ones, eps)
    xhat = (decode(x) - mean[:, None]) * rstd[:, None]
    assert np.max(np.abs(dx.sum(axis=1))) <= 1e-11, "w = 1: dx rows sum to 0"
    # with eps = 0 the output is scale invariant in x - mean: dx is orthogonal to xhat
    dx0, _, _ = o.layernorm_bwd(dy, x, ones, 0.0)
    _, m0, r0 = o.layernorm_fwd(x, ones, zeros, 0.0)
    xhat0 = (decode(x) - m0[:, None]) * r0[:, None]
    assert np.max(np.abs((dx0 * xhat0).sum(axis=1))) <= 1e-11, "eps = 0: dx orthogonal to xhat"
    assert all(db[j] == math.fsum(decode(dy)[:, j].tolist()) or
               abs(db[j] - math.fsum(decode(dy)[:, j].tolist())) <= 1e-14 for j in range(N))
    assert np.max(np.abs(dw - (decode(dy) * xhat).sum(axis=0))) <= 1e-12


def pin_layernorm_finite_differences(o):
    """The backward is the derivative of the forward: central differences of
    sum(g * y) with respect to every x, w and b element."""
    M, N, eps = 3, 5, 0.125
    x = _grid_rows(1950, M, N, 1.0 / 4, -2.0, 2.0)
    wb = _grid_rows(1951, 2, N, 1.0 / 4, -1.5, 1.5)
    w, b = np.ascontiguousarray(wb[0]), np.ascontiguousarray(wb[1])
    g = _grid_rows(1952, M, N, 1.0 / 8, -1.0, 1.0)
    dx, dw, db = o.layernorm_bwd(g, x, w, eps)
    h = 2.0 ** -14
    gd = g.astype(np.float64)

    def obj(xx, ww, bb):
        return float((o.layernorm_fwd(xx, ww, bb, eps)[0] * gd).sum())

    for i in range(M):
        for j in range(N):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += np.float32(h)
            xm[i, j] -= np.float32(h)
            fd = (obj(xp, w, b) - obj(xm, w, b)) / (2 * h)
            assert abs(fd - dx[i, j]) <= 1e-7, f"dx vs finite differences at ({i},{j})"
    for j in range(N):
        wp, wm = w.copy(), w.copy()
        wp[j] += np.float32(h)
        wm[j] -= np.float32(h)
        assert abs((obj(x, wp, b) - obj(x, wm, b)) / (2 * h) - dw[j]) <= 1e-7, f"dw {j}"
        bp, bm = b.copy(), b.copy()
        bp[j] += np.float32(h)
        bm[j] -= np.float32(h)
        assert abs((obj(x, w, bp) - obj(x, w, bm)) / (2 * h) - db[j]) <= 1e-7, f"db {j}"


# ------------------------------------------------------- reductions and upstream gradient
def pin_xent_reductions_finite_differences(o):
    """Each reduction's gradient, times its upstream value, is the derivative of that loss."""
    M, V = 5, 7
    x = _grid_rows(16, M, V, 1.0 / 4, -2.0, 2.0)
    t = np.array([3, -100, 0, 6, 2], dtype=np.int64)
    s = np.array([0.5, -2.0, 3.0, 1.25, -0.75])
    n = 4
    cases = [("none", s, lambda loss: float(np.dot(s, loss))),
             ("sum", -1.5, lambda loss: -1.5 * math.fsum(loss.tolist())),
             ("mean", 2.5, lambda loss: 2.5 * math.fsum(loss.tolist()) / n)]
    h = 2.0 ** -14
    for reduction, scale, objective in cases:
        grad, _, _, (nn, _) = o.xent(x, t, V, reduction=reduction, scale=scale)
        assert nn == n
        for i in range(M):
            for j in range(V):
                xp, xm = x.copy(), x.copy()
                xp[i, j] += np.float32(h)
                xm[i, j] -= np.float32(h)
                fp = objective(o.xent(xp, t, V, want_grad=False)[1])
                fm = objective(o.xent(xm, t, V, want_grad=False)[1])
                fd = (fp - fm) / (2 * h)
                assert abs(fd - grad[i, j]) <= 1e-8, f"{reduction}: gradient vs finite differences at ({i},{j})"


def pin_xent_reductions_match_torch(o):
    import torch
    import torch.nn.functional as F
    M, V = 11, 300
    x = synth.random_rows(1300, M, V, dtype="bf16", scale=3.0)
    t = synth.random_targets(1301, M, V, ignore_frac=0.3)
    s = synth.random_rows(1302, 1, M, dtype="f32", scale=2.0)[0].astype(np.float64)
    xt = torch.from_numpy(decode(x))
    tt = torch.from_numpy(t)
    # none: upstream gradient s_i on row i
    a = xt.clone().requires_grad_(True)
    ref = F.cross_entropy(a, tt, reduction="none")
    (ref * torch.from_numpy(s)).sum().backward()
    grad, loss, red, _ = o.xent(x, t, V, reduction="none", scale=s)
    assert red is None
    assert np.max(np.abs(loss - ref.detach().numpy())) <= 1e-12, "none: row losses vs torch"
    assert np.max(np.abs(grad - a.grad.numpy())) <= 1e-14, "none: gradient vs torch autograd"
    # sum: one upstream value for the scalar
    b = xt.clone().requires_grad_(True)
    ref = F.cross_entropy(b, tt, reduction="sum")
    (ref * -0.625).backward()
    grad, loss, red, _ = o.xent(x, t, V, reduction="sum", scale=-0.625)
    assert abs(red - ref.item()) <= 1e-13 * abs(ref.item()), "sum: loss vs torch"
    assert np.max(np.abs(grad - b.grad.numpy())) <= 1e-14, "sum: gradient vs torch autograd"
    # mean with an upstream value: torch's mean loss scaled
    c = xt.clone().requires_grad_(True)
    ref = F.cross_entropy(c, tt, reduction="mean")
    (ref * 3.0).backward()
    grad, _, red, _ = o.xent(x, t, V, reduction="mean", scale=3.0)
    assert abs(red - ref.item()) <= 1e-13 * abs(ref.item()), "mean: loss vs torch"
    assert np.max(np.abs(grad - c.grad.numpy())) <= 1e-14, "mean: gradient vs torch autograd"


def pin_xent_sum_is_exact_sum(o):
    t = synth.random_targets(1400, 700, 90, ignore_frac=0.2)
    x = synth.random_rows(1401, 700, 90, dtype="f32", scale=5.0)
    _, loss, red, (n, _) = o.xent(x, t, 90, reduction="sum", want_grad=False)
    assert abs(red - math.fsum(loss.tolist())) <= 1e-12 * abs(red), "sum = fsum(row losses)"
    _, _, mean, _ = o.xent(x, t, 90, want_grad=False)
    assert abs(mean * n - red) <= 1e-12 * abs(red), "sum = n * mean"
    assert o.sum(np.zeros(0)) == 0.0


def pin_element_mul_products(o):
    """Products with scales of few significant bits are exact in float64, so they must match
    the decoded inputs times the scale bit for bit; padding columns are never read."""
    M, V, ld = 6, 257, 300
    for dtype in ("bf16", "f32"):
        x = synth.random_rows(1500, M, V, ld=ld, dtype=dtype, scale=4.0)
        xd = decode(x)[:, :V]
        rows = np.array([2.0, 0.5, -1.0, 1.0, 0.0, -3.0])
        out = o.element_mul(x, rows, n_cols=V)
        assert np.array_equal(out, xd * rows[:, None]), f"{dtype}: per-row products"
        assert np.array_equal(out[3], xd[3]) and np.array_equal(out[2], -xd[2])
        assert np.all(out[4] == 0.0)
        out = o.element_mul(x, 0.25, n_cols=V)
        assert np.array_equal(out, xd * 0.25), f"{dtype}: one scale for every row"
        assert np.all(np.isfinite(out)), "padding (NaN) must never be read"


# --------------------------------------------------------------------------- worked examples
def pin_golden_worked_examples(o):
    with open(GOLDEN) as f:
        gold = json.load(f)
    for case in gold["softmax_fwd"]:
        y = o.softmax_fwd(as_input(case["x"], case["dtype"]))
        want = np.array([[closed_form(v) for v in r] for r in case["y"]])
        assert np.max(np.abs(y - want)) <= 1e-15, case["name"]
    for case in gold["softmax_bwd"]:
        dx = o.softmax_bwd(as_input(case["y"], case["dtype"]), as_input(case["dy"], case["dtype"]))
        want = np.array([[closed_form(v) for v in r] for r in case["dx"]])
        assert np.max(np.abs(dx - want)) <= 1e-15, case["name"]
    for case in gold["xent"]:
        x = as_input(case["x"], case["dtype"])
        t = np.array(case["target"], dtype=np.int64)
        V = x.shape[1]
        grad, loss, mean, (n, bad) = o.xent(x, t, V, ignore_index=case["ignore_index"])
        assert n == case["n"] and bad == 0, case["name"]
        assert np.max(np.abs(loss - [closed_form(v) for v in case["loss"]])) <= 1e-15, case["name"]
        assert abs(mean - closed_form(case["mean"])) <= 1e-15, case["name"]
        want = np.array([[closed_form(v) for v in r] for r in case["grad"]])
        assert np.max(np.abs(grad - want)) <= 1e-15, case["name"]
    for case in gold["xent_reduced"]:
        x = as_input(case["x"], case["dtype"])
        t = np.array(case["target"], dtype=np.int64)
        V = x.shape[1]
        grad, loss, red, (n, bad) = o.xent(x, t, V, ignore_index=case["ignore_index"],
                                           reduction=case["reduction"], scale=case["scale"])
        assert n == case["n"] and bad == 0, case["name"]
        assert np.max(np.abs(loss - [closed_form(v) for v in case["loss"]])) <= 1e-15, case["name"]
        if case["reduced"] is None:
            assert red is None, case["name"]
        else:
            assert abs(red - closed_form(case["reduced"])) <= 1e-15, case["name"]
        want = np.array([[closed_form(v) for v in r] for r in case["grad"]])
        assert np.max(np.abs(grad - want)) <= 1e-15, case["name"]
    for case in gold["element_mul"]:
        x = as_input(case["x"], case["dtype"])
        out = o.element_mul(x, case["scale"], n_cols=case["n_cols"])
        want = np.array([[closed_form(v) for v in r] for r in case["out"]])
        assert np.array_equal(out, want), case["name"]
    for case in gold["nll_fwd"]:
        x = as_input(case["x"], case["dtype"])
        out, loss = o.nll_fwd(x, np.array(case["idx"], dtype=np.int64))
        want = np.array([[closed_form(v) for v in r] for r in case["out"]])
        fin = np.isfinite(want)
        assert np.array_equal(np.isfinite(out), fin), case["name"]
        assert np.max(np.abs(out[fin] - want[fin])) <= 1e-14 and np.all(out[~fin] == want[~fin]), case["name"]
        wl = np.array([closed_form(v) for v in case["loss"]])
        assert np.array_equal(np.isnan(loss), np.isnan(wl)), case["name"]
        ok = ~np.isnan(wl)
        assert np.max(np.abs(loss[ok] - wl[ok])) <= 2e-7 * np.max(np.abs(wl[ok])), case["name"]
    for case in gold["layernorm"]:
        x = as_input(case["x"], case["dtype"])
        w = as_input([case["w"]], case["dtype"])[0]
        b = as_input([case["b"]], case["dtype"])[0]
        dy = as_input(case["dy"], case["dtype"])
        y, mean, rstd = o.layernorm_fwd(x, w, b, case["eps"])
        dx, dw, db = o.layernorm_bwd(dy, x, w, case["eps"])
        for got, key in ((y, "y"), (dx, "dx")):
            want = np.array([[closed_form(v) for v in r] for r in case[key]])
            assert np.max(np.abs(got - want)) <= 1e-15, f"{case['name']}: {key}"
        for got, key in ((mean, "mean"), (rstd, "rstd"), (dw, "dw"), (db, "db")):
            want = np.array([closed_form(v) for v in case[key]])
            assert np.max(np.abs(got - want)) <= 1e-15, f"{case['name']}: {key}"
    for case in gold["bsr_softmax_bwd"]:
        y = as_input(case["y"], case["dtype"])
        dy = as_input(case["dy"], case["dtype"])
        out = o.bsr_softmax_bwd(y, dy, np.array(case["lut"], dtype=np.int32), case["n_brows"],
                                case["block"], case["scale"])
        want = np.array([[closed_form(v) for v in r] for r in case["out"]])
        assert np.max(np.abs(out - want)) <= 1e-15, case["name"]


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
