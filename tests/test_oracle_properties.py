"""Property tests of the float64 oracle (CPU, Hypothesis): random shapes, shifts, -inf
patterns and ignore patterns, each checked against an identity that holds exactly in real
arithmetic and follows from the definitions the oracle restates:

* softmax (the fused-softmax tutorial page, its kernel): non-negative rows summing to 1,
  exact zeros at -inf, ratios exp(x_i - x_j), invariance under adding a constant to a row;
* softmax backward (the block-sparse softmax example page, its backward kernel with scale 1):
  sum_j dx_j = s (1 - sum_j y_j) with s = sum_j y_j dy_j, zeros where y is 0, linearity in dy;
* cross-entropy (the Liger-Kernel cross_entropy.py page, liger_cross_entropy_kernel and its
  forward): loss = logsumexp(x) - x_t >= 0, gradient rows summing to 0 with the sign pattern
  of p - onehot, ignored and out-of-range rows zero, n and the bad-target count, the mean;
* negative log-softmax (the fused-softmax page's log-softmax kernel): exp(-out) summing to
  1 per row, the gathered loss equal to the row's element at the index;
* layer norm (the layer-norm tutorial page, forward and backward): normalised rows of mean 0,
  db and dw the column sums of dy and dy * xhat, backward rows summing to 0 and their
  projection on xhat equal to eps rstd^3 sum_j dy_j w_j xhat_j.

Each planted mistake of the oracle's C source that touches these definitions (the mutants of
test_oracle_mutants.py) must fail these properties on their own, on fixed seeded cases.

Inputs lie on a grid of multiples of 1/8 in [-16, 16) and shifts are integers in [-8, 8), so
every input and every shifted input is exact in bf16 and fp32; rows that are entirely -inf,
and -inf target logits, are outside the contract and are not drawn.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import synth

# derandomized: every run draws the same cases (XR_PROPERTY_EXAMPLES draws more of them)
SETTINGS = settings(max_examples=int(os.environ.get("XR_PROPERTY_EXAMPLES", "40")),
                    deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def encode(values: np.ndarray, dtype: str) -> np.ndarray:
    """float64 grid values (exact in both types) as the oracle's input type."""
    f = values.astype(np.float32)
    return synth.bf16_bits_from_f32(f) if dtype == "bf16" else f


@st.composite
def grid_rows(draw, max_m=5, max_n=200, neg_inf=True):
    M = draw(st.integers(1, max_m))
    N = draw(st.integers(1, max_n))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    x = rng.integers(-128, 128, size=(M, N)).astype(np.float64) / 8.0
    if neg_inf and draw(st.booleans()):
        frac = draw(st.sampled_from([0.1, 0.5, 0.9, 1.0]))
        mask = rng.random((M, N)) < frac
        keep = rng.integers(0, N, size=M)  # one finite entry per row at least
        mask[np.arange(M), keep] = False
        x[mask] = -np.inf
    dtype = draw(st.sampled_from(["f32", "bf16"]))
    return x, dtype, rng


def check_softmax(orc, x, dtype, shift):
    y = orc.softmax_fwd(encode(x, dtype))
    assert np.all(y >= 0)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert np.all(y[np.isneginf(x)] == 0)
    # ratios: y_i / y_j = exp(x_i - x_j) between finite entries of a row
    for i in range(x.shape[0]):
        fin = np.flatnonzero(np.isfinite(x[i]))
        a, b = fin[0], fin[-1]
        np.testing.assert_allclose(y[i, a] / y[i, b], np.exp(x[i, a] - x[i, b]), rtol=1e-13)
    # adding a constant to a row changes nothing: x + c is exact, so are all differences
    ys = orc.softmax_fwd(encode(x + shift, dtype))
    assert np.array_equal(ys, y)


@SETTINGS
@given(grid_rows(), st.integers(-8, 7))
def test_softmax_properties(orc, rows, shift):
    x, dtype, _ = rows
    check_softmax(orc, x, dtype, shift)


def check_softmax_bwd(orc, x, dtype, rng):
    # y: softmax outputs rounded to the type, with some exact zeros
    y = orc.softmax_fwd(encode(x, dtype))
    y[rng.random(y.shape) < 0.2] = 0.0
    y_in = encode(y, dtype)
    yv = synth.f32_from_bf16_bits(y_in).astype(np.float64) if dtype == "bf16" \
        else y_in.astype(np.float64)
    dy = rng.integers(-64, 64, size=x.shape).astype(np.float64) / 8.0
    dx = orc.softmax_bwd(y_in, encode(dy, dtype))
    s = (yv * dy).sum(axis=1)
    scale = 1.0 + np.abs(yv * dy).sum(axis=1) + np.abs(s)
    np.testing.assert_allclose(dx.sum(axis=1), s * (1.0 - yv.sum(axis=1)), rtol=0,
                               atol=float(np.max(scale)) * 1e-13 * x.shape[1])
    assert np.all(dx[yv == 0] == 0)
    # twice dy (exact): twice dx, bit for bit
    dx2 = orc.softmax_bwd(y_in, encode(2 * dy, dtype))
    assert np.array_equal(dx2, 2 * dx)
    # each entry: y_j (dy_j - s)
    np.testing.assert_allclose(dx, yv * (dy - s[:, None]), rtol=1e-12,
                               atol=1e-13 * float(np.max(scale)))


@SETTINGS
@given(grid_rows(neg_inf=False), st.integers(0, 2 ** 32 - 1))
def test_softmax_bwd_properties(orc, rows, seed):
    x, dtype, _ = rows
    check_softmax_bwd(orc, x, dtype, np.random.default_rng(seed))


@st.composite
def xent_case(draw):
    x, dtype, rng = draw(grid_rows(max_m=6, max_n=150))
    M, V = x.shape
    kinds = draw(st.lists(st.sampled_from(["valid", "ignore", "low", "high"]), min_size=M,
                          max_size=M))
    t = np.empty(M, dtype=np.int64)
    for i, k in enumerate(kinds):
        if k == "valid":
            fin = np.flatnonzero(np.isfinite(x[i]))  # the target logit is finite
            t[i] = int(rng.choice(fin))
        else:
            t[i] = {"ignore": -100, "low": -3, "high": V + 2}[k]
    return x, dtype, t


def logsumexp(row: np.ndarray) -> float:
    m = np.max(row)
    return float(m + np.log(np.sum(np.exp(row - m))))


def check_xent(orc, x, dtype, t, shift):
    M, V = x.shape
    grad, loss, mean, (n, bad) = orc.xent(encode(x, dtype), t, V)
    valid = (t >= 0) & (t < V)
    assert n == int(np.sum(t != -100))
    assert bad == int(np.sum((t != -100) & ~valid))
    for i in range(M):
        if not valid[i]:
            assert np.all(grad[i] == 0) and loss[i] == 0
            continue
        want = logsumexp(x[i]) - x[i, t[i]]
        assert loss[i] >= 0
        np.testing.assert_allclose(loss[i], want, rtol=1e-13, atol=1e-13)
        g = grad[i]
        assert abs(g.sum()) <= 1e-13 / n
        others = np.delete(g, t[i])
        assert np.all(others >= 0) and g[t[i]] <= 0
        assert np.all(g[np.isneginf(x[i])] == 0)
        # the non-target entries are p_j / n
        p = np.exp(x[i] - logsumexp(x[i]))
        np.testing.assert_allclose(np.delete(g * n, t[i]), np.delete(p, t[i]), rtol=1e-12,
                                   atol=1e-300)
    if n == 0:
        assert np.isnan(mean)
    else:
        np.testing.assert_allclose(mean, loss.sum() / n, rtol=1e-14)
    # a constant added to every logit changes neither the loss nor the gradient
    grad_s, loss_s, _, _ = orc.xent(encode(x + shift, dtype), t, V)
    np.testing.assert_allclose(loss_s, loss, rtol=0, atol=1e-12)
    np.testing.assert_allclose(grad_s, grad, rtol=1e-12, atol=1e-300)
    # the sum reduction's gradient is n times the mean's
    grad_sum, _, total, _ = orc.xent(encode(x, dtype), t, V, reduction="sum")
    np.testing.assert_allclose(grad_sum, grad * max(n, 1), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(total, loss.sum(), rtol=1e-14)


@SETTINGS
@given(xent_case(), st.integers(-8, 7))
def test_xent_properties(orc, case, shift):
    x, dtype, t = case
    check_xent(orc, x, dtype, t, shift)


def check_nll(orc, x, dtype, rng):
    M, N = x.shape
    idx = rng.integers(-2, N + 2, size=M)
    idx[0] = N  # the first index past the row, and the last one inside it
    if M > 1:
        idx[-1] = N - 1
    out, loss = orc.nll_fwd(encode(x, dtype), idx)
    fin = np.isfinite(x)
    assert np.all(out[fin] >= 0) and np.all(np.isposinf(out[~fin]))
    np.testing.assert_allclose(np.exp(-out).sum(axis=1), 1.0, rtol=0, atol=1e-13)
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    for i in range(M):
        if 0 <= idx[i] < N:
            o = out[i, idx[i]]
            if np.isfinite(o):
                assert abs(loss[i] - o) <= rel * abs(o) + 1e-300
            else:
                assert loss[i] == o
        else:
            assert np.isnan(loss[i])


@SETTINGS
@given(grid_rows(), st.integers(0, 2 ** 32 - 1))
def test_nll_properties(orc, rows, seed):
    x, dtype, _ = rows
    check_nll(orc, x, dtype, np.random.default_rng(seed))


def check_layernorm(orc, x, dtype, rng):
    M, N = x.shape
    eps = 1e-5
    w = rng.integers(1, 32, size=N).astype(np.float64) / 8.0  # nonzero weights
    b = rng.integers(-32, 32, size=N).astype(np.float64) / 8.0
    xi, wi, bi = encode(x, dtype), encode(w, dtype), encode(b, dtype)
    y, mean, rstd = orc.layernorm_fwd(xi, wi, bi, eps)
    np.testing.assert_allclose(mean, x.mean(axis=1), rtol=1e-13, atol=1e-13)
    var = ((x - x.mean(axis=1, keepdims=True)) ** 2).mean(axis=1)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(var + eps), rtol=1e-12)
    xhat = (y - b) / w
    np.testing.assert_allclose(xhat.sum(axis=1), 0.0, rtol=0,
                               atol=1e-11 * N * (1 + np.abs(xhat).max()))
    dy = rng.integers(-64, 64, size=(M, N)).astype(np.float64) / 8.0
    dx, dw, db = orc.layernorm_bwd(encode(dy, dtype), xi, wi, eps)
    np.testing.assert_allclose(db, dy.sum(axis=0), rtol=1e-13, atol=1e-13)
    xh = (x - mean[:, None]) * rstd[:, None]
    np.testing.assert_allclose(dw, (dy * xh).sum(axis=0), rtol=1e-11, atol=1e-11)
    scale = np.abs(dx).sum(axis=1) + 1.0
    assert np.all(np.abs(dx.sum(axis=1)) <= 1e-11 * scale)
    # sum_j dx_j xhat_j = eps r^3 sum_j g_j xhat_j, g = dy w: the xhat part of the gradient
    # removes all but the eps share of g's projection on xhat
    g = dy * w
    lhs = (dx * xh).sum(axis=1)
    rhs = eps * rstd ** 3 * (g * xh).sum(axis=1)
    # dx_j is a difference of terms of the size of g_j: its rounding is relative to them
    tol = 1e-12 * rstd * N * (np.abs(g).sum(axis=1) * np.abs(xh).max(axis=1) + 1.0)
    assert np.all(np.abs(lhs - rhs) <= tol), (lhs, rhs)


@SETTINGS
@given(grid_rows(neg_inf=False, max_n=120), st.integers(0, 2 ** 32 - 1))
def test_layernorm_properties(orc, rows, seed):
    x, dtype, _ = rows
    check_layernorm(orc, x, dtype, np.random.default_rng(seed))


# ----------------------------------------------------------------------- planted mistakes
def fixed_case(seed: int):
    rng = np.random.default_rng(seed)
    M, N = int(rng.integers(2, 5)), int(rng.integers(3, 120))
    x = rng.integers(-128, 128, size=(M, N)).astype(np.float64) / 8.0
    if seed % 2:  # -inf patterns, one finite entry per row at least
        mask = rng.random((M, N)) < 0.5
        mask[np.arange(M), rng.integers(0, N, size=M)] = False
        x[mask] = -np.inf
    dtype = "bf16" if seed % 3 == 0 else "f32"
    t = np.empty(M, dtype=np.int64)
    for i in range(M):
        k = (seed + i) % 5
        fin = np.flatnonzero(np.isfinite(x[i]))
        t[i] = {3: -100, 4: N + 2}.get(k, int(rng.choice(fin)))
    return x, dtype, t, rng


def run_properties(orc, seed: int) -> None:
    x, dtype, t, rng = fixed_case(seed)
    finite = np.where(np.isfinite(x), x, 0.0)
    check_softmax(orc, x, dtype, int(rng.integers(-8, 8)))
    check_softmax_bwd(orc, finite, dtype, rng)
    check_xent(orc, x, dtype, t, int(rng.integers(-8, 8)))
    check_nll(orc, x, dtype, rng)
    check_layernorm(orc, finite, dtype, rng)


# The mutants whose mistake lies in what the properties above define (not row strides, the
# upstream gradient, the none reduction, element_mul, the block-sparse table, or how the
# gathered loss is rounded: the pins cover those).
PROPERTY_MUTANTS = [
    "softmax drops the max shift", "softmax takes the min", "softmax skips the division",
    "bf16 decoded with a wrong shift", "softmax backward flips the sign of s",
    "softmax backward multiplies by dy", "loss adds the target logit", "loss drops log d",
    "target logit read from row 0", "gradient not divided by n", "onehot at the wrong column",
    "onehot added instead of subtracted", "sum reduction divides by n",
    "sum skips the first loss", "nll drops log d", "nll adds the logit",
    "nll loss read at the next column", "nll accepts an index equal to N",
    "layer norm drops eps", "layer norm variance over N - 1", "layer norm multiplies by std",
    "layer norm skips the weight", "layer norm bias at the wrong column",
    "layer norm backward drops c1", "layer norm backward drops c2",
    "layer norm backward drops rstd", "layer norm backward c2 unweighted",
    "layer norm dw uses x instead of xhat", "layer norm db skips the last row",
    "ignored rows keep stale gradient", "ignored rows counted in n",
    "mean divides by the row count", "exp of the shifted logit uses the wrong sign",
    "sum of exponentials skips the last column",
]


def test_the_real_oracle_passes_the_fixed_cases(orc):
    for seed in range(12):
        run_properties(orc, seed)


@pytest.mark.parametrize("name", PROPERTY_MUTANTS)
def test_properties_catch_planted_mistakes(name, tmp_path):
    from test_oracle_mutants import MUTANTS
    find, replace = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(find) == 1
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(find, replace))
    mutant = oracle.Oracle(oracle.compile_library(str(mutant_src), str(tmp_path / "libm.so")))
    for seed in range(12):
        try:
            with np.errstate(all="ignore"):
                run_properties(mutant, seed)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            return
    pytest.fail(f"the properties miss the planted mistake {name!r}")
