"""The parity checkers of tests/gpu_util.py, on the CPU: oracle results rounded exactly to the
storage type must pass, and planted errors of the kinds a kernel could make must fail.

The cross-entropy cases are oracle gradient rows scaled like the benchmark workloads:
rows of the 8192 x 32000 bf16 (n = 7373), 16384 x 128256 bf16 (n = 15565) and
2048 x 256000 fp32 workloads, with each workload's own n. The gradient entries there are
s p_j / n for j != t (Liger-Kernel cross_entropy.py page, liger_cross_entropy_kernel
step 4's comment) and s (p_t - 1) / n at the target.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_bf16, check_output, check_probs, check_xent_grad, softmax_bwd_allow


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def stored(g: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values as the bytes a kernel would store: bf16 bits (RNE) or fp32."""
    g32 = g.astype(np.float32)
    return synth.bf16_bits_from_f32(g32) if dtype == "bf16" else g32


ROWS = 24
WORKLOADS = {
    # name: (generator, n of the whole workload, dtype)
    "c3": (lambda: synth.xent_c3(M=ROWS), 7373, "bf16"),
    "c4": (lambda: synth.xent_c4(M=ROWS), 15565, "bf16"),
    "c5": (lambda: synth.xent_c5(M=ROWS * 5), 2048, "f32"),
}


@pytest.fixture(scope="module", params=sorted(WORKLOADS))
def case(request, orc):
    make, n, dtype = WORKLOADS[request.param]
    w = make()
    V = w["N"]
    x, t = w["x"], w["target"].copy()
    M = x.shape[0]
    t[1] = -100  # one row without a gradient in every case
    g, _ = orc.xent_rows(x, t, V, n)
    return {"name": request.param, "x": x, "t": t, "V": V, "n": n, "M_full": {
        "c3": 8192, "c4": 16384, "c5": 2048}[request.param], "dtype": dtype, "g": g, "M": M}


def run(case, g_stored, n_r=None):
    return check_xent_grad(g_stored, case["g"], case["t"], case["V"],
                           case["n"] if n_r is None else n_r, case["name"])


def target_mask(case):
    m = np.zeros_like(case["g"], dtype=bool)
    live = np.flatnonzero((case["t"] >= 0) & (case["t"] < case["V"]))
    m[live, case["t"][live]] = True
    return m


def test_rounded_oracle_passes(case):
    worst = run(case, stored(case["g"], case["dtype"]))
    assert worst <= 0.51, worst  # one rounding uses about half of each bound


def test_small_entries_zeroed_fail(case):
    g = case["g"].copy()
    g[(np.abs(g) < 1e-6) & ~target_mask(case)] = 0.0
    with pytest.raises(AssertionError):
        run(case, stored(g, case["dtype"]))


def test_all_non_target_entries_zeroed_fail(case):
    g = np.where(target_mask(case), case["g"], 0.0)
    with pytest.raises(AssertionError):
        run(case, stored(g, case["dtype"]))


def test_non_target_scaled_fails(case):
    g = np.where(target_mask(case), case["g"], 1.04 * case["g"])
    with pytest.raises(AssertionError):
        run(case, stored(g, case["dtype"]))


def test_wrong_divisor_fails(case, orc):
    """1/n replaced by 1/M (the rows of the batch instead of the non-ignored ones). The fp32
    workload has no ignored rows (n = M), so there the divisor is taken 1 % off instead."""
    wrong = case["M_full"] if case["M_full"] != case["n"] else int(case["n"] * 0.99)
    g, _ = orc.xent_rows(case["x"], case["t"], case["V"], wrong)
    with pytest.raises(AssertionError):
        run(case, stored(g, case["dtype"]))


def test_target_off_by_one_percent_fails(case):
    g = np.where(target_mask(case), 1.01 * case["g"], case["g"])
    with pytest.raises(AssertionError):
        run(case, stored(g, case["dtype"]))


def test_dead_row_must_be_zero(case):
    g = stored(case["g"], case["dtype"]).copy()
    g[1, 5] = g[0, 5]  # row 1 is ignored
    with pytest.raises(AssertionError, match="exactly zero"):
        run(case, g)


def test_target_allowance_bounds(orc):
    """A one-column row has gradient 0 in exact arithmetic; fp32 leaves a residue of a few
    ulps of 1/n, which passes, while an error of 1e-4/n does not."""
    x = np.array([[0.5], [-2.0]], dtype=np.float32)
    t = np.array([0, 0], dtype=np.int64)
    g, _ = orc.xent_rows(x, t, 1, 2)
    assert np.all(g == 0.0)
    ok = np.array([[-2.0 ** -24 / 2], [2.0 ** -23 / 2]], dtype=np.float32)
    check_xent_grad(ok, g, t, 1, 2, "residue")
    bad = np.array([[-1e-4 / 2], [0.0]], dtype=np.float32)
    with pytest.raises(AssertionError):
        check_xent_grad(bad, g, t, 1, 2, "error")


def test_upstream_scale_scales_the_allowance(orc):
    x = synth.random_rows(5, 6, 50, dtype="f32", scale=3.0)
    t = np.array([0, 3, -100, 49, 7, 8], dtype=np.int64)
    s = np.array([2.0, -0.5, 1.0, 3.0, -1.0, 0.25])
    g, _ = orc.xent_rows(x, t, 50, 1, reduction="none", scale=s)
    check_xent_grad(g.astype(np.float32), g, t, 50, 1, "scaled", scale=s)
    with pytest.raises(AssertionError):
        check_xent_grad((g * 1.001).astype(np.float32), g, t, 50, 1, "scaled x1.001", scale=s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_probs_checker(orc, dtype):
    w = synth.softmax_c2(M=16) if dtype == "bf16" else synth.softmax_c1()
    y = orc.softmax_fwd(w["x"])
    check_probs(stored(y, dtype), y, "rounded")
    for name, bad in (("x1.04", 1.04 * y), ("small zeroed", np.where(y < 2e-5, 0.0, y)),
                      ("every 97th entry 1 % off",
                       np.where(np.arange(y.size).reshape(y.shape) % 97 == 0, 1.01 * y, y))):
        with pytest.raises(AssertionError):
            check_probs(stored(bad, dtype), y, name)


def test_cancelling_checker_has_no_absolute_floor():
    """The bf16 bound for outputs that cross zero is relative to the row's largest entry
    (2e-2 x 2^-7 of it), with no absolute floor: rows of small values are held to their own
    scale."""
    want = np.array([[1e-6, -3e-7, 2e-7, 0.0]])
    check_bf16(stored(want, "bf16"), want, "rounded")
    with pytest.raises(AssertionError):
        check_bf16(stored(np.array([[1e-6, -3e-7, 0.0, 0.0]]), "bf16"), want, "entry dropped")


def test_softmax_bwd_allowance(orc):
    """The softmax backward's arithmetic allowance (softmax_bwd_allow): the oracle's result
    rounded once to bf16 passes; a result 4 % off, one that drops a column's term of s, and
    one whose s carries the wrong sign still fail. On a row where dy_i is close to s (y_i
    about 1) the allowance covers the fp32 rounding of s, which is all such an entry holds."""
    M, N = 64, 1000
    x = synth.random_rows(31, M, N, dtype="f32", scale=3.0)
    y = synth.bf16_bits_from_f32(orc.softmax_fwd(x).astype(np.float32))
    dy = synth.random_rows(32, M, N, dtype="bf16", scale=1.0)
    want = orc.softmax_bwd(y, dy)
    allow = softmax_bwd_allow(y, dy)
    check_output(synth.bf16_bits_from_f32(want.astype(np.float32)), want, "rounded once", allow)
    yw, dw = synth.f32_from_bf16_bits(y).astype(np.float64), synth.f32_from_bf16_bits(dy).astype(np.float64)
    s = np.sum(yw * dw, axis=1, keepdims=True)
    s_drop = s - (yw * dw)[:, :1]
    for name, bad in (("4 % off", want * 1.04), ("a term of s dropped", yw * (dw - s_drop)),
                      ("s with the wrong sign", yw * (dw + s))):
        with pytest.raises(AssertionError):
            check_output(synth.bf16_bits_from_f32(bad.astype(np.float32)), want, name, allow)
    # one dominant column whose dy equals s up to fp32 rounding: dx there is cancellation
    y1 = np.full((1, 7), 1e-6, dtype=np.float32)
    y1[0, 3] = 1.0
    dy1 = np.array([[-0.115, -0.715, -0.081, 1.3984375, 1.22, -0.416, 0.9375]], dtype=np.float32)
    w1 = orc.softmax_bwd(y1, dy1)
    s1 = np.float32(np.sum((y1 * dy1).astype(np.float32), dtype=np.float32))
    got = (y1 * (dy1 - s1)).astype(np.float32)  # the fp32 formula, as a kernel computes it
    check_output(synth.bf16_bits_from_f32(got), w1, "cancellation row",
                 softmax_bwd_allow(y1, dy1))
