"""GPU parity of the layer norm forward and backward (xr_layernorm_fwd / _bwd) against the
float64 oracle.

Tolerances: y and dx as the rest of the suite, except that layer norm outputs are not
bounded by 1 (dx carries a factor rstd, which is 1/sqrt(eps) on a constant row), so the
fp32 bound is 1e-5 times the larger of 1 and the row's largest |value|; bf16 2e-2 relative
with the row floor; mean and rstd (fp32) 1e-5 relative. dw and db are sums over the M rows in
fp32, whose rounding error grows with the sum of the magnitudes of the terms: they must lie
within 2e-5 * sum_i |term_i| (+1e-6) of the oracle, plus one bf16 rounding (2^-8 |value|)
for bf16 outputs.
"""
from __future__ import annotations

import json

import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import synth
from gpu_util import FP32_ABS, check_bf16, to_device, to_host, widen

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import cross_entropy_reductions_amd as xr
else:  # collected on a machine without a GPU: every test here is skipped
    xr = None
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no HIP device")]


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(autouse=True)
def _reset_options():
    xr.reset_options()
    yield
    xr.reset_options()


def inputs(seed, M, N, dtype, ld=None):
    x = synth.random_rows(seed, M, N, ld=ld, dtype=dtype, scale=2.0, pad_nan=ld is not None)
    wb = synth.random_rows(seed + 1, 2, N, dtype=dtype, scale=1.0)
    dy = synth.random_rows(seed + 2, M, N, ld=ld, dtype=dtype, scale=1.0, pad_nan=ld is not None)
    return x, np.ascontiguousarray(wb[0]), np.ascontiguousarray(wb[1]), dy


def check_output(got: np.ndarray, want: np.ndarray, what: str) -> None:
    if got.dtype == np.uint16:
        check_bf16(got, want, what)
        return
    g = widen(got)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    tol = FP32_ABS * np.maximum(1.0, np.max(np.abs(want), axis=-1, keepdims=True))
    bad = np.argwhere(np.abs(g - want) > tol)
    assert bad.size == 0, f"{what}: element {tuple(bad[0])} {g[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


def check_sums(got: np.ndarray, want: np.ndarray, abs_sum: np.ndarray, what: str) -> None:
    g = widen(got)
    tol = 2e-5 * abs_sum + 1e-6
    if got.dtype == np.uint16:
        tol = tol + 2.0 ** -8 * np.abs(want)
    bad = np.flatnonzero(np.abs(g - want) > tol)
    assert bad.size == 0, f"{what}: column {bad[0]} {g[bad[0]]} vs {want[bad[0]]}"


def check_stats(mean, rstd, want_mean, want_rstd, what):
    assert np.max(np.abs(mean - want_mean) / np.maximum(np.abs(want_mean), 1.0)) <= 1e-5, what
    assert np.max(np.abs(rstd - want_rstd) / want_rstd) <= 1e-5, what


def run_case(orc, x_h, w_h, b_h, dy_h, N, eps, what, in_place=False, dx_alias=None):
    M = x_h.shape[0]
    x = to_device(x_h)[:, :N]
    w, b = to_device(w_h), to_device(b_h)
    xin = x.clone() if in_place else x
    y, mean, rstd = xr.layernorm_fwd(xin, w, b, eps, out=xin if in_place else None)
    dyd = to_device(dy_h)[:, :N]
    dxo = {"dy": dyd, "x": x}.get(dx_alias)
    dx, dw, db = xr.layernorm_bwd(dyd, x, w, mean, rstd, dx=dxo)
    torch.cuda.synchronize()
    yw, mw, rw = orc.layernorm_fwd(x_h, w_h, b_h, eps, n_cols=N)
    dxw, dww, dbw = orc.layernorm_bwd(dy_h, x_h, w_h, eps, n_cols=N)
    check_output(to_host(y), yw, f"{what}: y")
    check_stats(to_host(mean).astype(np.float64), to_host(rstd).astype(np.float64), mw, rw,
                f"{what}: mean / rstd")
    check_output(to_host(dx), dxw, f"{what}: dx")
    xd = widen(x_h)[:, :N]
    dyd_h = widen(dy_h)[:, :N]
    xhat = (xd - mw[:, None]) * rw[:, None]
    check_sums(to_host(dw), dww, np.abs(dyd_h * xhat).sum(axis=0), f"{what}: dw")
    check_sums(to_host(db), dbw, np.abs(dyd_h).sum(axis=0), f"{what}: db")


def test_worked_examples(orc):
    with open(oracle_pins.GOLDEN) as f:
        gold = json.load(f)
    for case in gold["layernorm"]:
        x_h = oracle_pins.as_input(case["x"], case["dtype"])
        w_h = oracle_pins.as_input([case["w"]], case["dtype"])[0]
        b_h = oracle_pins.as_input([case["b"]], case["dtype"])[0]
        dy_h = oracle_pins.as_input(case["dy"], case["dtype"])
        x, w, b, dy = (to_device(a) for a in (x_h, w_h, b_h, dy_h))
        y, mean, rstd = xr.layernorm_fwd(x, w, b, case["eps"])
        dx, dw, db = xr.layernorm_bwd(dy, x, w, mean, rstd)
        cf = oracle_pins.closed_form
        check_output(to_host(y), np.array([[cf(v) for v in r] for r in case["y"]]), case["name"])
        check_output(to_host(dx), np.array([[cf(v) for v in r] for r in case["dx"]]), case["name"])
        for got, key in ((dw, "dw"), (db, "db")):
            want = np.array([cf(v) for v in case[key]])
            check_sums(to_host(got), want, np.abs(want) + 1.0, f"{case['name']}: {key}")
        check_stats(to_host(mean).astype(np.float64), to_host(rstd).astype(np.float64),
                    np.array([cf(v) for v in case["mean"]]), np.array([cf(v) for v in case["rstd"]]),
                    case["name"])


SHAPES = [(1, 8, "f32"), (3, 16, "bf16"), (33, 1000, "f32"), (257, 4096, "bf16"),
          (64, 8192, "bf16"), (16, 16384, "bf16"), (8, 32768, "bf16"), (5, 16384, "f32"),
          (100, 1001, "f32"), (100, 4099, "bf16"), (2000, 512, "bf16")]


@pytest.mark.parametrize("M,N,dtype", SHAPES, ids=[f"{m}x{n}-{d}" for m, n, d in SHAPES])
def test_layernorm_shapes(orc, M, N, dtype):
    x, w, b, dy = inputs(13000 + N % 89, M, N, dtype)
    run_case(orc, x, w, b, dy, N, 1e-5, f"{M}x{N} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layernorm_strides_and_aliases(orc, dtype):
    M, N, ld = 70, 2048, 2056  # rows 16-byte aligned in a padded pitch
    x, w, b, dy = inputs(13100, M, N, dtype, ld=ld)
    run_case(orc, x, w, b, dy, N, 1e-5, f"{dtype} padded")
    run_case(orc, x, w, b, dy, N, 1e-5, f"{dtype} y = x", in_place=True)
    run_case(orc, x, w, b, dy, N, 1e-5, f"{dtype} dx = dy", dx_alias="dy")
    run_case(orc, x, w, b, dy, N, 1e-5, f"{dtype} dx = x", dx_alias="x")
    # rows off 16-byte boundaries: the element-wise kernels
    x2, w2, b2, dy2 = inputs(13101, M, N, dtype, ld=N + 3)
    run_case(orc, x2, w2, b2, dy2, N, 1e-5, f"{dtype} unaligned rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layernorm_all_paths_agree(orc, dtype):
    M, N = 600, 1024
    x, w, b, dy = inputs(13200, M, N, dtype)
    for name, path, grid in (("auto", 0, 0), ("resident", 1, 0), ("one per CU", 1, 1),
                             ("stream", 3, 0)):
        xr.set_option("path", path)
        xr.set_option("grid", grid)
        run_case(orc, x, w, b, dy, N, 1e-4, f"{dtype} {name}")


def test_layernorm_eps_and_constant_rows(orc):
    M, N = 40, 256
    x, w, b, dy = inputs(13300, M, N, "f32")
    x[::3] = 1.5  # constant rows: y = b, rstd = 1/sqrt(eps)
    for eps in (0.0, 1e-5, 0.25):
        if eps == 0.0:
            xx = x[1::3].copy()  # no constant rows without eps
            run_case(orc, xx, w, b, dy[1::3].copy(), N, eps, f"eps {eps}")
        else:
            run_case(orc, x, w, b, dy, N, eps, f"eps {eps}")


def test_layernorm_deterministic():
    M, N = 3000, 4096
    x_h, w_h, b_h, dy_h = inputs(13400, M, N, "bf16")
    x, w, b, dy = (to_device(a) for a in (x_h, w_h, b_h, dy_h))
    outs = []
    for _ in range(3):
        y, mean, rstd = xr.layernorm_fwd(x, w, b)
        dx, dw, db = xr.layernorm_bwd(dy, x, w, mean, rstd)
        outs.append([to_host(t) for t in (y, dx, dw, db)])
    for o in outs[1:]:
        for a, b_ in zip(o, outs[0]):
            assert np.array_equal(a, b_)


def test_layernorm_autograd(orc):
    M, N = 48, 1024
    x_h, w_h, b_h, dy_h = inputs(13500, M, N, "f32")
    x = to_device(x_h).reshape(4, 12, N).requires_grad_(True)
    w = to_device(w_h).requires_grad_(True)
    b = to_device(b_h).requires_grad_(True)
    y = xr.layer_norm(x, w, b, 1e-5)
    y.backward(to_device(dy_h).reshape(4, 12, N))
    yw, _, _ = orc.layernorm_fwd(x_h, w_h, b_h, 1e-5)
    dxw, dww, dbw = orc.layernorm_bwd(dy_h, x_h, w_h, 1e-5)
    check_output(to_host(y.detach()).reshape(M, N), yw, "autograd y")
    check_output(to_host(x.grad).reshape(M, N), dxw, "autograd dx")
    xd, dyd = widen(x_h), widen(dy_h)
    xhat = (xd - xd.mean(axis=1, keepdims=True)) / np.sqrt(xd.var(axis=1, keepdims=True) + 1e-5)
    check_sums(to_host(w.grad), dww, np.abs(dyd * xhat).sum(axis=0), "autograd dw")
    check_sums(to_host(b.grad), dbw, np.abs(dyd).sum(axis=0), "autograd db")


def test_layernorm_full_workload(orc):
    """16384 x 8192 bf16 (the benchmark's layer norm workload), in the launch configuration
    the benchmark times: every mean / rstd, dw and db in full, y and dx on sampled rows."""
    wl = synth.layernorm_ln()
    x_h, dy_h, w_h, b_h, eps = wl["x"], wl["dy"], wl["w"], wl["b"], wl["eps"]
    M, N = wl["M"], wl["N"]
    x, dy, w, b = (to_device(a) for a in (x_h, dy_h, w_h, b_h))
    y, mean, rstd = xr.layernorm_fwd(x, w, b, eps)
    dx, dw, db = xr.layernorm_bwd(dy, x, w, mean, rstd)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2, 4095, 8191, 12345, M - 1])
    ridx = torch.from_numpy(rows).cuda()
    yw, mw, rw = orc.layernorm_fwd(x_h[rows], w_h, b_h, eps)
    check_output(to_host(y[ridx]), yw, "full workload y")
    dxw, _, _ = orc.layernorm_bwd(dy_h[rows], x_h[rows], w_h, eps)
    check_output(to_host(dx[ridx]), dxw, "full workload dx")
    _, mw_all, rw_all = orc.layernorm_fwd(x_h, w_h, b_h, eps)
    check_stats(to_host(mean).astype(np.float64), to_host(rstd).astype(np.float64), mw_all,
                rw_all, "full workload mean / rstd")
    _, dww, dbw = orc.layernorm_bwd(dy_h, x_h, w_h, eps)
    xd, dyd = widen(x_h), widen(dy_h)
    xhat = (xd - mw_all[:, None]) * rw_all[:, None]
    check_sums(to_host(dw), dww, np.abs(dyd * xhat).sum(axis=0), "full workload dw")
    check_sums(to_host(db), dbw, np.abs(dyd).sum(axis=0), "full workload db")
