"""GPU parity of the negative log-softmax forward with a gathered loss (xr_nll_fwd) against
the float64 oracle.

Outputs: fp32 within 1e-5 absolute, bf16 within the suite's 2e-2 relative bound (floored
at 2^-7 of the row's largest value) plus the absolute error the fp32 arithmetic can leave
before the bf16 rounding: the output (m + log d) - x_j is one fp32 subtraction of values up
to |m| + log d, after one fp32 addition and a log accurate to a few ulps, so each row gets
2^-21 (max_j |x_j| + log d + 1), a few ulps of its largest magnitude (this matters where
the result is near 0: the row's maximum when d is near 1, e.g. a one-column row, where the
exact result is 0). The loss is the stored output element, so it carries the output's
rounding: fp32 losses within 1e-5, bf16 losses within the bf16 bound of their row. +inf
outputs (from -inf logits) and NaN losses (indices outside the row) must match exactly.
"""
from __future__ import annotations

import json

import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import synth
from gpu_util import BF16_FLOOR, BF16_REL, FP32_ABS, to_device, to_host, widen

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


def check_nll(out_gpu: np.ndarray, loss_gpu: np.ndarray, out_want: np.ndarray,
              loss_want: np.ndarray, what: str, x: np.ndarray) -> None:
    """x: the input rows (host bytes; their first out_want.shape[1] columns are the rows)."""
    g = widen(out_gpu)
    assert g.shape == out_want.shape, what
    inf = np.isinf(out_want)
    assert np.array_equal(np.isinf(g), inf) and np.all(g[inf] == out_want[inf]), f"{what}: +inf"
    fin = ~inf
    if out_gpu.dtype == np.uint16:
        xin = widen(np.ascontiguousarray(x[:, :out_want.shape[1]]))
        xmax = np.max(np.where(np.isfinite(xin), np.abs(xin), 0.0), axis=1, keepdims=True)
        logd = np.min(np.where(fin, out_want, np.inf), axis=1, keepdims=True)
        allow = 2.0 ** -21 * (xmax + np.abs(logd) + 1.0)
        rmax = np.max(np.where(fin, np.abs(out_want), 0.0), axis=1, keepdims=True)
        bound = BF16_REL * np.maximum(np.abs(out_want), BF16_FLOOR * rmax) + allow
        with np.errstate(invalid="ignore"):
            scaled = np.where(fin, np.abs(g - out_want) / bound, 0.0)
        worst = float(np.max(scaled)) if scaled.size else 0.0
        assert worst <= 1.0, f"{what}: worst error over its bound {worst:.3e}"
        ltol = BF16_REL * np.maximum(np.abs(loss_want), BF16_FLOOR * rmax[:, 0]) + allow[:, 0]
    else:
        err = np.where(fin, np.abs(g - out_want), 0.0)
        worst = float(np.max(err)) if err.size else 0.0
        assert worst <= FP32_ABS, f"{what}: max abs error {worst:.3e}"
        ltol = np.full(loss_want.shape, FP32_ABS)
    nan = np.isnan(loss_want)
    assert np.array_equal(np.isnan(loss_gpu), nan), f"{what}: NaN losses"
    lerr = np.abs(loss_gpu.astype(np.float64) - loss_want)
    with np.errstate(invalid="ignore"):
        ok = (lerr <= ltol) | (loss_gpu.astype(np.float64) == loss_want)  # equal infinities
    bad = np.flatnonzero(~nan & ~ok)
    assert bad.size == 0, f"{what}: row {bad[0]} loss {loss_gpu[bad[0]]} vs {loss_want[bad[0]]}"


def run(x_host: np.ndarray, idx: np.ndarray, N: int, in_place: bool = False,
        out_ld: int | None = None):
    x = to_device(x_host)
    xv = x[:, :N]
    if in_place:
        out = xv
    elif out_ld is not None:
        out = torch.empty((x_host.shape[0], out_ld), dtype=x.dtype, device="cuda")[:, :N]
    else:
        out = None
    out, loss = xr.nll_fwd(xv, to_device(idx), out)
    torch.cuda.synchronize()
    return to_host(out), to_host(loss), to_host(x)


def test_worked_example(orc):
    with open(oracle_pins.GOLDEN) as f:
        gold = json.load(f)
    for case in gold["nll_fwd"]:
        x = oracle_pins.as_input(case["x"], case["dtype"])
        out, loss, _ = run(x, np.array(case["idx"], dtype=np.int64), x.shape[1])
        want = np.array([[oracle_pins.closed_form(v) for v in r] for r in case["out"]])
        wl = np.array([oracle_pins.closed_form(v) for v in case["loss"]])
        check_nll(out, loss, want, wl, case["name"], x)


SHAPES = [(1, 1, "f32"), (3, 2, "bf16"), (19, 257, "f32"), (128, 1000, "f32"),
          (64, 4096, "bf16"), (8, 4099, "bf16"), (6, 33333, "f32"), (4, 65536, "bf16"),
          (3, 70000, "f32"), (2, 300000, "bf16"), (700, 3001, "bf16")]


@pytest.mark.parametrize("M,N,dtype", SHAPES, ids=[f"{m}x{n}-{d}" for m, n, d in SHAPES])
def test_nll_shapes(orc, M, N, dtype):
    x = synth.random_rows(12000 + N % 101, M, N, dtype=dtype, scale=4.0)
    idx = synth.random_targets(12001 + N % 101, M, N)
    if M > 2:
        idx[1] = N  # outside the row: NaN loss
        idx[2] = -1
    out, loss, _ = run(x, idx, N)
    want, wl = orc.nll_fwd(x, idx)
    check_nll(out, loss, want, wl, f"nll {M}x{N} {dtype}", x)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nll_in_place_strides_and_unaligned(orc, dtype):
    M, N, ld = 50, 5001, 5010
    x = synth.random_rows(12100, M, N, ld=ld, dtype=dtype, scale=3.0, pad_nan=True)
    idx = synth.random_targets(12101, M, N)
    want, wl = orc.nll_fwd(x, idx, n_cols=N)
    out, loss, full = run(x, idx, N, in_place=True)
    check_nll(out, loss, want, wl, f"{dtype} in place", x)
    assert np.array_equal(full[:, N:].view(np.uint8), x[:, N:].view(np.uint8)), "padding changed"
    # a separate output with another row stride (rows at other addresses mod 16: stream path)
    out, loss, _ = run(x, idx, N, out_ld=N + 3)
    check_nll(out, loss, want, wl, f"{dtype} out-of-place, other stride", x)


def test_nll_neg_inf_entries(orc):
    M, N = 12, 2000
    x = synth.random_rows(12200, M, N, dtype="f32", scale=3.0)
    x[:, ::3] = -np.inf
    idx = synth.random_targets(12201, M, N)
    idx[0] = 3  # a -inf entry: loss +inf
    out, loss, _ = run(x, idx, N)
    want, wl = orc.nll_fwd(x, idx)
    check_nll(out, loss, want, wl, "-inf entries", x)
    assert np.isinf(loss[0]) and loss[0] > 0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nll_all_paths_agree(orc, dtype):
    M, N = 300, 20000
    x = synth.random_rows(12300, M, N, dtype=dtype, scale=3.0)
    idx = synth.random_targets(12301, M, N)
    want, wl = orc.nll_fwd(x, idx)
    for name, path, grid, split in (("auto", 0, 0, 0), ("resident", 1, 0, 0),
                                    ("persistent", 1, 2, 0), ("split2", 2, 0, 2),
                                    ("split5", 2, 0, 5), ("stream", 3, 0, 0)):
        xr.set_option("path", path)
        xr.set_option("grid", grid)
        xr.set_option("split", split)
        out, loss, _ = run(x, idx, N)
        check_nll(out, loss, want, wl, f"{dtype} {name}", x)


def test_nll_without_workspace_keeps_rows_whole(orc):
    """No workspace: long rows run whole (one workgroup each) and give the same results."""
    import ctypes
    M, N = 6, 128256
    x_h = synth.random_rows(12400, M, N, dtype="bf16", scale=2.0)
    idx = synth.random_targets(12401, M, N)
    assert xr.plan("nll_fwd", M, N, torch.bfloat16)["split"] > 1
    x, ix = to_device(x_h), to_device(idx)
    out = torch.empty_like(x)
    loss = torch.empty(M, dtype=torch.float32, device="cuda")
    st = xr.lib.xr_nll_fwd(out.data_ptr(), N, x.data_ptr(), N, ix.data_ptr(), loss.data_ptr(),
                           M, N, xr.BF16, None, 0,
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    want, wl = orc.nll_fwd(x_h, idx)
    check_nll(to_host(out), to_host(loss), want, wl, "no workspace", x_h)
    out2, loss2, _ = run(x_h, idx, N)  # split rows
    check_nll(out2, loss2, want, wl, "split rows", x_h)


def test_nll_c4_matrix(orc):
    """The 16384 x 128256 bf16 logits of the cross-entropy workload, every loss and a sample
    of full rows, in the launch configuration the benchmark times (a separate output)."""
    w = synth.xent_c4()
    x_h, M, N = w["x"], w["M"], w["N"]
    idx = np.where(w["target"] < 0, 0, w["target"]).astype(np.int64)
    x = to_device(x_h)
    out, loss = xr.nll_fwd(x, to_device(idx))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2, 777, 8191, 12000, M - 1])
    got = to_host(out[torch.from_numpy(rows).cuda()])
    want, wl = orc.nll_fwd(x_h[rows], idx[rows])
    check_nll(got, to_host(loss)[rows], want, wl, "16384 x 128256 sampled rows", x_h[rows])
    # every loss: -log p of the gathered element, against the float64 loss of each row
    loss_h = to_host(loss).astype(np.float64)
    _, l_all = orc.xent_rows(x_h, idx, N, 1, ignore_index=-(1 << 62), want_grad=False)
    rel = np.abs(loss_h - l_all) / np.maximum(np.abs(l_all), 1.0)
    assert np.max(rel) <= 2.0 ** -8, "losses vs float64 row losses (one bf16 rounding)"
