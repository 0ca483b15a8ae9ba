"""Seeded random cases for every entry point against the float64 oracle: random sizes
(ragged, one element to several chunks), row pitches, dtypes, ignore fractions, reductions,
upstream gradients and forced launch paths. Each case prints its parameters before it runs,
so a failure names its case."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_losses, check_output, to_device, to_host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import cross_entropy_reductions_amd as xr
else:  # collected on a machine without a GPU: every test here is skipped
    xr = None
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no HIP device")]

CASES = 24


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(autouse=True)
def _reset_options():
    xr.reset_options()
    yield
    xr.reset_options()


def draw(rng, seed):
    M = int(rng.choice([1, 2, 3, 17, 64, 300]))
    N = int(rng.choice([1, 7, 8, 100, 1000, 4097, 20000, 70001]))
    dtype = str(rng.choice(["f32", "bf16"]))
    ld = N + int(rng.choice([0, 0, 1, 8, 13]))
    path = int(rng.choice([0, 0, 0, 1, 2, 3]))
    return M, N, dtype, ld, path


def force(path, N, dtype):
    xr.reset_options()
    if path:
        xr.set_option("path", path)
        if path == 2:
            xr.set_option("split", 2)


@pytest.mark.parametrize("case", range(CASES))
def test_random_xent(orc, case):
    rng = np.random.Generator(np.random.PCG64(16000 + case))
    M, V, dtype, ld, path = draw(rng, case)
    reduction = str(rng.choice(["mean", "sum", "none"]))
    ign = float(rng.choice([0.0, 0.3, 1.0]))
    scale = [None, 1.5, -0.5][int(rng.integers(3))]
    print(f"xent case {case}: M={M} V={V} ld={ld} {dtype} path={path} {reduction} ignore={ign} scale={scale}", flush=True)
    x = synth.random_rows(16100 + case, M, V, ld=ld, dtype=dtype, scale=3.0, pad_nan=ld > V)
    t = synth.random_targets(16200 + case, M, V, ignore_frac=ign)
    force(path, V, dtype)
    xd = to_device(x)
    try:
        loss, rows, counts = xr.xent_fwd_bwd(xd[:, :V], to_device(t), reduction=reduction,
                                             grad_scale=scale)
    except xr.XrError as e:
        assert path in (1, 2) and e.status == 2, e  # a forced path these sizes cannot take
        return
    torch.cuda.synchronize()
    g, l_rows, red, (n, bad) = orc.xent(x, t, V, reduction=reduction, scale=scale)
    assert to_host(counts).tolist()[:2] == [n, bad] and int(to_host(counts)[2]) == 0
    got = to_host(xd)
    if scale is None or got.dtype == np.uint16:
        check_output(got[:, :V], g, f"case {case} gradient")
    else:
        from gpu_util import check_fp32
        check_fp32(got[:, :V], g, f"case {case} gradient", tol=1e-5 * max(1.0, abs(scale)))
    if ld > V:
        assert np.array_equal(got[:, V:].view(np.uint8), x[:, V:].view(np.uint8))
    want_red = 0.0 if red is None else red
    got_red = 0.0 if reduction == "none" else float(loss.item())
    if reduction == "sum" and n == 0:
        want_red = 0.0
    check_losses(to_host(rows), got_red, l_rows, want_red, f"case {case} losses",
                 mean_abs=1e-5 * (M if reduction == "sum" else 1))


@pytest.mark.parametrize("case", range(CASES))
def test_random_softmax(orc, case):
    rng = np.random.Generator(np.random.PCG64(17000 + case))
    M, N, dtype, ld, path = draw(rng, case)
    path = 0 if path == 2 else path  # softmax rows are never split
    print(f"softmax case {case}: M={M} N={N} ld={ld} {dtype} path={path}", flush=True)
    x = synth.random_rows(17100 + case, M, N, ld=ld, dtype=dtype, scale=3.0, pad_nan=ld > N)
    dy = synth.random_rows(17200 + case, M, N, ld=ld, dtype=dtype, scale=1.0, pad_nan=ld > N)
    force(path, N, dtype)
    xd, dyd = to_device(x), to_device(dy)
    try:
        y = xr.softmax_fwd(xd[:, :N])
        dx = xr.softmax_bwd(y, dyd[:, :N])
    except xr.XrError as e:
        assert path == 1 and e.status == 2, e
        return
    torch.cuda.synchronize()
    y_h = to_host(y)
    check_output(y_h, orc.softmax_fwd(x, n_cols=N), f"case {case} softmax")
    dy_c = np.ascontiguousarray(dy[:, :N])
    check_output(to_host(dx), orc.softmax_bwd(y_h, dy_c), f"case {case} softmax backward")


@pytest.mark.parametrize("case", range(CASES))
def test_random_nll(orc, case):
    rng = np.random.Generator(np.random.PCG64(18000 + case))
    M, N, dtype, ld, path = draw(rng, case)
    print(f"nll case {case}: M={M} N={N} ld={ld} {dtype} path={path}", flush=True)
    x = synth.random_rows(18100 + case, M, N, ld=ld, dtype=dtype, scale=3.0, pad_nan=ld > N)
    idx = synth.random_targets(18200 + case, M, N)
    if M > 1:
        idx[0] = N  # outside the row
    force(path, N, dtype)
    try:
        out, loss = xr.nll_fwd(to_device(x)[:, :N], to_device(idx))
    except xr.XrError as e:
        assert path in (1, 2) and e.status == 2, e
        return
    torch.cuda.synchronize()
    want, wl = orc.nll_fwd(x, idx, n_cols=N)
    got = to_host(out)
    from test_gpu_nll import check_nll
    check_nll(got, to_host(loss), want, wl, f"case {case} nll")
