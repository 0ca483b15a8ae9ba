"""Seeded random cases for every entry point against the float64 oracle: random sizes
(ragged, one element to several chunks), row pitches, dtypes, ignore fractions, reductions,
upstream gradients, forced launch paths and, for the softmax family, rows moved by large
offsets. Each case prints its parameters before it runs,
so a failure names its case."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (check_losses, check_output, check_probs, check_xent_grad, softmax_bwd_allow,
                      to_device, to_host)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import cross_entropy_reductions_amd as xr
else:  # collected on a machine without a GPU: every test here is skipped
    xr = None
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no HIP device")]

# cases per entry point (XR_RANDOM_CASES widens the sweep; the default keeps the suite short)
CASES = int(os.environ.get("XR_RANDOM_CASES", "24"))


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


def shift_rows(seed, x, N, dtype):
    """A third of the cases move each row by a common offset of large magnitude (+-100,
    +-1e4 or +-1e6, one per row; padding untouched): the results depend only on x - max, and
    such rows take the kernels' other exponent forms. Drawn from a generator of its own, so
    the other draws of a case stay as they are. Returns the rows and the offsets (or None)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if rng.random() >= 1.0 / 3.0:
        return x, None
    off = rng.choice([-1e6, -1e4, -100.0, 100.0, 1e4, 1e6], size=x.shape[0])
    vals = synth.f32_from_bf16_bits(x[:, :N]) if dtype == "bf16" else x[:, :N]
    vals = (vals.astype(np.float64) + off[:, None]).astype(np.float32)
    x = x.copy()
    x[:, :N] = synth.bf16_bits_from_f32(vals) if dtype == "bf16" else vals
    return x, off


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
    x = synth.random_rows(16100 + case, M, V, ld=ld, dtype=dtype, scale=3.0, pad_nan=ld > V)
    x, off = shift_rows(16300 + case, x, V, dtype)
    print(f"xent case {case}: M={M} V={V} ld={ld} {dtype} path={path} {reduction} ignore={ign} "
          f"scale={scale} offsets={None if off is None else sorted(set(off.tolist()))}", flush=True)
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
    check_xent_grad(got[:, :V], g, t, V, n if reduction == "mean" else 1, f"case {case} gradient",
                    scale=scale)
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
    # rows split over workgroups need a workspace; without one they stay whole
    use_ws = path == 2 or bool(rng.integers(2))
    x = synth.random_rows(17100 + case, M, N, ld=ld, dtype=dtype, scale=3.0, pad_nan=ld > N)
    x, off = shift_rows(17300 + case, x, N, dtype)
    print(f"softmax case {case}: M={M} N={N} ld={ld} {dtype} path={path} workspace={use_ws} "
          f"offsets={None if off is None else sorted(set(off.tolist()))}", flush=True)
    dy = synth.random_rows(17200 + case, M, N, ld=ld, dtype=dtype, scale=1.0, pad_nan=ld > N)
    force(path, N, dtype)
    xd, dyd = to_device(x), to_device(dy)
    try:
        ws = None if use_ws else False
        y = xr.softmax_fwd(xd[:, :N], workspace=ws)
        dx = xr.softmax_bwd(y, dyd[:, :N], workspace=ws)
    except xr.XrError as e:
        assert path in (1, 2) and e.status == 2, e  # a forced path these sizes cannot take
        return
    torch.cuda.synchronize()
    y_h = to_host(y)
    check_probs(y_h, orc.softmax_fwd(x, n_cols=N), f"case {case} softmax")
    dy_c = np.ascontiguousarray(dy[:, :N])
    check_output(to_host(dx), orc.softmax_bwd(y_h, dy_c), f"case {case} softmax backward",
                 softmax_bwd_allow(y_h, dy_c))


@pytest.mark.parametrize("case", range(CASES))
def test_random_softmax_bwd_resident(orc, case):
    """The backward on y, dy and dx sharing one row pitch (so the row-resident kernels take
    them, partial first / last vectors included): the one-row form and the persistent form,
    against the oracle, and the two forms to the same bits."""
    rng = np.random.Generator(np.random.PCG64(17500 + case))
    M = int(rng.choice([1, 3, 64, 300, 700]))
    N = int(rng.choice([1, 7, 9, 100, 1000, 3001, 4096, 8191]))
    dtype = str(rng.choice(["f32", "bf16"]))
    ld = N + int(rng.choice([0, 1, 3, 8, 13]))
    print(f"softmax bwd case {case}: M={M} N={N} ld={ld} {dtype}", flush=True)
    x = synth.random_rows(17600 + case, M, N, dtype="f32", scale=3.0)
    y_rows = orc.softmax_fwd(x)
    y_h = synth.random_rows(17700 + case, M, N, ld=ld, dtype=dtype, scale=0.0, pad_nan=ld > N)
    y_h[:, :N] = synth.bf16_bits_from_f32(y_rows.astype(np.float32)) if dtype == "bf16" \
        else y_rows.astype(np.float32)
    dy_h = synth.random_rows(17800 + case, M, N, ld=ld, dtype=dtype, scale=1.0, pad_nan=ld > N)
    want = orc.softmax_bwd(np.ascontiguousarray(y_h[:, :N]), np.ascontiguousarray(dy_h[:, :N]))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    outs = []
    for grid in (0, 1):
        xr.set_option("grid", grid)
        p = xr.plan("softmax_bwd", M, N, tdt, aligned=1)
        y, dy = to_device(y_h), to_device(dy_h)
        dx = torch.full((M, ld), float("nan"), dtype=tdt, device="cuda")
        xr.softmax_bwd(y[:, :N], dy[:, :N], dx[:, :N])
        torch.cuda.synchronize()
        got = to_host(dx)
        check_output(np.ascontiguousarray(got[:, :N]), want, f"case {case} grid {grid} {p['path']}",
                     softmax_bwd_allow(y_h[:, :N], dy_h[:, :N]))
        outs.append(got[:, :N].copy())
    assert np.array_equal(outs[0].view(np.uint8), outs[1].view(np.uint8)), "forms differ"


@pytest.mark.parametrize("case", range(CASES))
def test_random_nll(orc, case):
    rng = np.random.Generator(np.random.PCG64(18000 + case))
    M, N, dtype, ld, path = draw(rng, case)
    x = synth.random_rows(18100 + case, M, N, ld=ld, dtype=dtype, scale=3.0, pad_nan=ld > N)
    x, off = shift_rows(18300 + case, x, N, dtype)
    print(f"nll case {case}: M={M} N={N} ld={ld} {dtype} path={path} "
          f"offsets={None if off is None else sorted(set(off.tolist()))}", flush=True)
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
    check_nll(got, to_host(loss), want, wl, f"case {case} nll", x)


@pytest.mark.parametrize("case", range(12))
def test_random_layernorm(orc, case):
    rng = np.random.Generator(np.random.PCG64(19000 + case))
    M = int(rng.choice([1, 5, 64, 700]))
    N = int(rng.choice([8, 16, 1000, 1001, 4096, 12288, 20000]))
    dtype = str(rng.choice(["f32", "bf16"]))
    ld = N + int(rng.choice([0, 0, 8, 3]))
    path = int(rng.choice([0, 0, 1, 3]))
    eps = float(rng.choice([1e-5, 1e-3, 0.5]))
    print(f"layernorm case {case}: M={M} N={N} ld={ld} {dtype} path={path} eps={eps}", flush=True)
    x = synth.random_rows(19100 + case, M, N, ld=ld, dtype=dtype, scale=2.0, pad_nan=ld > N)
    dy = synth.random_rows(19200 + case, M, N, ld=ld, dtype=dtype, scale=1.0, pad_nan=ld > N)
    wb = synth.random_rows(19300 + case, 2, N, dtype=dtype, scale=1.0)
    w_h, b_h = np.ascontiguousarray(wb[0]), np.ascontiguousarray(wb[1])
    force(path, N, dtype)
    from test_gpu_layernorm import run_case
    try:
        run_case(orc, x, w_h, b_h, dy, N, eps, f"layernorm case {case}")
    except xr.XrError as e:
        assert path == 1 and e.status == 2, e  # rows these sizes cannot hold in registers


@pytest.mark.parametrize("case", range(12))
def test_random_element_mul(orc, case):
    rng = np.random.Generator(np.random.PCG64(20000 + case))
    M = int(rng.choice([1, 3, 100, 2000]))
    N = int(rng.choice([1, 5, 8, 1000, 8193, 70000]))
    dtype = str(rng.choice(["f32", "bf16"]))
    ld = N + int(rng.choice([0, 1, 8]))
    per_row = bool(rng.integers(2))
    print(f"element_mul case {case}: M={M} N={N} ld={ld} {dtype} per_row={per_row}", flush=True)
    x = synth.random_rows(20100 + case, M, N, ld=ld, dtype=dtype, scale=2.0, pad_nan=ld > N)
    if per_row:
        s = synth.random_rows(20200 + case, 1, M, dtype="f32", scale=2.0)[0]
        s[::3] = 1.0
        s_dev, s_host = to_device(s), s.astype(np.float64)
    else:
        s_host = float(rng.choice([0.25, -3.0, 1.0]))
        s_dev = torch.tensor([s_host], dtype=torch.float32, device="cuda")
    xd = to_device(x)
    xr.element_mul(xd[:, :N], s_dev)
    torch.cuda.synchronize()
    got = to_host(xd)
    want = orc.element_mul(x, s_host, n_cols=N)
    from test_gpu_reductions import check_products
    check_products(got[:, :N], want, float(np.max(np.abs(np.atleast_1d(s_host)))), f"case {case}")
    if ld > N:
        assert np.array_equal(got[:, N:].view(np.uint8), x[:, N:].view(np.uint8))
