"""GPU parity of the softmax forward and backward over split rows (xr_softmax_fwd_ex /
xr_softmax_bwd_ex with a workspace: several workgroups per row exchanging (max, sum) pairs
or partial dot products) against the float64 oracle, with the suite's tolerances (fp32
within 1e-5 absolute, bf16 within 2e-2 relative of the row's scale). Covers long rows, rows
too few to fill the GPU, forced chunk counts (including chunks left empty), in-place calls,
row pitches, -inf entries, determinism and the workspace's argument checks."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_output, check_probs, to_device, to_host, widen

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


def fwd_bwd(x_h: np.ndarray, dy_h: np.ndarray, N: int, workspace=None):
    x, dy = to_device(x_h), to_device(dy_h)
    y = xr.softmax_fwd(x[:, :N], workspace=workspace)
    dx = xr.softmax_bwd(y, dy[:, :N], workspace=workspace)
    torch.cuda.synchronize()
    return to_host(y), to_host(dx)


def check(orc, x_h, dy_h, N, y_h, dx_h, what):
    check_probs(y_h, orc.softmax_fwd(x_h, n_cols=N), f"{what} forward")
    # the backward on the GPU's own y isolates the backward kernel
    check_output(dx_h, orc.softmax_bwd(y_h, np.ascontiguousarray(dy_h[:, :N])),
                 f"{what} backward")


# (M, N, dtype): long rows (64 KB chunks up to 512 KB rows, 128 KB above), 32-64 KB rows (16 KB chunks), rows
# too few for the GPU (chunks for every compute unit), ragged sizes, and batches whose rows
# are written back in groups of 8 (chunks of 32 KiB and more, at most 8 per row; the last
# group cut short by M).
SHAPES = [(1, 300001, "bf16"), (3, 70001, "f32"), (5, 128256, "bf16"), (64, 40000, "bf16"),
          (200, 20000, "f32"), (7, 5000, "f32"), (2, 1 << 20, "f32"), (16, 262147, "bf16"),
          (300, 8193, "f32"), (261, 66000, "bf16"), (259, 40000, "f32")]


@pytest.mark.parametrize("M,N,dtype", SHAPES, ids=[f"{m}x{n}-{d}" for m, n, d in SHAPES])
def test_split_shapes(orc, M, N, dtype):
    fw = xr.plan("softmax_fwd_ws", M, N, torch.float32 if dtype == "f32" else torch.bfloat16)
    bw = xr.plan("softmax_bwd_ws", M, N, torch.float32 if dtype == "f32" else torch.bfloat16)
    print(f"split {M}x{N} {dtype}: forward S={fw['split']}, backward S={bw['split']}", flush=True)
    assert fw["split"] > 1 and bw["split"] > 1, "these sizes are meant to take the split path"
    x = synth.random_rows(19000 + N % 97, M, N, dtype=dtype, scale=3.0)
    dy = synth.random_rows(19001 + N % 97, M, N, dtype=dtype, scale=1.0)
    y, dx = fwd_bwd(x, dy, N)
    check(orc, x, dy, N, y, dx, f"{M}x{N} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forced_chunk_counts(orc, dtype):
    """Chunk counts from 2 to far more chunks than the row has vectors (empty chunks), each
    against the oracle and bit-identical to the whole-row result where that is exact."""
    M, N = 37, 3001
    x = synth.random_rows(19100, M, N, dtype=dtype, scale=3.0)
    dy = synth.random_rows(19101, M, N, dtype=dtype, scale=1.0)
    for S in (2, 3, 7, 64, 1000):
        xr.set_option("split", S)
        xr.set_option("path", 2)
        print(f"{dtype} forced S={S}", flush=True)
        y, dx = fwd_bwd(x, dy, N)
        check(orc, x, dy, N, y, dx, f"{dtype} S={S}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_in_place_and_pitches(orc, dtype):
    """y == x for the forward, dx == dy and dx == y for the backward, on rows with a pitch
    (rows at varying addresses modulo 16, all operands sharing it); padding untouched."""
    M, N, ld = 9, 90001, 90013
    x_h = synth.random_rows(19200, M, N, ld=ld, dtype=dtype, scale=3.0, pad_nan=True)
    dy_h = synth.random_rows(19201, M, N, ld=ld, dtype=dtype, scale=1.0, pad_nan=True)
    assert xr.plan("softmax_fwd_ws", M, N, torch.float32, aligned=1)["split"] > 1
    want_y = orc.softmax_fwd(x_h, n_cols=N)
    x = to_device(x_h)
    xr.softmax_fwd(x[:, :N], x[:, :N])
    torch.cuda.synchronize()
    full = to_host(x)
    y_h = np.ascontiguousarray(full[:, :N])
    check_probs(y_h, want_y, f"{dtype} in place forward")
    assert np.array_equal(full[:, N:].view(np.uint8), x_h[:, N:].view(np.uint8)), "padding"
    want_dx = orc.softmax_bwd(y_h, np.ascontiguousarray(dy_h[:, :N]))
    # dx written over dy
    dy = to_device(dy_h)
    xr.softmax_bwd(x[:, :N], dy[:, :N], dy[:, :N])
    torch.cuda.synchronize()
    full = to_host(dy)
    check_output(np.ascontiguousarray(full[:, :N]), want_dx, f"{dtype} dx over dy")
    assert np.array_equal(full[:, N:].view(np.uint8), dy_h[:, N:].view(np.uint8)), "padding"
    # dx written over y
    dy = to_device(dy_h)
    xr.softmax_bwd(x[:, :N], dy[:, :N], x[:, :N])
    torch.cuda.synchronize()
    check_output(np.ascontiguousarray(to_host(x)[:, :N]), want_dx, f"{dtype} dx over y")


def test_split_neg_inf_and_constant_rows(orc):
    """Rows with -inf runs that leave whole chunks at -inf, a constant row, one finite
    entry per row: the chunk combine must weigh empty chunks as zero."""
    M, N = 6, 200000
    x = synth.random_rows(19300, M, N, dtype="f32", scale=3.0)
    dy = synth.random_rows(19301, M, N, dtype="f32", scale=1.0)
    x[0, : N // 2] = -np.inf          # first half of the row (whole chunks) at -inf
    x[1, N // 3:] = -np.inf           # tail chunks at -inf
    x[2, :] = 1.25                    # constant: 1 / N everywhere
    x[3, :] = -np.inf
    x[3, 12345] = 0.0                 # a single finite entry: probability 1
    x[4, ::2] = -np.inf
    y, dx = fwd_bwd(x, dy, N)
    check(orc, x, dy, N, y, dx, "-inf / constant rows")
    assert y[3, 12345] == 1.0 and np.count_nonzero(y[3]) == 1


def test_split_deterministic(orc):
    """Chunk-ordered combines: repeated calls give the same bits."""
    M, N = 4, 500000
    x = to_device(synth.random_rows(19400, M, N, dtype="bf16", scale=3.0))
    dy = to_device(synth.random_rows(19401, M, N, dtype="bf16", scale=1.0))
    outs = []
    for _ in range(3):
        y = xr.softmax_fwd(x)
        outs.append((to_host(y), to_host(xr.softmax_bwd(y, dy))))
    for y, dx in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(dx, outs[0][1])


def test_split_agrees_with_whole_rows(orc):
    """The same rows whole (no workspace, one workgroup per row) and split: both within the
    tolerance of the oracle, and within a few roundings of each other."""
    M, N = 12, 150000
    x = synth.random_rows(19500, M, N, dtype="f32", scale=3.0)
    dy = synth.random_rows(19501, M, N, dtype="f32", scale=1.0)
    y1, dx1 = fwd_bwd(x, dy, N, workspace=False)
    y2, dx2 = fwd_bwd(x, dy, N)
    check(orc, x, dy, N, y1, dx1, "whole rows")
    check(orc, x, dy, N, y2, dx2, "split rows")
    assert np.max(np.abs(widen(y1) - widen(y2))) <= 1e-6


def test_sm_vocab_sampled(orc):
    """The long-row softmax workload (4096 x 128256 bf16, forward + backward) in the launch
    configuration the benchmark times (split rows through one shared workspace), on sampled
    rows; every row's sum checked."""
    w = synth.softmax_long()
    M, N = w["M"], w["N"]
    x, dy = to_device(w["x"]), to_device(w["dy"])
    ws = torch.empty(xr.softmax_workspace_bytes(M, N, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    y = xr.softmax_fwd(x, workspace=ws)
    dx = xr.softmax_bwd(y, dy, workspace=ws)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2, 1000, 2047, 4000, M - 1])
    idx = torch.from_numpy(rows).cuda()
    y_h, dx_h = to_host(y[idx]), to_host(dx[idx])
    check(orc, w["x"][rows], w["dy"][rows], N, y_h, dx_h, "4096 x 128256 sampled rows")
    s = y.float().sum(dim=1).cpu().numpy()
    assert np.max(np.abs(s - 1.0)) < 2e-2 * 1.0 + 1e-3


def test_sm_few_sampled(orc):
    """The few-row softmax workload (16 x 2^20 fp32, forward + backward), every row."""
    w = synth.softmax_few()
    M, N = w["M"], w["N"]
    y, dx = fwd_bwd(w["x"], w["dy"], N)
    check(orc, w["x"], w["dy"], N, y, dx, "16 x 2^20 fp32")


def test_workspace_errors():
    M, N = 4, 100000
    x = torch.randn(M, N, device="cuda")
    y = torch.empty_like(x)
    need = xr.softmax_workspace_bytes(M, N, torch.float32)
    # each direction's own need: a counts block and one slot per row chunk
    nf = 256 + 8 * M * xr.plan("softmax_fwd_ws", M, N, torch.float32)["split"]
    nb = 256 + 8 * M * xr.plan("softmax_bwd_ws", M, N, torch.float32)["split"]
    assert nf > 256 and nb > 256 and need == max(nf, nb)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f, g = xr.lib.xr_softmax_fwd_ex, xr.lib.xr_softmax_bwd_ex
    # too small
    assert f(y.data_ptr(), N, x.data_ptr(), N, M, N, xr.F32, ws.data_ptr(), nf - 8, s) == 6
    assert g(y.data_ptr(), N, y.data_ptr(), N, x.data_ptr(), N, M, N, xr.F32, ws.data_ptr(),
             nb - 8, s) == 6
    # the workspace inside an operand
    assert f(y.data_ptr(), N, x.data_ptr(), N, M, N, xr.F32, x.data_ptr() + 64, need, s) == 5
    assert g(y.data_ptr(), N, y.data_ptr(), N, x.data_ptr(), N, M, N, xr.F32,
             y.data_ptr() + 4096, need, s) == 5
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stream_long_rows_without_workspace(orc, dtype):
    """Rows longer than any row-resident shape and no workspace: the two-pass stream
    kernels (vector loads), with the output sharing the input's alignment (vector stores)
    and not sharing it (element stores)."""
    M, N = 3, (1 << 20) + 5
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    assert xr.plan("softmax_fwd", M, N, dt)["path"] == "stream"
    assert xr.plan("softmax_bwd", M, N, dt)["path"] == "stream"
    x = synth.random_rows(19600, M, N, dtype=dtype, scale=3.0)
    dy = synth.random_rows(19601, M, N, dtype=dtype, scale=1.0)
    y, dx = fwd_bwd(x, dy, N, workspace=False)
    check(orc, x, dy, N, y, dx, f"stream {dtype}")
    # an output one element further along each row: other alignment, element stores
    xd, dyd = to_device(x), to_device(dy)
    yo = torch.empty((M, N + 1), dtype=dt, device="cuda")[:, 1:]
    xr.softmax_fwd(xd, yo, workspace=False)
    dxo = torch.empty((M, N + 1), dtype=dt, device="cuda")[:, 1:]
    xr.softmax_bwd(yo, dyd, dxo, workspace=False)
    torch.cuda.synchronize()
    y2 = to_host(yo)
    check_probs(y2, orc.softmax_fwd(x), f"stream {dtype} other alignment forward")
    check_output(to_host(dxo), orc.softmax_bwd(y2, dy), f"stream {dtype} other alignment backward")


def test_plans_for_rows_beyond_the_resident_chunks():
    """A split row's chunks must be able to be resident together; rows of hundreds of MB,
    whose chunks could not, take the stream kernels, rows of tens of MB still split."""
    bf = torch.bfloat16
    assert xr.plan("softmax_fwd_ws", 1, 1 << 24, bf)["path"] == "split"
    for op in ("softmax_fwd_ws", "softmax_bwd_ws", "xent", "nll_fwd"):
        assert xr.plan(op, 1, 1 << 29, bf)["path"] == "stream", op


def test_stream_row_across_windows(orc):
    """One bf16 row of 2^29 + 37 elements (just over 1 GiB): the stream kernels walk it in
    1 GiB windows, so the second window starts mid-row; every element is checked against
    the oracle, slice by slice."""
    M, N = 1, (1 << 29) + 37
    x = synth.random_rows(19700, M, N, dtype="bf16", scale=3.0)
    assert xr.plan("softmax_fwd", M, N, torch.bfloat16)["path"] == "stream"
    xd = to_device(x)
    y = xr.softmax_fwd(xd, workspace=False)
    torch.cuda.synchronize()
    y_h = to_host(y)
    del xd, y
    want = orc.softmax_fwd(x)
    rmax = float(np.max(want))
    step = 1 << 24
    worst = 0.0
    for a in range(0, N, step):
        g = widen(y_h[:, a:a + step])
        o = want[:, a:a + step]
        denom = np.maximum(np.abs(o), max(2.0 ** -7 * rmax, 5e-5 * rmax))
        worst = max(worst, float(np.max(np.abs(g - o) / denom)))
    print(f"2^29 + 37 row: worst scaled error {worst:.3e}", flush=True)
    assert worst <= 2e-2
    s = float(np.sum(widen(y_h)))
    assert abs(s - 1.0) < 1e-2, s


@pytest.mark.parametrize("shape,dtype", [((3, 5, 1000), "f32"), ((2, 3, 70001), "bf16"),
                                         ((4, 300000), "f32")],
                         ids=["3x5x1000-f32", "2x3x70001-bf16", "4x300000-f32"])
def test_softmax_autograd(orc, shape, dtype):
    """xr.softmax as an autograd function: the forward against the oracle, and x.grad for an
    upstream gradient w against the oracle's backward on the GPU's own y."""
    N = shape[-1]
    M = int(np.prod(shape[:-1]))
    x_h = synth.random_rows(19800 + N % 89, M, N, dtype=dtype, scale=3.0)
    w_h = synth.random_rows(19801 + N % 89, M, N, dtype=dtype, scale=1.0)
    x = to_device(x_h).reshape(shape).requires_grad_(True)
    w = to_device(w_h).reshape(shape)
    y = xr.softmax(x)
    (y * w).sum().backward()
    torch.cuda.synchronize()
    y_h = to_host(y.detach().reshape(M, N))
    check_probs(y_h, orc.softmax_fwd(x_h), f"autograd {shape} forward")
    # the upstream gradient is w rounded to the dtype: exactly w_h
    check_output(to_host(x.grad.reshape(M, N)), orc.softmax_bwd(y_h, w_h),
                 f"autograd {shape} backward")


def _rows_correct_or_nan(got: np.ndarray, want: np.ndarray, what: str) -> int:
    """Every row either passes the suite's check or holds NaN; returns the NaN rows."""
    g = widen(got)
    bad = 0
    for i in range(g.shape[0]):
        if np.isnan(g[i]).any():
            bad += 1
            continue
        check_output(got[i:i + 1], want[i:i + 1], f"{what} row {i}")
    return bad


def test_exchange_that_does_not_wait(orc):
    """The bounded wait of the split-row exchange, forced from the host (XR_OPT_NO_WAIT: a
    chunk reads each partner's slot once and gives up if it is not yet published): every
    call returns, the cross-entropy reports the timeout flag, every row is either correct
    or NaN; the same workspace then gives exact results again once the option is off."""
    M, V = 64, 128256
    x_h = synth.random_rows(19900, M, V, dtype="bf16", scale=2.0)
    t_h = synth.random_targets(19901, M, V)
    assert xr.plan("xent", M, V, torch.bfloat16)["split"] > 1
    ws = torch.empty(max(xr.xent_workspace_bytes(M, V, torch.bfloat16),
                         xr.softmax_workspace_bytes(M, V, torch.bfloat16)),
                     dtype=torch.uint8, device="cuda")
    g_want, l_want, _, _ = orc.xent(x_h, t_h, V)
    sm_want = orc.softmax_fwd(x_h)
    for no_wait in (1, 0):
        xr.set_option("no_wait", no_wait)
        xd = to_device(x_h)
        _, rows, counts = xr.xent_fwd_bwd(xd, to_device(t_h), workspace=ws)
        y = xr.softmax_fwd(to_device(x_h), workspace=ws)
        torch.cuda.synchronize()
        c = to_host(counts).tolist()
        assert c[2] == no_wait, c
        nan_g = _rows_correct_or_nan(to_host(xd), g_want, f"no_wait={no_wait} gradient")
        nan_y = _rows_correct_or_nan(to_host(y), sm_want, f"no_wait={no_wait} softmax")
        loss = to_host(rows).astype(np.float64)
        ok = np.isnan(loss) | (np.abs(loss - l_want) <= 1e-4 * np.abs(l_want) + 1e-5)
        assert ok.all()
        print(f"no_wait={no_wait}: {nan_g} NaN gradient rows, {nan_y} NaN softmax rows, "
              f"{int(np.isnan(loss).sum())} NaN losses", flush=True)
        if not no_wait:
            assert nan_g == 0 and nan_y == 0 and not np.isnan(loss).any()


def test_workspace_status_reports_the_timeout(orc):
    """xr_workspace_status: the softmax forward / backward and the negative log-softmax report
    a timed-out exchange (forced from the host) in the workspace's status word, and a later
    call on the same workspace leaves it defined again: 0 after split rows that completed,
    0 after rows that were not split at all."""
    M, N = 16, 262147
    x_h = synth.random_rows(19950, M, N, dtype="bf16", scale=2.0)
    dy_h = synth.random_rows(19951, M, N, dtype="bf16", scale=1.0)
    idx = synth.random_targets(19952, M, N)
    assert xr.plan("softmax_fwd_ws", M, N, torch.bfloat16)["split"] > 1
    assert xr.plan("softmax_bwd_ws", M, N, torch.bfloat16)["split"] > 1
    assert xr.plan("nll_fwd", M, N, torch.bfloat16)["split"] > 1
    ws = torch.empty(max(xr.softmax_workspace_bytes(M, N, torch.bfloat16),
                         int(xr.lib.xr_nll_fwd_workspace_bytes(M, N, xr.BF16))),
                     dtype=torch.uint8, device="cuda")
    x, dy = to_device(x_h), to_device(dy_h)
    small = to_device(synth.random_rows(19953, 4, 100, dtype="bf16", scale=2.0))
    assert xr.plan("softmax_fwd_ws", 4, 100, torch.bfloat16)["split"] == 1

    def status():
        return int(xr.workspace_status(ws).item())

    for no_wait in (1, 0):
        xr.set_option("no_wait", no_wait)
        y = xr.softmax_fwd(x, workspace=ws)
        assert status() == no_wait, f"softmax forward, no_wait={no_wait}"
        xr.softmax_bwd(y, dy, workspace=ws)
        assert status() == no_wait, f"softmax backward, no_wait={no_wait}"
        xr.nll_fwd(x, to_device(idx), workspace=ws)
        assert status() == no_wait, f"negative log-softmax, no_wait={no_wait}"
        if no_wait:
            xr.set_option("no_wait", 0)
            xr.softmax_fwd(small, workspace=ws)  # rows held whole: the word is cleared
            assert status() == 0, "a call without split rows leaves 0"
            xr.set_option("no_wait", 1)
            xr.softmax_fwd(x, workspace=ws)
            assert status() == 1
            xr.softmax_bwd(xr.softmax_fwd(small, workspace=False), small, workspace=ws)
            assert status() == 0, "the backward without split rows leaves 0"
    y = xr.softmax_fwd(x, workspace=ws)
    check_probs(to_host(y), orc.softmax_fwd(x_h), "after the forced timeouts")


def test_empty_batches():
    """Zero rows: every call succeeds, enqueues nothing and returns empty results."""
    for dt in (torch.float32, torch.bfloat16):
        x = torch.empty((0, 1000), dtype=dt, device="cuda")
        y = xr.softmax_fwd(x)
        dx = xr.softmax_bwd(y, torch.empty_like(x))
        assert y.shape == (0, 1000) and dx.shape == (0, 1000)
        out, loss = xr.nll_fwd(x, torch.empty(0, dtype=torch.int64, device="cuda"))
        assert out.shape == (0, 1000) and loss.numel() == 0
        w = torch.ones(1000, dtype=dt, device="cuda")
        b = torch.zeros(1000, dtype=dt, device="cuda")
        yl, mean, rstd = xr.layernorm_fwd(x, w, b)
        assert yl.shape == (0, 1000) and mean.numel() == 0
        xr.element_mul(x, 2.0)
    torch.cuda.synchronize()
