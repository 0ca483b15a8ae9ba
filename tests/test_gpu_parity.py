"""GPU parity: the HIP library against the float64 oracle, element by element.

Inputs come from the seeded generators in ``synth``; expected values only from
``oracle``. Cases cover the five benchmark workloads (at full size; the largest
ones compare every row loss, the mean and a sample of full gradient rows, plus
properties that hold on every row), several-tile and ragged sizes, unaligned row
starts and strides, degenerate rows and batches, every launch path, and
run-to-run determinism.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import synth
from gpu_util import (check_bf16, check_fp32, check_losses, check_output, check_probs,
                      check_xent_grad, to_device, to_host, widen)

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


def run_xent(x_host: np.ndarray, target: np.ndarray, V: int, ignore_index: int = -100):
    """Run the library on a copy of x_host (M, ld); returns (grad bits/values (M, ld), rows, mean, counts)."""
    x = to_device(x_host)
    t = to_device(target)
    mean, rows, counts = xr.xent_fwd_bwd(x[:, :V], t, ignore_index)
    torch.cuda.synchronize()
    return to_host(x), to_host(rows), float(mean.item()), to_host(counts)


def compare_xent(orc, x_host, target, V, grad_gpu, rows_gpu, mean_gpu, counts_gpu, what,
                 ignore_index=-100, rows=None, grad_rows=None):
    """Counts, every row loss, the mean, and the gradient of every row (rows=None: grad_gpu is
    the whole (M, ld) matrix, whose padding must be unchanged) or of the listed rows
    (grad_gpu[i] is row rows[i]); with grad_rows, every row's gradient is fetched through
    grad_rows(row indices) 256 rows at a time instead."""
    n, bad = orc.xent_count(target, V, ignore_index)
    assert int(counts_gpu[0]) == n and int(counts_gpu[1]) == bad, f"{what}: counts"
    assert int(counts_gpu[2]) == 0, f"{what}: error flags {int(counts_gpu[2])}"
    _, loss_all = orc.xent_rows(x_host, target, V, n, ignore_index, want_grad=False)
    check_losses(rows_gpu, mean_gpu, loss_all, orc.mean(loss_all, n), what)
    sel = np.arange(x_host.shape[0]) if rows is None else np.asarray(rows)
    for c0 in range(0, sel.size, 256):
        part = sel[c0:c0 + 256]
        g, _ = orc.xent_rows(x_host, target, V, n, ignore_index, rows=part)
        if grad_rows is not None:
            got = grad_rows(part)[:, :V]
        else:
            got = grad_gpu[part, :V] if rows is None else grad_gpu[c0:c0 + 256, :V]
        check_xent_grad(got, g, target[part], V, n, f"{what} rows {part[0]}..",
                        ignore_index=ignore_index)
    if rows is None and grad_rows is None and x_host.shape[1] > V:
        assert np.array_equal(grad_gpu[:, V:].view(np.uint8), x_host[:, V:].view(np.uint8)), \
            f"{what}: padding changed"


# ----------------------------------------------------------------------------- worked examples
def test_worked_examples():
    with open(oracle_pins.GOLDEN) as f:
        gold = json.load(f)
    for case in gold["softmax_fwd"]:
        x = oracle_pins.as_input(case["x"], case["dtype"])
        y = to_host(xr.softmax_fwd(to_device(x)))
        want = np.array([[oracle_pins.closed_form(v) for v in r] for r in case["y"]])
        check_probs(y, want, case["name"])
    for case in gold["softmax_bwd"]:
        y = oracle_pins.as_input(case["y"], case["dtype"])
        dy = oracle_pins.as_input(case["dy"], case["dtype"])
        dx = to_host(xr.softmax_bwd(to_device(y), to_device(dy)))
        want = np.array([[oracle_pins.closed_form(v) for v in r] for r in case["dx"]])
        check_output(dx, want, case["name"])
    for case in gold["xent"]:
        x = oracle_pins.as_input(case["x"], case["dtype"])
        t = np.array(case["target"], dtype=np.int64)
        g, rows, mean, counts = run_xent(x, t, x.shape[1], case["ignore_index"])
        assert int(counts[0]) == case["n"]
        want_g = np.array([[oracle_pins.closed_form(v) for v in r] for r in case["grad"]])
        check_xent_grad(g, want_g, t, x.shape[1], case["n"], case["name"],
                        ignore_index=case["ignore_index"])
        want_l = np.array([oracle_pins.closed_form(v) for v in case["loss"]])
        check_losses(rows, mean, want_l, oracle_pins.closed_form(case["mean"]), case["name"])


# ----------------------------------------------------------------------------- the five workloads
def test_c1_softmax_fp32(orc):
    w = synth.softmax_c1()
    y = to_host(xr.softmax_fwd(to_device(w["x"])))
    check_probs(y, orc.softmax_fwd(w["x"]), "c1 softmax")


def test_c2_softmax_fwd_bwd_bf16(orc):
    w = synth.softmax_c2()
    x, dy = to_device(w["x"]), to_device(w["dy"])
    y = xr.softmax_fwd(x)
    dx = xr.softmax_bwd(y, dy)
    y_h, dx_h = to_host(y), to_host(dx)
    check_probs(y_h, orc.softmax_fwd(w["x"]), "c2 softmax forward")
    # The backward is checked on the GPU's own bf16 y, which isolates the backward kernel.
    check_bf16(dx_h, orc.softmax_bwd(y_h, w["dy"]), "c2 softmax backward")
    # dx rows sum to ~0 (sum y ~ 1 up to bf16 rounding of y).
    s = widen(dx_h).sum(axis=1)
    assert np.max(np.abs(s)) < 0.05
    # The forward -> backward chain against the oracle's own y (float64, held as float32):
    # it carries the bf16 rounding of y into dx, so it is reported, with a looser bound.
    y_orc = orc.softmax_fwd(w["x"]).astype(np.float32)
    dy32 = widen(w["dy"]).astype(np.float32)
    chain = orc.softmax_bwd(y_orc, dy32)
    g = widen(dx_h)
    floor = 2.0 ** -7 * np.max(np.abs(chain), axis=1, keepdims=True)
    worst = float(np.max(np.abs(g - chain) / np.maximum(np.abs(chain), floor)))
    print(f"c2 forward -> backward chain vs the oracle's y: worst scaled error {worst:.3e}")
    assert worst <= 0.1


def test_c3_xent_bf16(orc):
    w = synth.xent_c3()
    g, rows, mean, counts = run_xent(w["x"], w["target"], w["N"])
    compare_xent(orc, w["x"], w["target"], w["N"], g, rows, mean, counts, "c3")


def test_c4_xent_bf16_large_vocab(orc):
    """The metric's workload at full size: counts, every row loss, the mean, and every entry
    of all 16384 gradient rows (copied back and compared 256 rows at a time)."""
    w = synth.xent_c4()
    x_host, t, V = w["x"], w["target"], w["N"]
    x = to_device(x_host)
    mean, rows, counts = xr.xent_fwd_bwd(x, to_device(t), -100)
    torch.cuda.synchronize()
    compare_xent(orc, x_host, t, V, None, to_host(rows), float(mean.item()), to_host(counts),
                 "c4", grad_rows=lambda part: to_host(x[torch.from_numpy(part).cuda()]))


def test_c5_xent_fp32_padded(orc):
    w = synth.xent_c5()
    V = w["N"]
    g, rows, mean, counts = run_xent(w["x"], w["target"], V)
    compare_xent(orc, w["x"], w["target"], V, g, rows, mean, counts, "c5")
    # Special rows: the all-equal rows have loss log V, -inf entries get exactly 0.
    assert np.allclose(rows[w["equal_rows"]], math.log(V), rtol=1e-5)
    for r in w["half_inf_rows"]:
        assert np.all(g[r, :V][np.isneginf(w["x"][r, :V])] == 0.0)


# ----------------------------------------------------------------------------- shapes and layouts
XENT_SHAPES = [
    # (M, V, ld, dtype, ignore_frac, scale)
    (1, 1, 1, "f32", 0.0, 1.0),
    (3, 7, 7, "bf16", 0.0, 2.0),
    (5, 8, 8, "bf16", 0.2, 2.0),
    (17, 100, 103, "bf16", 0.2, 3.0),
    (9, 1000, 1000, "f32", 0.1, 3.0),
    (33, 4099, 4101, "bf16", 0.1, 2.0),
    (64, 32005, 32005, "bf16", 0.1, 2.0),
    (7, 32000, 32003, "f32", 0.0, 8.0),
    (300, 5000, 5000, "bf16", 0.05, 1.0),
    (12, 128256, 128256, "bf16", 0.25, 1.0),
    (4, 131073, 131080, "bf16", 0.0, 1.0),
    (6, 256000, 256064, "f32", 0.0, 8.0),
    (3, 70001, 70001, "f32", 0.0, 4.0),
]


@pytest.mark.parametrize("M,V,ld,dtype,ign,scale", XENT_SHAPES,
                         ids=[f"{m}x{v}ld{l}-{d}" for m, v, l, d, _, _ in XENT_SHAPES])
def test_xent_shapes(orc, M, V, ld, dtype, ign, scale):
    x = synth.random_rows(7000 + M + V, M, V, ld=ld, dtype=dtype, scale=scale)
    t = synth.random_targets(8000 + M + V, M, V, ignore_frac=ign)
    if M >= 2:
        t[0], t[-1] = 0, V - 1  # first and last columns as targets
        if ign == 0.0 and M > 2:
            t[1] = -100
    g, rows, mean, counts = run_xent(x, t, V)
    compare_xent(orc, x, t, V, g, rows, mean, counts, f"xent {M}x{V}")


@pytest.mark.parametrize("shift", [1, 3, 5])
def test_xent_unaligned_rows(orc, shift):
    """Row starts off the 16-byte grid (a view that starts `shift` elements in)."""
    M, V, ld = 11, 3001, 3011
    x = synth.random_rows(9100 + shift, M, ld, dtype="bf16", scale=2.0)
    t = synth.random_targets(9200 + shift, M, V, ignore_frac=0.2)
    t[2] = V - 1
    xd = to_device(x)
    view = xd[:, shift:shift + V]
    mean, rows, counts = xr.xent_fwd_bwd(view, to_device(t))
    torch.cuda.synchronize()
    g = to_host(xd)
    sub = np.ascontiguousarray(x[:, shift:shift + V])
    compare_xent(orc, sub, t, V, np.ascontiguousarray(g[:, shift:shift + V]), to_host(rows),
                 float(mean.item()), to_host(counts), f"unaligned +{shift}")
    # Elements outside the view are untouched.
    assert np.array_equal(g[:, :shift], x[:, :shift])
    assert np.array_equal(g[:, shift + V:], x[:, shift + V:])


def test_xent_degenerate(orc):
    V = 4096
    x = synth.random_rows(9300, 6, V, dtype="bf16", scale=2.0)
    # Every row ignored: n = 0, zero gradient and loss, mean NaN.
    t = np.full(6, -100, dtype=np.int64)
    g, rows, mean, counts = run_xent(x, t, V)
    assert int(counts[0]) == 0 and math.isnan(mean)
    assert np.all(g == 0) and np.all(rows == 0)
    # Out-of-range targets are counted and their rows zeroed; they still count in n.
    t = np.array([5, -3, V, 7, -100, V - 1], dtype=np.int64)
    g, rows, mean, counts = run_xent(x, t, V)
    assert int(counts[1]) == 2
    assert np.all(g[[1, 2, 4]] == 0) and np.all(rows[[1, 2, 4]] == 0)
    assert int(counts[0]) == orc.xent_count(t, V)[0]
    # ignore_index inside [0, V) is compared first.
    t = np.array([3, 3, 0, 9, 3, 1], dtype=np.int64)
    g, rows, mean, counts = run_xent(x, t, V, ignore_index=3)
    compare_xent(orc, x, t, V, g, rows, mean, counts, "ignore_index=3", ignore_index=3)
    # M = 0: mean NaN, counts zero, nothing else touched.
    xd = torch.zeros((0, V), dtype=torch.bfloat16, device="cuda")
    mean, rows, counts = xr.xent_fwd_bwd(xd, torch.zeros(0, dtype=torch.int64, device="cuda"))
    assert math.isnan(mean.item()) and to_host(counts).tolist() == [0, 0, 0]


def test_xent_neg_inf_chunks(orc):
    """-inf runs covering whole workgroup chunks, and -inf in the first and last columns."""
    M, V = 4, 200000
    x = synth.random_rows(9400, M, V, dtype="f32", scale=4.0)
    x[0, :150000] = -np.inf
    x[1, 100:] = -np.inf
    x[2, ::2] = -np.inf
    x[3, 0] = -np.inf
    x[3, -1] = -np.inf
    t = np.array([160000, 5, 1, 17], dtype=np.int64)
    for path in (0, 2, 3):
        xr.set_option("path", path)
        g, rows, mean, counts = run_xent(x, t, V)
        compare_xent(orc, x, t, V, g, rows, mean, counts, f"-inf chunks path {path}")
        assert np.all(g[np.isneginf(x)] == 0)


# ----------------------------------------------------------------------------- paths
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_xent_all_paths_agree(orc, dtype):
    M, V = 40, 50000
    x = synth.random_rows(9500, M, V, dtype=dtype, scale=3.0)
    t = synth.random_targets(9501, M, V, ignore_frac=0.1)
    outs = {}
    for name, path, split, grid in (("auto", 0, 0, 0), ("resident", 1, 0, 0),
                                    ("resident-persistent", 1, 0, 2), ("split2", 2, 2, 0),
                                    ("split5", 2, 5, 0), ("split3-cooperative", 2, 3, 1),
                                    ("stream", 3, 0, 0)):
        xr.set_option("path", path)
        xr.set_option("split", split)
        xr.set_option("grid", grid)
        g, rows, mean, counts = run_xent(x, t, V)
        compare_xent(orc, x, t, V, g, rows, mean, counts, f"{dtype} {name}")
        outs[name] = g
    xr.reset_options()


@pytest.mark.parametrize("threads", [64, 128, 256, 512, 1024])
def test_xent_workgroup_sizes(orc, threads):
    M, V = 10, 8000
    x = synth.random_rows(9600, M, V, dtype="bf16", scale=2.0)
    t = synth.random_targets(9601, M, V, ignore_frac=0.2)
    xr.set_option("threads", threads)
    xr.set_option("split", 2 if threads == 64 else 0)
    g, rows, mean, counts = run_xent(x, t, V)
    compare_xent(orc, x, t, V, g, rows, mean, counts, f"threads {threads}")


@pytest.mark.parametrize("V,dtype,split,want", [
    (32000, "bf16", 0, (128, 8, 4)),    # 64 KB rows: four 16 KB chunks on 128 x 8
    (32000, "bf16", 2, (256, 8, 2)),    # the same rows forced into two 32 KB chunks
    (16000, "f32", 0, (128, 8, 4)),     # 64 KB fp32 rows
    (64000, "bf16", 0, (256, 16, 2)),   # 128 KB rows: two 64 KB chunks on 256 x 16
    (128256, "bf16", 0, (256, 16, 4)),  # 256 KB rows: four ~64 KB chunks on 256 x 16
    (128256, "bf16", 2, (512, 16, 2)),  # the same rows forced into two 128 KB chunks
    (256000, "f32", 0, (512, 16, 8)),   # 1 MB rows: eight 128 KB chunks (64 KB would be 16)
])
def test_xent_chunk_shapes(orc, V, dtype, split, want):
    """Cross-entropy chunks of up to 32 KB take the smallest shape of at most 8 vectors per
    thread that holds them; larger chunks (64 KB up to 512 KB rows, 128 KB above) the
    smallest shape that holds them; each plan matches the oracle."""
    M = 300
    xr.set_option("split", split)
    p = xr.plan("xent", M, V, torch.bfloat16 if dtype == "bf16" else torch.float32)
    assert (p["threads"], p["vec_per_thread"], p["split"]) == want, p
    x = synth.random_rows(9650 + V % 97, M, V, dtype=dtype, scale=2.0)
    t = synth.random_targets(9651 + V % 97, M, V, ignore_frac=0.1)
    g, rows, mean, counts = run_xent(x, t, V)
    compare_xent(orc, x, t, V, g, rows, mean, counts, f"V {V} {dtype} split {split}")


@pytest.mark.parametrize("M,V,dtype,ld", [
    (261, 66000, "bf16", None),   # three 43 KiB chunks per row; a last group of 5 rows
    (259, 40000, "f32", 40064),   # three 53 KB chunks per padded row; a last group of 3
    (264, 128256, "bf16", None),  # four 64 KB chunks per row; 33 whole groups
    (40, 256000, "f32", 256064),  # eight 128 KB chunks per row; 5 whole groups
])
def test_xent_write_groups(orc, M, V, dtype, ld):
    """Split rows with chunks of 32 KiB and more (at most 8 per row) are written back in
    groups of adjacent rows (a chunk holds its stores until its neighbours' chunks have
    published): ignored rows and out-of-range targets inside a group, and a last group cut
    short by M, give the oracle's results and leave no error flag."""
    x = synth.random_rows(9800 + M, M, V, ld=ld, dtype=dtype, scale=2.0)
    t = synth.random_targets(9801 + M, M, V, ignore_frac=0.25)
    t[min(3, M - 1)] = V + 5
    t[min(6, M - 1)] = -7
    p = xr.plan("xent", M, V, torch.bfloat16 if dtype == "bf16" else torch.float32)
    assert p["path"] == "split" and p["chunk_vecs"] * 16 >= 32 << 10 and p["group_rows"] == 8, p
    g, rows, mean, counts = run_xent(x, t, V)
    compare_xent(orc, x, t, V, g, rows, mean, counts, f"groups M {M} V {V} {dtype}")
    # the wait decides nothing: a second call gives bit-identical results
    g2, rows2, mean2, _ = run_xent(x, t, V)
    assert np.array_equal(g.view(np.uint8), g2.view(np.uint8)), "gradient differs between runs"
    assert np.array_equal(rows.view(np.uint8), rows2.view(np.uint8)) and mean == mean2


@pytest.mark.parametrize("M,V,dtype", [(300, 32000, "bf16"), (72, 128256, "bf16"),
                                       (33, 70001, "f32")])
def test_xent_write_groups_decide_nothing(orc, M, V, dtype):
    """Write groups forced off, automatic and forced on (XR_OPT_GROUPS 1, 0, 2) give
    bit-identical gradients and losses that match the oracle."""
    x = synth.random_rows(9850 + M, M, V, dtype=dtype, scale=2.0)
    t = synth.random_targets(9851 + M, M, V, ignore_frac=0.2)
    outs = []
    for groups in (1, 0, 2):
        xr.set_option("groups", groups)
        outs.append(run_xent(x, t, V))
    xr.set_option("groups", 0)
    g, rows, mean, counts = outs[1]
    compare_xent(orc, x, t, V, g, rows, mean, counts, f"groups {M}x{V} {dtype}")
    for g2, rows2, mean2, _ in outs[::2]:
        assert np.array_equal(g.view(np.uint8), g2.view(np.uint8)), "gradient differs"
        assert np.array_equal(rows.view(np.uint8), rows2.view(np.uint8)) and mean == mean2


@pytest.mark.parametrize("grid", [1, 2, -1])
def test_xent_grid_shapes(orc, grid):
    """Persistent grids (rows g, g + G, ... with the next row's loads issued while the
    current one is written) and one workgroup per row, on rows held whole and split."""
    M, V = 700, 3000
    x = synth.random_rows(9700, M, V, dtype="bf16", scale=2.0)
    t = synth.random_targets(9701, M, V, ignore_frac=0.1)
    xr.set_option("grid", grid)
    g, rows, mean, counts = run_xent(x, t, V)
    compare_xent(orc, x, t, V, g, rows, mean, counts, f"grid {grid}")
    M, V = 300, 40000
    x = synth.random_rows(9702, M, V, dtype="bf16", scale=2.0)
    t = synth.random_targets(9703, M, V, ignore_frac=0.1)
    assert xr.plan("xent", M, V, torch.bfloat16)["path"] == "split"
    g, rows, mean, counts = run_xent(x, t, V)
    compare_xent(orc, x, t, V, g, rows, mean, counts, f"split grid {grid}")


@pytest.mark.parametrize("M,V,dtype,path", [(600, 32000, "bf16", 0), (40, 50000, "f32", 3),
                                             (300, 5000, "bf16", 1), (9, 128256, "bf16", 0)])
def test_xent_row_loss_in_workspace(orc, M, V, dtype, path):
    """row_loss = NULL: the row losses are kept in the workspace (whose size query allows for
    them); the gradient, the mean and the sum match the oracle and, bit for bit, a call that
    is given row_loss."""
    x = synth.random_rows(9900 + M, M, V, dtype=dtype, scale=2.0)
    t = synth.random_targets(9901 + M, M, V, ignore_frac=0.1)
    xr.set_option("path", path)
    for reduction in ("mean", "sum"):
        a, b = to_device(x), to_device(x)
        la, ra, ca = xr.xent_fwd_bwd(a, to_device(t), reduction=reduction)
        lb, rb, cb = xr.xent_fwd_bwd(b, to_device(t), reduction=reduction, row_loss=False)
        torch.cuda.synchronize()
        assert rb is None
        assert torch.equal(a.view(torch.int16 if dtype == "bf16" else torch.int32),
                           b.view(torch.int16 if dtype == "bf16" else torch.int32))
        assert torch.equal(la, lb) and torch.equal(ca, cb)
        g, rows, red, (n, _) = orc.xent(x, t, V, reduction=reduction)
        check_xent_grad(to_host(b), g, t, V, n if reduction == "mean" else 1,
                        f"{M}x{V} {reduction} without row_loss")
        check_losses(to_host(ra), float(lb.item()), rows, red, f"{M}x{V} {reduction}",
                     mean_abs=1e-5 * (M if reduction == "sum" else 1))


def test_xent_deterministic():
    w = synth.xent_c3(M=600)
    outs = [run_xent(w["x"], w["target"], w["N"]) for _ in range(3)]
    for g, rows, mean, counts in outs[1:]:
        assert np.array_equal(g, outs[0][0]) and np.array_equal(rows, outs[0][1])
        assert mean == outs[0][2]


def test_xent_small_batch_uses_split(orc):
    p = xr.plan("xent", 8, 128256, torch.bfloat16)
    assert p["path"] == "split" and p["split"] > 1
    x = synth.random_rows(9800, 8, 128256, dtype="bf16", scale=1.0)
    t = synth.random_targets(9801, 8, 128256)
    g, rows, mean, counts = run_xent(x, t, 128256)
    compare_xent(orc, x, t, 128256, g, rows, mean, counts, "small batch")


# ----------------------------------------------------------------------------- softmax
SOFTMAX_SHAPES = [(1, 1, "f32"), (3, 2, "bf16"), (5, 7, "bf16"), (19, 257, "f32"),
                  (128, 1000, "f32"), (64, 4096, "bf16"), (8, 4099, "bf16"),
                  (6, 33333, "f32"), (4, 65536, "bf16"), (3, 70000, "f32"), (2, 300000, "bf16")]


@pytest.mark.parametrize("M,N,dtype", SOFTMAX_SHAPES, ids=[f"{m}x{n}-{d}" for m, n, d in SOFTMAX_SHAPES])
def test_softmax_shapes(orc, M, N, dtype):
    x = synth.random_rows(10000 + N, M, N, dtype=dtype, scale=3.0)
    dy = synth.random_rows(11000 + N, M, N, dtype=dtype, scale=1.0)
    y = xr.softmax_fwd(to_device(x))
    y_h = to_host(y)
    check_probs(y_h, orc.softmax_fwd(x), f"softmax {M}x{N}")
    dx = to_host(xr.softmax_bwd(y, to_device(dy)))
    check_output(dx, orc.softmax_bwd(y_h, dy), f"softmax bwd {M}x{N}")


def test_softmax_in_place_and_strides(orc):
    M, N, ld = 9, 3000, 3016
    x = synth.random_rows(12000, M, N, ld=ld, dtype="bf16", scale=3.0)
    want = orc.softmax_fwd(x, n_cols=N)
    xd = to_device(x)
    xr.softmax_fwd(xd[:, :N], xd[:, :N])  # exactly in place
    got = to_host(xd)
    check_probs(got[:, :N], want, "in place")
    assert np.array_equal(got[:, N:], x[:, N:]), "padding changed"
    # Output with a different row stride and alignment than the input (stream path).
    out = torch.full((M, N + 5), float("nan"), dtype=torch.bfloat16, device="cuda")
    xr.softmax_fwd(to_device(x)[:, :N], out[:, 1:N + 1])
    got = to_host(out)
    check_probs(got[:, 1:N + 1], want, "misaligned output")
    assert np.all(np.isnan(widen(got[:, 0]))) and np.all(np.isnan(widen(got[:, N + 1:])))


def test_softmax_bwd_aliases(orc):
    M, N = 7, 5000
    y = synth.random_rows(12100, M, N, dtype="f32", scale=0.01)
    dy = synth.random_rows(12101, M, N, dtype="f32", scale=1.0)
    want = orc.softmax_bwd(y, dy)
    yd, dyd = to_device(y), to_device(dy)
    xr.softmax_bwd(yd, dyd, dyd)  # dx == dy
    check_fp32(to_host(dyd), want, "dx == dy")
    yd, dyd = to_device(y), to_device(dy)
    xr.softmax_bwd(yd, dyd, yd)  # dx == y
    check_fp32(to_host(yd), want, "dx == y")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_softmax_bwd_grid_forms(orc, dtype):
    """The backward's two forms: one workgroup per row (the loop-free form the plans pick) and
    persistent grids of 1 and 2 workgroups per compute unit (rows r, r + G, ... with the next
    row's loads issued while the current one is written). Same bits from all three, matching
    the oracle; the rows' pitch puts partial vectors at both ends of most rows."""
    M, N, ld = 700, 3001, 3013
    y_h = synth.random_rows(12300, M, N, ld=ld, dtype=dtype, scale=0.01)
    dy_h = synth.random_rows(12301, M, N, ld=ld, dtype=dtype, scale=1.0)
    want = orc.softmax_bwd(np.ascontiguousarray(y_h[:, :N]), np.ascontiguousarray(dy_h[:, :N]))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    outs = []
    for grid in (0, 1, 2):
        xr.set_option("grid", grid)
        p = xr.plan("softmax_bwd", M, N, tdt, aligned=1)
        assert p["path"] == "resident" and (p["grid"] == M) == (grid == 0), p
        y, dy = to_device(y_h), to_device(dy_h)
        dx = torch.full((M, ld), float("nan"), dtype=tdt, device="cuda")
        xr.softmax_bwd(y[:, :N], dy[:, :N], dx[:, :N])
        got = to_host(dx)
        check_output(np.ascontiguousarray(got[:, :N]), want, f"{dtype} grid {grid}")
        assert np.all(np.isnan(widen(got[:, N:]))), "padding written"
        outs.append(got[:, :N].copy())
    xr.reset_options()
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint8), outs[0].view(np.uint8)), "forms differ"


def test_softmax_neg_inf(orc):
    x = synth.random_rows(12200, 5, 3000, dtype="f32", scale=3.0)
    x[0, :2999] = -np.inf
    x[1, ::3] = -np.inf
    y = to_host(xr.softmax_fwd(to_device(x)))
    check_probs(y, orc.softmax_fwd(x), "softmax -inf")
    assert np.all(y[np.isneginf(x)] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nonfinite_inputs(orc, dtype):
    """A row holding a NaN or a +inf gives NaN in every output of that row, on every launch
    path, as the oracle does: the softmax, its backward, the cross-entropy's gradient and row
    loss, and then the mean. An ignored row is not read, so a NaN in it changes nothing (zero
    gradient, zero loss). The other rows match the oracle as usual."""
    M, N = 6, 3001
    x = synth.random_rows(12300, M, N, dtype=dtype, scale=3.0)
    nan, inf = (0x7FC0, 0x7F80) if dtype == "bf16" else (np.nan, np.inf)
    x[1, 17] = nan
    x[3, 2900] = inf
    x[5, 0] = nan
    bad, good = [1, 3], [0, 2, 4]
    dy = synth.random_rows(12301, M, N, dtype=dtype, scale=1.0)
    t = synth.random_targets(12302, M, N)
    t[5] = -100
    for name, path, split in (("auto", 0, 0), ("resident", 1, 0), ("split2", 2, 2),
                              ("stream", 3, 0)):
        xr.set_option("path", path)
        xr.set_option("split", split)
        what = f"{dtype} {name}"
        # softmax forward and backward
        y = to_host(xr.softmax_fwd(to_device(x)))
        want = orc.softmax_fwd(x)
        assert np.array_equal(np.isnan(widen(y)), np.isnan(want)), f"{what}: softmax NaN pattern"
        assert np.all(np.isnan(widen(y)[bad + [5]])), f"{what}: softmax rows with NaN / +inf"
        check_probs(y[good], want[good], f"{what}: softmax")
        dx = to_host(xr.softmax_bwd(to_device(y), to_device(dy)))
        want_dx = orc.softmax_bwd(y, dy)
        assert np.array_equal(np.isnan(widen(dx)), np.isnan(want_dx)), f"{what}: backward NaN pattern"
        check_output(dx[good], want_dx[good], f"{what}: backward")
        # cross-entropy: row 5 is ignored, so its NaN is never read
        g, rows, mean, counts = run_xent(x, t, N)
        n, nbad = orc.xent_count(t, N, -100)
        assert int(counts[0]) == n and int(counts[1]) == nbad and int(counts[2]) == 0, what
        gw, lw = orc.xent_rows(x, t, N, n, -100)
        assert np.all(np.isnan(widen(g)[bad])) and np.all(np.isnan(gw[bad])), f"{what}: gradient"
        assert np.all(np.isnan(rows[bad])) and np.all(np.isnan(lw[bad])), f"{what}: row losses"
        assert np.all(widen(g)[5] == 0) and rows[5] == 0 and lw[5] == 0, f"{what}: ignored row"
        assert math.isnan(mean), f"{what}: mean"
        check_xent_grad(g[good], gw[good], t[good], N, n, f"{what}: gradient")
        check_losses(rows[good], 0.0, lw[good], 0.0, f"{what}: row losses")
    xr.reset_options()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_large_magnitude_rows(orc, dtype):
    """Rows of large magnitude keep the results of the definitions, on every launch path: a
    row filled with a large negative mask value (-1e10) gives the uniform softmax, -log p =
    log N and the loss log N; rows of values up to +-1e30, a maximum of 3e38 over -3e38, a
    common offset of 1e9 and one of 5000 keep the maximum's term at exactly 1 (such rows form
    their exponents from x - m; only rows whose m log2 e stays under 2^7 fold m into the
    exponent's constant). Softmax, negative log-softmax and cross-entropy against the
    oracle."""
    M, N = 6, 3001
    rng = np.random.default_rng(12400)
    xf = rng.standard_normal((M, N)).astype(np.float32)          # row 4: an ordinary row
    xf[0] = -1e10                                                 # a fully masked row
    xf[1] = ((rng.random(N) * 2 - 1) * 1e30).astype(np.float32)
    xf[2] = -3e38
    xf[2, 7] = 3e38
    xf[3] = (1e9 + rng.standard_normal(N) * 300).astype(np.float32)
    xf[5] = (5000 + rng.standard_normal(N) * 4).astype(np.float32)  # a moderate offset
    x = synth.bf16_bits_from_f32(xf) if dtype == "bf16" else xf
    t = np.array([5, int(np.argmax(widen(x)[1])), 7, 11, 13, 17], dtype=np.int64)
    idx = np.array([5, 100, 7, 11, 13, 17], dtype=np.int64)
    for name, path, split in (("auto", 0, 0), ("resident", 1, 0), ("split2", 2, 2),
                              ("stream", 3, 0)):
        xr.set_option("path", path)
        xr.set_option("split", split)
        what = f"{dtype} {name}"
        y = to_host(xr.softmax_fwd(to_device(x)))
        want = orc.softmax_fwd(x)
        check_probs(y, want, f"{what}: softmax")
        assert np.allclose(widen(y)[0], 1.0 / N, rtol=2.0 ** -7, atol=0), f"{what}: uniform row"
        out, loss = xr.nll_fwd(to_device(x), to_device(idx))
        out_h, loss_h = widen(to_host(out)), to_host(loss).astype(np.float64)
        out_w, loss_w = orc.nll_fwd(x, idx)
        rel = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -20
        # -log p beyond the fp32 range (6e38 in the 3e38 row) is stored as +inf
        big = np.abs(out_w) > float(np.finfo(np.float32).max)
        assert np.all(np.isposinf(out_h[big])), f"{what}: -log p past the fp32 range"
        scale = np.max(np.where(big, 0.0, np.abs(out_w)), axis=1, keepdims=True)
        assert np.all((np.abs(out_h - out_w) <= rel * np.abs(out_w) + 2.0 ** -20 * scale) | big), \
            f"{what}: -log softmax"
        assert np.all(np.abs(loss_h - loss_w) <= rel * np.abs(loss_w) + 2.0 ** -20 * scale[:, 0]), \
            f"{what}: gathered loss"
        one = 2.0 ** -8 if dtype == "bf16" else 1e-5  # the stored -log p: one rounding
        assert abs(out_h[0, 0] - math.log(N)) <= one * math.log(N), f"{what}: -log p of the masked row"
        g, rows, mean, counts = run_xent(x, t, N)
        compare_xent(orc, x, t, N, g, rows, mean, counts, f"{what}: cross-entropy")
        assert abs(rows[0] - math.log(N)) <= 1e-4 * math.log(N), f"{what}: loss of the masked row"
    xr.reset_options()


def test_partial_overlap_is_rejected():
    x = torch.zeros((4, 100), dtype=torch.float32, device="cuda")
    with pytest.raises(xr.XrError, match="overlap"):
        xr.softmax_fwd(x[:, :50], x[:, 10:60])
