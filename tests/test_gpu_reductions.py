"""GPU parity of the cross-entropy reductions, the folded upstream gradient, element_mul and
the autograd wrapper, against the float64 oracle.

Tolerances are those of the rest of the parity suite, with the fp32 bound scaled by the
largest |upstream gradient| of the case: an upstream factor s multiplies every gradient
value, and with it the rounding error of the fp32 result (1e-5 * max(1, |s|)).
"""
from __future__ import annotations

import json

import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import synth
from gpu_util import (FP32_ABS, check_losses, check_rel, check_xent_grad, to_device, to_host,
                      widen)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import cross_entropy_reductions_amd as xr
else:  # collected on a machine without a GPU: every test here is skipped
    xr = None
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no HIP device")]

MEAN_REL = 1e-4


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(autouse=True)
def _reset_options():
    xr.reset_options()
    yield
    xr.reset_options()


def check_products(gpu: np.ndarray, want: np.ndarray, smax: float, what: str) -> None:
    """element_mul's products: one rounding each, relative; fp32 also within 1e-5 max(1, s)."""
    check_rel(gpu, want, what, abs_tol=FP32_ABS * max(1.0, smax))


def upstream(kind: str, M: int, seed: int):
    """(host values for the oracle: None / float / array, device argument for the library)."""
    if kind == "none":
        return None, None
    if kind in ("pos", "neg", "zero"):
        v = {"pos": 2.5, "neg": -0.75, "zero": 0.0}[kind]
        return v, v
    if kind == "rows":
        s = synth.random_rows(seed, 1, M, dtype="f32", scale=2.0)[0]
        s[::7] = 1.0
        s[3::11] = -1.0
        return s.astype(np.float64), to_device(s)
    if kind == "rows-broadcast":  # one value seen through a stride-0 view
        return -1.25, torch.full((1,), -1.25, dtype=torch.float32, device="cuda").expand(M)
    raise ValueError(kind)


def run_and_compare(orc, x_host, t, V, reduction, kind, seed, what, ignore_index=-100):
    M = x_host.shape[0]
    s_host, s_dev = upstream(kind, M, seed)
    x = to_device(x_host)
    loss, rows, counts = xr.xent_fwd_bwd(x[:, :V], to_device(t), ignore_index,
                                         reduction=reduction, grad_scale=s_dev)
    torch.cuda.synchronize()
    g_gpu, rows_gpu, counts_gpu = to_host(x), to_host(rows), to_host(counts)
    n, bad = orc.xent_count(t, V, ignore_index)
    assert int(counts_gpu[0]) == n and int(counts_gpu[1]) == bad and int(counts_gpu[2]) == 0, what
    g, loss_all, red, _ = orc.xent(x_host, t, V, ignore_index, reduction=reduction, scale=s_host)
    check_xent_grad(g_gpu[:, :V], g, t, V, n if reduction == "mean" else 1, what, scale=s_host,
                    ignore_index=ignore_index)
    if reduction == "none":
        assert loss.data_ptr() == rows.data_ptr(), f"{what}: none returns the row losses"
        check_losses(rows_gpu, 0.0, loss_all, 0.0, what)
    else:
        got = float(loss.item())
        check_losses(rows_gpu, got, loss_all, red, what)
    if x_host.shape[1] > V:
        assert np.array_equal(g_gpu[:, V:].view(np.uint8), x_host[:, V:].view(np.uint8)), \
            f"{what}: padding changed"
    return g_gpu


# ----------------------------------------------------------------------------- worked examples
def test_worked_examples_reduced():
    with open(oracle_pins.GOLDEN) as f:
        gold = json.load(f)
    for case in gold["xent_reduced"]:
        x_h = oracle_pins.as_input(case["x"], case["dtype"])
        t = np.array(case["target"], dtype=np.int64)
        sc = case["scale"]
        s_dev = to_device(np.array(sc, dtype=np.float32)) if isinstance(sc, list) else float(sc)
        x = to_device(x_h)
        loss, rows, counts = xr.xent_fwd_bwd(x, to_device(t), case["ignore_index"],
                                             reduction=case["reduction"], grad_scale=s_dev)
        want_g = np.array([[oracle_pins.closed_form(v) for v in r] for r in case["grad"]])
        n_r = case["n"] if case["reduction"] == "mean" else 1
        check_xent_grad(to_host(x), want_g, t, x_h.shape[1], n_r, case["name"],
                        scale=np.array(sc, dtype=np.float64), ignore_index=case["ignore_index"])
        want_l = np.array([oracle_pins.closed_form(v) for v in case["loss"]])
        red = case["reduced"]
        check_losses(to_host(rows), 0.0 if red is None else float(loss.item()), want_l,
                     0.0 if red is None else oracle_pins.closed_form(red), case["name"])
        assert int(to_host(counts)[0]) == case["n"]
    for case in gold["element_mul"]:
        x_h = oracle_pins.as_input(case["x"], case["dtype"])
        x = to_device(x_h)
        xr.element_mul(x[:, :case["n_cols"]], to_device(np.array(case["scale"], dtype=np.float32)))
        got = to_host(x)
        want = np.array([[oracle_pins.closed_form(v) for v in r] for r in case["out"]])
        assert np.array_equal(widen(got[:, :case["n_cols"]]), want), case["name"]
        assert np.array_equal(got[:, case["n_cols"]:], x_h[:, case["n_cols"]:]), case["name"]


# ----------------------------------------------------------------------------- reductions
SHAPES = [(300, 5003, 5003, "bf16"), (300, 5003, 5010, "f32"), (64, 40000, 40000, "bf16"),
          (40, 70001, 70016, "f32"), (7, 33, 40, "bf16")]
KINDS = ["none", "pos", "neg", "zero", "rows", "rows-broadcast"]


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("M,V,ld,dtype", SHAPES, ids=[f"{m}x{v}-{d}" for m, v, _, d in SHAPES])
def test_xent_reductions(orc, reduction, M, V, ld, dtype):
    x = synth.random_rows(11000 + V % 97, M, V, ld=ld, dtype=dtype, scale=3.0,
                          pad_nan=ld > V)
    t = synth.random_targets(11001 + V % 97, M, V, ignore_frac=0.2)
    t[1] = V + 5  # out of range: zero row, still counted in n
    for k, kind in enumerate(KINDS):
        run_and_compare(orc, x, t, V, reduction, kind, 11100 + k,
                        f"{M}x{V} {dtype} {reduction} upstream={kind}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_xent_reductions_all_paths(orc, dtype):
    M, V = 40, 50000
    x = synth.random_rows(11200, M, V, dtype=dtype, scale=3.0)
    t = synth.random_targets(11201, M, V, ignore_frac=0.1)
    for name, path, split in (("resident", 1, 0), ("split3", 2, 3), ("stream", 3, 0)):
        xr.set_option("path", path)
        xr.set_option("split", split)
        for reduction, kind in (("sum", "neg"), ("none", "rows"), ("mean", "pos")):
            run_and_compare(orc, x, t, V, reduction, kind, 11202,
                            f"{dtype} {name} {reduction} {kind}")


def test_xent_unit_upstream_matches_plain_call():
    """An upstream gradient of exactly 1 gives the plain call's bits."""
    w = synth.xent_c3(M=256)
    x1, x2 = to_device(w["x"]), to_device(w["x"])
    t = to_device(w["target"])
    m1, r1, _ = xr.xent_fwd_bwd(x1, t)
    m2, r2, _ = xr.xent_fwd_bwd(x2, t, grad_scale=1.0)
    torch.cuda.synchronize()
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16))
    assert torch.equal(r1, r2) and torch.equal(m1, m2)


def test_xent_sum_of_empty_batch():
    x = torch.empty((0, 10), dtype=torch.float32, device="cuda")
    t = torch.empty((0,), dtype=torch.int64, device="cuda")
    loss, _, counts = xr.xent_fwd_bwd(x, t, reduction="sum")
    assert float(loss.item()) == 0.0 and to_host(counts).tolist() == [0, 0, 0]


# ----------------------------------------------------------------------------- element_mul
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["pos", "neg", "zero", "rows", "rows-broadcast"])
def test_element_mul(orc, dtype, kind):
    M, N, ld = 257, 7001, 7003  # rows start off 16-byte boundaries; several chunks per row
    x_h = synth.random_rows(11300, M, N, ld=ld, dtype=dtype, scale=2.0, pad_nan=True)
    s_host, s_dev = upstream(kind, M, 11301)
    x = to_device(x_h)
    if not isinstance(s_dev, torch.Tensor):
        s_dev = torch.tensor([s_dev], dtype=torch.float32, device="cuda")
    xr.element_mul(x[:, :N], s_dev)
    torch.cuda.synchronize()
    got = to_host(x)
    want = orc.element_mul(x_h, s_host, n_cols=N)
    smax = float(np.max(np.abs(np.atleast_1d(s_host))))
    check_products(got[:, :N], want, smax, f"element_mul {dtype} {kind}")
    assert np.array_equal(got[:, N:].view(np.uint8), x_h[:, N:].view(np.uint8)), "padding"
    if kind == "rows":
        ones = np.flatnonzero(np.asarray(s_host) == 1.0)
        assert np.array_equal(got[ones].view(np.uint8), x_h[ones].view(np.uint8)), \
            "rows scaled by exactly 1 are untouched"


def test_element_mul_unit_factor_leaves_bits():
    """A factor of exactly 1 neither reads nor writes: even NaN payloads survive bit for bit."""
    x_h = synth.random_rows(11400, 33, 1000, dtype="bf16", scale=1.0)
    x_h[5, 7] = 0x7FC1  # a NaN with a payload
    x = to_device(x_h)
    xr.element_mul(x, torch.ones(1, dtype=torch.float32, device="cuda"))
    assert np.array_equal(to_host(x), x_h)


def test_element_mul_c4_matrix(orc):
    """The backward's scaling at the size of the 16384 x 128256 bf16 workload (sampled rows,
    the launch configuration the benchmark times)."""
    w = synth.xent_c4()
    x_h = w["x"]
    x = to_device(x_h)
    xr.element_mul(x, torch.tensor([0.3], dtype=torch.float32, device="cuda"))
    rows = np.array([0, 1, 4097, 9999, x_h.shape[0] - 1])
    after = to_host(x[torch.from_numpy(rows).cuda()])
    check_products(after, orc.element_mul(x_h[rows], 0.3), 0.3, "element_mul 16384 x 128256 rows")


# ----------------------------------------------------------------------------- autograd
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_autograd_mean_sum_none(orc, dtype):
    M, V = 96, 3001
    x_h = synth.random_rows(11500, M, V, dtype=dtype, scale=2.0)
    t_h = synth.random_targets(11501, M, V, ignore_frac=0.15)
    t = to_device(t_h)

    x = to_device(x_h).requires_grad_(True)
    loss = xr.cross_entropy(x, t)
    assert loss.dim() == 0
    (loss * 2.5).backward()
    g, _, red, (n, _) = orc.xent(x_h, t_h, V, reduction="mean", scale=2.5)
    # the stored gradient is scaled by a second pass (element_mul): two roundings in bf16
    check_xent_grad(to_host(x.grad), g, t_h, V, n, f"{dtype} autograd mean x 2.5", scale=2.5,
                    roundings=2)
    assert abs(float(loss.item()) - red) <= MEAN_REL * abs(red)

    x = to_device(x_h).requires_grad_(True)
    loss = xr.cross_entropy(x, t, reduction="sum")
    loss.backward()  # upstream 1: element_mul skips every row
    g, _, red, _ = orc.xent(x_h, t_h, V, reduction="sum")
    check_xent_grad(to_host(x.grad), g, t_h, V, 1, f"{dtype} autograd sum")
    assert abs(float(loss.item()) - red) <= MEAN_REL * abs(red)

    x = to_device(x_h).requires_grad_(True)
    loss = xr.cross_entropy(x, t, reduction="none")
    assert loss.shape == (M,)
    w_h = synth.random_rows(11502, 1, M, dtype="f32", scale=1.5)[0]
    loss.backward(to_device(w_h))
    g, loss_rows, _, _ = orc.xent(x_h, t_h, V, reduction="none", scale=w_h.astype(np.float64))
    check_xent_grad(to_host(x.grad), g, t_h, V, 1, f"{dtype} autograd none",
                    scale=w_h.astype(np.float64), roundings=2)
    check_losses(to_host(loss.detach()), 0.0, loss_rows, 0.0, f"{dtype} autograd none losses")

    x = to_device(x_h).requires_grad_(True)
    loss, counts = xr.cross_entropy(x, t, return_counts=True)  # counts without a host sync
    assert not counts.requires_grad and counts.dtype == torch.int32
    n, bad = orc.xent_count(t_h, V)
    assert to_host(counts).tolist() == [n, bad, 0]
    loss.backward()

    x = to_device(x_h).requires_grad_(True)
    xr.cross_entropy(x, t, reduction="none").sum().backward()  # stride-0 upstream of ones
    g, _, _, _ = orc.xent(x_h, t_h, V, reduction="none")
    check_xent_grad(to_host(x.grad), g, t_h, V, 1, f"{dtype} autograd none summed")
