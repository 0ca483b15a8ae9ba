"""GPU parity of the block-sparse softmax backward (xr_bsr_softmax_bwd) against the float64
oracle: every element of the block storage is compared (listed rows to the tolerance,
everything else bit for bit unchanged).

Tolerances: fp32 1e-5 times the larger of 1 and the batch's largest |value| (the outputs
are y (dy - s) scale, not bounded by 1); bf16 the suite's 2e-2 relative bound.
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


def check(got: np.ndarray, want: np.ndarray, listed: np.ndarray, what: str) -> None:
    """got / want (Z, stride); listed: bool mask of the elements the table covers."""
    if got.dtype == np.uint16:
        g = np.where(listed, got, 0)
        check_bf16(g, np.where(listed, want, 0.0), what)
    else:
        g = widen(got)
        tol = FP32_ABS * np.maximum(1.0, np.max(np.abs(np.where(listed, want, 0.0)), axis=1,
                                                keepdims=True))
        bad = np.argwhere(listed & (np.abs(g - want) > tol))
        assert bad.size == 0, f"{what}: element {tuple(bad[0])} {g[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a


def listed_mask(lut: np.ndarray, n_brows: int, block: int, Z: int, stride: int,
                n_blocks: int) -> np.ndarray:
    m = np.zeros((Z, stride), dtype=bool)
    for r in range(n_brows):
        size, off = lut[2 * r], lut[2 * r + 1]
        for k in range(size):
            bid = lut[off + 4 * k]
            if 0 <= bid < n_blocks:
                m[:, bid * block * block:(bid + 1) * block * block] = True
    return m


def run(y_h, d_h, lut, n_brows, n_blocks, block, scale, alias=False):
    y = to_device(y_h)
    d = y if alias else to_device(d_h)
    xr.bsr_softmax_bwd(y, d, to_device(lut), n_brows, n_blocks, block, scale)
    torch.cuda.synchronize()
    return to_host(d)


def test_worked_example(orc):
    with open(oracle_pins.GOLDEN) as f:
        gold = json.load(f)
    for case in gold["bsr_softmax_bwd"]:
        y = oracle_pins.as_input(case["y"], case["dtype"])
        dy = oracle_pins.as_input(case["dy"], case["dtype"])
        lut = np.array(case["lut"], dtype=np.int32)
        n_blocks = y.shape[1] // (case["block"] ** 2)
        if case["block"] * y.itemsize < 16:
            # blocks narrower than one 16-byte vector are outside the library's contract
            with pytest.raises(xr.XrError):
                run(y, dy, lut, case["n_brows"], n_blocks, case["block"], case["scale"])
            continue
        got = run(y, dy, lut, case["n_brows"], n_blocks, case["block"], case["scale"])
        want = np.array([[oracle_pins.closed_form(v) for v in r] for r in case["out"]])
        assert np.max(np.abs(widen(got) - want)) <= 1e-6, case["name"]


# (block, dtype, block-rows, local window, global stride, batches); rows of the 16-wide
# fp32 case with 40 block-rows and the 64-wide one with 30 list more than 12 blocks (the
# two-read path)
CASES = [(16, "bf16", 8, 2, 3, 2), (32, "f32", 6, 3, 2, 3), (64, "bf16", 16, 4, 8, 2),
         (16, "f32", 40, 4, 2, 1), (128, "bf16", 4, 4, 1, 1), (8, "bf16", 12, 3, 4, 2),
         (4, "f32", 10, 2, 3, 2), (512, "bf16", 2, 2, 1, 1), (256, "f32", 2, 2, 1, 1),
         (64, "f32", 30, 2, 2, 1)]


@pytest.mark.parametrize("block,dtype,nb,local,stride,Z", CASES,
                         ids=[f"b{c[0]}-{c[1]}-nb{c[2]}" for c in CASES])
def test_bsr_layouts(orc, block, dtype, nb, local, stride, Z):
    lay = synth.bsr_layout(nb, local, stride)
    per_z = lay["n_blocks"] * block * block
    ld = per_z + 24  # spare elements after the blocks of each batch: never written
    y = synth.random_rows(14000 + block, Z, per_z, ld=ld, dtype=dtype, scale=1.0, pad_nan=True)
    d = synth.random_rows(14001 + block, Z, per_z, ld=ld, dtype=dtype, scale=1.0, pad_nan=True)
    got = run(y, d, lay["lut"], nb, lay["n_blocks"], block, 0.5)
    want = orc.bsr_softmax_bwd(y, d, lay["lut"], nb, block, 0.5)
    listed = listed_mask(lay["lut"], nb, block, Z, ld, lay["n_blocks"])
    check(got, want, listed, f"block {block} {dtype} {nb} block-rows")
    assert np.array_equal(bits(got[~listed]), bits(d[~listed])), "unlisted storage changed"


def test_bsr_alias_and_scale(orc):
    block, nb = 32, 8
    lay = synth.bsr_layout(nb, 3, 4)
    per_z = lay["n_blocks"] * block * block
    y = synth.random_rows(14100, 2, per_z, dtype="f32", scale=1.0)
    for scale in (1.0, -2.0, 0.0):
        got = run(y, y, lay["lut"], nb, lay["n_blocks"], block, scale, alias=True)
        want = orc.bsr_softmax_bwd(y, y, lay["lut"], nb, block, scale)
        check(got, want, np.ones_like(got, dtype=bool), f"y = dx, scale {scale}")


def test_bsr_bad_table_entries(orc):
    """A block index outside the storage reads zeros and writes nothing; a list running past
    the table stops at its end: the same as the valid table without those entries."""
    block, nb = 16, 6
    lay = synth.bsr_layout(nb, 2, 2)
    lut = lay["lut"].copy()
    n_blocks = lay["n_blocks"]
    per_z = n_blocks * block * block
    y = synth.random_rows(14200, 2, per_z, dtype="f32", scale=1.0)
    d = synth.random_rows(14201, 2, per_z, dtype="f32", scale=1.0)
    # block-row 3: its last entry points outside the storage
    size3, off3 = lut[6], lut[7]
    bad = lut.copy()
    bad[off3 + 4 * (size3 - 1)] = n_blocks + 7
    clean = lut.copy()
    clean[6] = size3 - 1
    # block-row 5 (the table's last): claims 100 entries
    bad[10] = 100
    got = run(y, d, bad, nb, n_blocks, block, 1.0)
    want = orc.bsr_softmax_bwd(y, d, clean, nb, block, 1.0)
    listed = listed_mask(clean, nb, block, 2, per_z, n_blocks)
    check(got, want, listed, "bad entries")
    assert np.array_equal(bits(got[~listed]), bits(d[~listed]))


def test_bsr_workload_sampled(orc):
    """The benchmark's layout (32 batches of 4096 x 4096 in 64 x 64 bf16 blocks, local 4 +
    every 8th column), in the launch configuration the benchmark times; two batches are
    compared in full against the oracle."""
    w = synth.bsr_softmax()
    y_h, d_h = w["y"], w["dy"]
    got = run(y_h, d_h, w["lut"], w["n_brows"], w["n_blocks"], w["block"], w["scale"])
    for z in (0, w["Z"] - 1):
        want = orc.bsr_softmax_bwd(y_h[z:z + 1], d_h[z:z + 1], w["lut"], w["n_brows"],
                                   w["block"], w["scale"])
        check(got[z:z + 1], want, np.ones_like(want, dtype=bool), f"workload batch {z}")
