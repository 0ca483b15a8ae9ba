"""Launch plans on a modelled MI355X, on the CPU (xr_plan_model: no device needed).

A split row's chunk workgroups wait, with a bound, for the other chunks of their row, and
write groups wait for the chunks of 8 adjacent rows. Those waits always end without the
bound when every workgroup they wait for can be resident at the same time as the waiting
ones. A normal launch deals workgroups to the 8 XCDs in id order, round robin, and each
XCD starts its workgroups in id order; a row's S chunks (a group's 8 S) have consecutive
ids, so each XCD holds at most ceil(S / 8) (S) of them. The plans therefore split rows only
when S <= the workgroups the GPU holds at once, and group rows only when 4 x 8 S do; rows
longer than that run the stream kernels, whose workgroups wait for nobody. These tests
check those conditions over shapes from 8192 x 32000 to rows of 2^29 elements, for every
op that splits rows and several occupancies.
"""
from __future__ import annotations

import math

import pytest
import torch

CUS = 256   # MI355X compute units
XCDS = 8    # accelerator complex dies, each with its own share of the compute units
MAX_GRID = 2 ** 31 - 1

SHAPES = [
    (8192, 32000, torch.bfloat16), (16384, 128256, torch.bfloat16),
    (2048, 256000, torch.float32), (4096, 4096, torch.bfloat16),
    (4096, 128256, torch.bfloat16), (16, 1 << 20, torch.float32), (8, 128256, torch.bfloat16),
    (1, 300001, torch.bfloat16), (64, 40000, torch.bfloat16), (261, 66000, torch.bfloat16),
    (1, 1 << 24, torch.bfloat16), (2, 1 << 26, torch.float32), (1, 1 << 27, torch.bfloat16),
    (1, 1 << 29, torch.bfloat16), (3, 1 << 29, torch.float32), (1 << 20, 4096, torch.bfloat16),
    (1 << 24, 128256, torch.bfloat16),
]
OPS = ["xent", "softmax_fwd_ws", "softmax_bwd_ws", "nll_fwd"]


@pytest.fixture(scope="module")
def xr():
    import cross_entropy_reductions_amd as xr
    xr.reset_options()
    return xr


def vectors(N: int, dtype) -> int:
    return -(-N // (8 if dtype == torch.bfloat16 else 4))


@pytest.mark.parametrize("per_cu", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("op", OPS)
def test_split_rows_fit_the_gpu(xr, op, per_cu):
    resident = CUS * per_cu
    seen = set()
    for M, N, dt in SHAPES:
        p = xr.plan_model(op, M, N, dt, CUS, per_cu)
        what = f"{op} {M}x{N} {dt} at {per_cu}/CU: {p}"
        seen.add(p["path"])
        if p["path"] == "split" and not p["cooperative"]:
            S = p["split"]
            assert S >= 2, what
            assert S <= resident, what                                  # the row's chunks
            assert math.ceil(S / XCDS) <= resident // XCDS, what       # ... on every XCD
            assert p["grid_total"] == M * S <= MAX_GRID, what
            assert S * p["chunk_vecs"] >= vectors(N, dt), what         # the chunks hold the row
            if p["group_rows"] > 1:
                assert p["group_rows"] == 8, what
                assert S <= 8 and p["chunk_vecs"] * 16 >= 32 << 10, what
                assert 4 * 8 * S <= resident, what                      # a group, four times over
                assert 8 * S // XCDS <= resident // XCDS, what
        elif p["path"] == "split":
            assert p["grid_total"] <= resident, what                   # all co-resident
        if p["path"] == "resident":
            assert p["split"] == 1 and p["grid_total"] <= MAX_GRID, what
    assert "split" in seen and "stream" in seen


def test_rows_beyond_the_gpu_take_the_stream_kernels(xr):
    """A 2^29-element bf16 row needs thousands of chunk workgroups; at low occupancy they cannot
    all be resident, so the row runs the stream kernels instead of waiting on chunks that
    could not start."""
    for op in OPS:
        p = xr.plan_model(op, 1, 1 << 29, torch.bfloat16, CUS, 1)
        assert p["path"] == "stream", (op, p)


def test_write_groups_need_room(xr):
    """16384 x 128256 bf16 cross-entropy rows in two 128 KB chunks are grouped by 8 when the GPU
    holds at least 4 x 16 of their workgroups, and not when it holds fewer."""
    assert xr.plan_model("xent", 16384, 128256, torch.bfloat16, CUS, 2)["group_rows"] == 8
    p = xr.plan_model("xent", 16384, 128256, torch.bfloat16, 1, 1)
    assert p["group_rows"] == 1


def test_model_argument_errors(xr):
    with pytest.raises(xr.XrError):
        xr.plan_model("xent", 4, 100, torch.float32, 0, 1)
    with pytest.raises(xr.XrError):
        xr.plan_model("xent", 4, 100, torch.float32, 256, 0)


@pytest.mark.parametrize("per_cu", [1, 2, 4, 8, 16, 32])
def test_load_priority_only_for_one_round_softmax_grids(xr, per_cu):
    """Whole softmax rows issue their loads at a raised wave priority exactly when the grid is
    resident at once (grid <= compute units x workgroups per compute unit); no other plan
    (the cross-entropy, the negative log-softmax, split rows, the stream kernels) does."""
    resident = CUS * per_cu
    for M, N, dt in SHAPES + [(2048, 4096, torch.bfloat16), (16384, 1024, torch.float32)]:
        for op in ("softmax_fwd", "softmax_bwd", "softmax_fwd_ws", "softmax_bwd_ws", "xent",
                   "nll_fwd"):
            p = xr.plan_model(op, M, N, dt, CUS, per_cu)
            want = (op in ("softmax_fwd", "softmax_bwd", "softmax_fwd_ws", "softmax_bwd_ws")
                    and p["path"] == "resident" and p["grid_total"] <= resident)
            assert p["load_priority"] == want, (op, M, N, dt, per_cu, p)
    # 4096 x 4096 bf16: 4096 one-wave workgroups, resident at once from 16 per compute unit
    p = xr.plan_model("softmax_bwd", 4096, 4096, torch.bfloat16, CUS, 16)
    assert p["load_priority"] and p["threads"] == 64 and p["grid_total"] == 4096
    assert not xr.plan_model("softmax_bwd", 4096, 4096, torch.bfloat16, CUS, 8)["load_priority"]
