"""Host-side logic of bench.py (no GPU): the one-GPU contract, the minimal-bytes formula, the
counter summary's scaling, the comment-blind source hash and the CPU oracle baselines."""
from __future__ import annotations

import csv
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    """`--gpus N` with N > 1 exits with status 2 and a message; nothing runs on a GPU."""
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_minimal_bytes():
    """Non-ignored rows read once, every row written once, 8-byte targets, 4-byte row losses
    and the 4-byte mean: the 16384 x 128256 bf16 workload with 15565 rows kept."""
    M, V, keep = 16384, 128256, 15565
    assert bench.xent_bmin(M, V, keep, 2) == keep * V * 2 + M * V * 2 + 12 * M + 4
    assert bench.xent_bmin(M, V, keep, 2) == 8195498500
    # fp32 rows, none ignored: twice the matrix plus targets and losses
    assert bench.xent_bmin(2048, 256000, 2048, 4) == 2 * 2048 * 256000 * 4 + 12 * 2048 + 4


def test_code_only_ignores_comments_and_spacing():
    a = "int f(int x) {  // the answer\n  return x + 1; /* one\n more */ }\n"
    b = "int f(int x) { return x + 1; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only("return x + 2;") != bench._code_only("return x + 1;")


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Value": value})


def test_counter_summary_scales_by_the_copy(tmp_path):
    """Each counter is scaled by what it reads for the runtime's copy of the known-size logit
    matrix; the row kernel's median over its dispatches is taken."""
    matrix = bench.C4_M * bench.C4_V * 2
    kib = matrix / 1024.0
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    copy = "__amd_rocclr_copyBuffer"
    row = "void xr::xent_rows_kernel<1, 512, 16, 2>(xr::XentParams)"
    # the counters read (a hair under) half the copy's fetch bytes and all of its written
    # bytes; the runtime's small copies are left out
    _write_counters(fetch, [(copy, kib * 0.4999), (copy, kib * 0.4999), (copy, 1.0),
                            (row, kib * 0.475), (row, kib * 0.476), (row, kib * 0.477)])
    _write_counters(write, [(copy, kib), (copy, kib), (copy, 0.0), (row, kib), (row, kib),
                            (row, kib * 1.01)])
    out = bench.summarize_counters(str(fetch), str(write))
    assert out["copy_scale_fetch"] == round(1 / 0.4999, 4) and out["copy_scale_write"] == 1.0
    assert out["fetch_bytes_per_launch"] == round(matrix * 0.476 / 0.4999)
    assert out["write_bytes_per_launch"] == round(matrix)
    assert out["dispatches"] == {"row_kernel": 3, "copy": 2}
    assert out["kernel_source_hash"] == bench.kernel_source_hash()


def test_counter_summary_of_every_workload(tmp_path):
    """Every workload's kernels are told apart by name (the forward's split kernel is not the
    backward's), and traffic equal to the minimal bytes reads as 1.0."""
    copy = "__amd_rocclr_copyBuffer"
    names = {"softmax_split_kernel": "void xr::softmax_split_kernel<1, 512, 16, 8, false>(xr::SoftmaxFwdParams)",
             "softmax_bwd_split_kernel": "void xr::softmax_bwd_split_kernel<1, 512, 16, 8>(xr::SoftmaxBwdParams)"}
    for wl in ["c2", "c3", "c5", "c4-mul", "c4-nll", "ln", "bsr", "sm-vocab", "sm-few"]:
        matrix, kernels = bench.counter_workload(wl)
        fetch_rows, write_rows = [(copy, matrix / 2048.0)] * 2, [(copy, matrix / 1024.0)] * 2
        for k, bmin in kernels:
            name = names.get(k, f"void xr::{k}<1, 256, 8>(xr::Params)")
            fetch_rows += [(name, bmin / 2 / 2048.0)] * 3   # half of it read, at half scale
            write_rows += [(name, bmin / 2 / 1024.0)] * 3
        f, w = tmp_path / f"{wl}_f.csv", tmp_path / f"{wl}_w.csv"
        _write_counters(f, fetch_rows)
        _write_counters(w, write_rows)
        out = bench.summarize_counters(str(f), str(w), workload=wl)
        got = {k: v["traffic_over_bytes_min"] for k, v in out["kernels"].items()}
        assert got == {k: 1.0 for k, _ in kernels}, (wl, got)
    # the block-sparse workload: 32 maps of 453 stored 64 x 64 bf16 blocks
    assert bench.counter_workload("bsr")[0] == 32 * 453 * 64 * 64 * 2


def test_cpu_baselines_on_small_inputs():
    """The oracle baselines run on a small sample and report the contract's fields."""
    x = synth.random_rows(31, 40, 1024, dtype="bf16", scale=1.0)
    t = synth.random_targets(32, 40, 1024, ignore_frac=0.1)
    w = {"M": 40, "N": 1024, "x": x, "target": t, "dtype": "bf16"}
    lines = [bench.cpu_baseline(w, 40, min_seconds=0.05),
             bench.cpu_baseline_element_mul(w, 40, 0.5, min_seconds=0.05),
             bench.cpu_baseline_nll(w, np.clip(t, 0, None), 40, min_seconds=0.05)]
    ln = synth.layernorm_ln(M=64, N=512)
    lines.append(bench.cpu_baseline_layernorm(ln, 64, min_seconds=0.05))
    for c in lines:
        assert c["kind"] == "oracle" and c["unit"] == "GB/s"
        assert c["value"] > 0 and c["cores"] >= 1 and c["seconds"] > 0
        assert "whole passes" in c["sample"]


def test_trace_summary_takes_the_headline_launches(tmp_path):
    """The headline kernel's average comes from its own launches only (the same kernel on
    other workloads has other template arguments or grids), the last `steps` in launch
    order."""
    path = tmp_path / "trace.csv"
    _, threads, items, _ = bench.traced_launches()["c4"]["xent"]
    head = f"void xr::xent_rows_kernel<1, {threads}, 16, 2>(xr::XentParams)"
    rows = [(head, items, threads, 1000 + 10 * k, 1000 + 10 * k + d)
            for k, d in enumerate([9, 9, 9, 1, 2, 3])]
    rows += [("void xr::xent_rows_kernel<1, 128, 8, 2>(xr::XentParams)", 32768 * 128, 128, 5000,
              5100),
             (head, 512 * threads, threads, 6000, 9000),
             ("void xr::xent_rows_kernel<0, 512, 16, 2>(xr::XentParams)", items, 512, 6500, 6600),
             ("__amd_rocclr_copyBuffer", 1024, 512, 7000, 7500)]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, grid, wg, s, e in reversed(rows):
            w.writerow({"Kernel_Name": name, "Grid_Size_X": grid, "Workgroup_Size_X": wg,
                        "Start_Timestamp": s, "End_Timestamp": e})
    out = bench.summarize_trace(str(path), 3)
    assert out["calls"] == 3 and out["launches_traced"] == 6
    # the 8192 x 32000 workload's one launch is told apart by its shape; c2 and c5 are absent
    assert out["other_configs"]["c3"]["xent"]["calls"] == 1
    assert out["other_configs"]["c3"]["xent"]["kernel_ms_avg"] == round(100 / 1e6, 5)
    assert out["other_configs"]["c2"] == {} and out["other_configs"]["c5"] == {}
    assert out["kernel_ms_avg"] == round(2 / 1e6, 5) and out["kernel_ms_min"] == round(1 / 1e6, 5)
    assert out["kernel_source_hash"] == bench.kernel_source_hash()


def test_probe_shapes_hold_the_row():
    """The ceiling probe's launch shapes: each holds a chunk of the row, filled more than half,
    in 1-32 chunks of at least 64 vectors; two-input shapes come from the backward's menu."""
    for nv, two in ((512, False), (512, True), (4000, False), (16032, False), (64000, False)):
        shapes = bench.probe_shapes(nv, two)
        assert shapes
        for t, v, s in shapes:
            chunk = -(-nv // s)
            assert chunk <= t * v < 2 * chunk and chunk >= 64
            assert (t, v) in (bench.BWD_SHAPES if two else bench.FWD_SHAPES)
    assert (128, 8, 4) in bench.probe_shapes(4000, False)  # the 8192 x 32000 plan
    assert (512, 16, 2) in bench.probe_shapes(16032, False)  # the 16384 x 128256 plan
