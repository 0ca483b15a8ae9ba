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
