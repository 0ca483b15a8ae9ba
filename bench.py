"""Benchmark: fused cross-entropy forward + backward, V = 128256, bf16, on one MI355X.

One step is one pass of the whole hot path over one batch: the target scan, the row
kernel (row loss + in-place gradient) and the mean, for M = 16384 token rows of a
128256-wide bf16 vocabulary with 5 % ignored rows, the logits already resident in HBM.
The gradient overwrites the logits, so every step runs on its own copy of the synthetic
logits (made before the timed region).

Prints one JSON line on stdout. Throughput is B_min / t, where B_min is the method's
minimal traffic: every non-ignored row read once, every row written once, the targets read
and the row losses written. `roofline` reports the row kernel alone, timed with HIP events
recorded around it on its stream; `cpu_baseline` times the float64 oracle on a sample of
the same workload on this host's cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--cpu-rows R]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
COUNTERS = os.path.join(ROOT, "profiles", "xent_c4_hbm_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "cross_entropy_reductions_amd", "csrc", f)
                  for f in ("xr_xent.hip", "xr_softmax.hip", "xr_rows.h", "xr_device.h",
                            "xr_internal.h", "xr_api.cpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def xent_bmin(M: int, V: int, n_keep: int, elt: int) -> int:
    """Minimal bytes: non-ignored rows read once, all rows written once, targets, losses."""
    return n_keep * V * elt + M * V * elt + 8 * M + 4 * M + 4


def measured_traffic():
    """HBM bytes per launch of the row kernel from committed rocprofv3 counters, or None if
    they are absent or were taken on other kernel sources."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own launch stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventSynchronize(ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e: int) -> None:
        self.hip.hipEventDestroy(ctypes.c_void_p(e))


def cpu_baseline(workload: dict, rows: int) -> dict:
    """The oracle as it stands on the first `rows` rows (count, loss + gradient, mean), in
    1024-row chunks so its float64 gradient buffer stays near 1 GB."""
    import oracle

    orc = oracle.get()
    V = workload["N"]
    x = workload["x"][:rows]
    t = workload["target"][:rows]
    t0 = time.perf_counter()
    n, _ = orc.xent_count(t, V)
    losses = []
    for r0 in range(0, rows, 1024):
        _, loss = orc.xent_rows(x[r0:r0 + 1024], t[r0:r0 + 1024], V, n, want_grad=True)
        losses.append(loss)
    import numpy as np
    orc.mean(np.concatenate(losses), n)
    sec = time.perf_counter() - t0
    b = xent_bmin(rows, V, int((t != -100).sum()), 2)
    return {"value": round(b / sec / 1e9, 3), "unit": "GB/s", "cores": orc.num_threads(),
            "kind": "oracle", "rows_per_s": round(rows / sec, 1), "seconds": round(sec, 3),
            "sample": f"first {rows} of {workload['M']} rows of the same workload "
                      f"(V={V} bf16): float64 count, loss, gradient and mean, one run"}


def run(args) -> dict:
    import torch

    import cross_entropy_reductions_amd as xr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    w = synth.xent_c4()
    M, V = w["M"], w["N"]
    t = torch.from_numpy(w["target"]).to(dev)
    x0 = torch.from_numpy(w["x"].view("int16")).view(torch.bfloat16).to(dev)
    n_keep = int((w["target"] != -100).sum())
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] workload ready in {gen_s:.1f}s: M={M} V={V} n={n_keep}", file=sys.stderr,
          flush=True)

    steps, warmup = args.steps, args.warmup
    copies = [x0.clone() for _ in range(warmup + steps)]
    del x0
    row_loss = torch.empty(M, dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    counts = torch.empty(3, dtype=torch.int32, device=dev)
    ws = torch.empty(max(256, xr.xent_workspace_bytes(M, V, torch.bfloat16)), dtype=torch.uint8,
                     device=dev)
    ev = HipEvents()
    starts = [ev.create() for _ in range(steps)]
    stops = [ev.create() for _ in range(steps)]

    for i in range(warmup):
        xr.xent_fwd_bwd(copies[i], t, -100, row_loss=row_loss, mean_loss=mean, counts=counts,
                        workspace=ws)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(steps):
        xr.set_profile_events(starts[i], stops[i])
        xr.xent_fwd_bwd(copies[warmup + i], t, -100, row_loss=row_loss, mean_loss=mean,
                        counts=counts, workspace=ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    xr.set_profile_events(None, None)
    kernel_ms = [ev.elapsed_ms(a, b) for a, b in zip(starts, stops)]
    for e in starts + stops:
        ev.destroy(e)
    c = counts.cpu().tolist()
    assert c[0] == n_keep and c[2] == 0, f"unexpected counts {c}"

    bmin = xent_bmin(M, V, n_keep, 2)
    ms_step = wall * 1e3 / steps
    gbs = bmin / (wall / steps) / 1e9
    kavg = statistics.mean(kernel_ms)
    kgbs = bmin / (kavg / 1e3) / 1e9
    p = xr.plan("xent", M, V, torch.bfloat16)
    out = {
        "metric": "achieved HBM GB/s (% of peak) and rows/s for fused xent fwd+bwd, V=128256 bf16",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fused cross-entropy loss+grad, M=16384 tokens, V=128256, bf16 "
                               "logits N(0,1) + 4 spikes of +20 per row, int64 targets, 5% "
                               "ignore_index=-100, mean reduction",
                   "M": M, "V": V, "n_non_ignore": n_keep, "bytes_min": bmin,
                   "path": p["path"], "threads": p["threads"], "grid": p["grid"]},
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "rows_per_s": round(M / (wall / steps), 1),
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "xent_rows_kernel", "kernel_ms_avg": round(kavg, 4),
                     "kernel_ms_min": round(min(kernel_ms), 4)},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=16384)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (--gpus {args.gpus} "
              "requested).", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.steps + args.warmup > 40:
        print("need 1 <= steps and steps + warmup <= 40 (one 4.2 GB copy of the logits per step)",
              file=sys.stderr)
        return 2
    print(json.dumps(run(args)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
