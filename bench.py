"""Benchmark: fused cross-entropy forward + backward, V = 128256, bf16, on one MI355X.

One step is one pass of the whole hot path over one batch: the target scan, the row
kernel (row loss + in-place gradient) and the mean, for M = 16384 token rows of a
128256-wide bf16 vocabulary with 5 % ignored rows, the logits already resident in HBM.
The gradient overwrites the logits, so every step runs on its own copy of the synthetic
logits (made before the timed region).

Prints one JSON line on stdout. Throughput is B_min / t, where B_min is the method's
minimal traffic: every non-ignored row read once, every row written once, the targets read
and the row losses written. `roofline` reports the row kernel alone, timed with HIP events
the library records around that launch on its stream (and, under `profiled`, the same
kernel's average from the committed rocprofv3 trace of this command, while that trace
matches the kernel sources); `cpu_baseline` times the float64 oracle on the same workload
on this host's cores. After the headline, the default run times the other configurations
of the 75 %-of-peak target in the same process -- the softmax forward and backward over
4096 x 4096 bf16, the cross-entropy over 8192 x 32000 bf16 and over 2048 x 256000 fp32 --
and reports each kernel's figures under `other_configs` (`value`, `config` and
`ms_per_step` stay the headline's). Beside each of these kernels, `ceiling` times the
no-arithmetic probe of the row kernels' launch shapes over the same rows (xr_probe_rows);
and `ceiling.copy` a plain stream of the same traffic, nothing else (xr_probe_copy: one read
and one write of every byte of the matrix, or two reads per write for the softmax backward,
through the runtime's device-to-device copy and a grid-stride copy kernel over a range of
grids), the achievable rate of that traffic at that size in any launch shape; for the
kernels that overwrite their input (the cross-entropy, element_mul), `ceiling.copy.in_place`
times the copy kernel in place as well, every vector written back where it was read.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--cpu-rows R]
                    [--workload c4|c3|c5|c2|c1|c4-mul|c4-nll|ln|bsr|sm-vocab|sm-few]
                    [--reduction mean|sum|none]
                    [--grad-scale S] [--rows M] [--no-extras]
    python bench.py --summarize-counters FETCH.csv WRITE.csv [--workload <name>]
                                                               (rocprofv3 --pmc output)
    python bench.py --summarize-trace KERNEL_TRACE.csv [--steps K] (rocprofv3 --kernel-trace)

The other workloads (c1 softmax fp32 128x1000, c2 softmax forward + backward bf16 4096^2,
c3 cross-entropy bf16 8192x32000, c5 cross-entropy fp32 2048x256000 padded) print the same
kind of line; small inputs are rotated through >= 1 GB of copies so no step reads data a
previous step left in the 256 MB Infinity Cache. `--reduction` / `--grad-scale` run the
cross-entropy workloads with another reduction or an upstream gradient folded into the
gradient write; `c4-mul` times the backward's element_mul (the stored gradient times an
upstream gradient of 0.5) over the 16384 x 128256 bf16 matrix; `c4-nll` the negative
log-softmax forward with a gathered loss over the same matrix, into a separate output;
`ln` a layer norm forward + backward (both stages) over 16384 x 8192 bf16 rows; `bsr` the
block-sparse softmax backward over 32 causal 4096 x 4096 maps of 64 x 64 bf16 blocks;
`sm-vocab` / `sm-few` the softmax forward + backward over split rows (4096 x 128256 bf16,
16 x 2^20 fp32) through one workspace. The softmax workloads time the oracle's softmax
(forward, then backward) as their CPU baseline; c4-mul, c4-nll, ln and bsr the oracle's
element_mul, negative log-softmax, layer norm (forward, then backward) and block-sparse
backward on a leading sample of the same inputs.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import re
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
TRACE = os.path.join(ROOT, "profiles", "xent_c4_kernel_trace.json")
KERNEL_SOURCES = [os.path.join(ROOT, "cross_entropy_reductions_amd", "csrc", f)
                  for f in ("xr_xent.hip", "xr_softmax.hip", "xr_rows.h", "xr_device.h",
                            "xr_internal.h", "xr_api.cpp")]
ROW_KERNEL = "xent_rows_kernel"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
C4_M, C4_V, C4_KEEP = 16384, 128256, 15565

DESCRIPTIONS = {
    "bsr": "block-sparse softmax backward through a look-up table, 32 maps of 4096 x 4096 in "
           "64 x 64 bf16 blocks (causal: local window of 4 blocks + every 8th block column, 453 "
           "blocks per map), in place, scale 0.125",
    "ln": "layer norm forward + backward (dx, and dw / db in two stages), M=16384, N=8192, "
          "bf16 x / dy / w / b, fp32 statistics and sums, eps=1e-5",
    "c4-nll": "negative log-softmax forward + loss gathered at each row's target, M=16384, "
              "N=128256, bf16 logits in, bf16 -log p out (separate buffer), fp32 losses",
    "c4-mul": "element_mul (stored gradient x upstream gradient 0.5, in place), M=16384, "
              "V=128256, bf16",
    "c1": "softmax forward, M=128, N=1000, fp32 logits 3 N(0,1), contiguous",
    "sm-vocab": "softmax forward + backward over long rows, M=4096, N=128256, bf16 in / fp32 "
                "accumulation, x and dy N(0,1), split rows through a workspace",
    "sm-few": "softmax forward + backward with few rows, M=16, N=1048576, fp32, x and dy "
              "N(0,1), split rows through a workspace",
    "c2": "softmax forward + backward, M=4096, N=4096, bf16 in / fp32 accumulation, "
          "x and dy N(0,1)",
    "c3": "fused cross-entropy loss+grad, M=8192 tokens (B=4, T=2048), V=32000, bf16 logits "
          "2 N(0,1), int64 targets, 10% ignore_index=-100, mean reduction",
    "c4": "fused cross-entropy loss+grad, M=16384 tokens, V=128256, bf16 logits N(0,1) + 4 "
          "spikes of +20 per row, int64 targets, 5% ignore_index=-100, mean reduction",
    "c5": "fused cross-entropy loss+grad, M=2048, V=256000, fp32 logits 8 N(0,1), row stride "
          "V+64, 1% all-equal rows, 1% half -inf rows, no ignored rows, mean reduction",
}


def _code_only(text: str) -> str:
    """Source text with comments and blank space removed, so that the hash below changes
    with the code and not with its comments."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
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


def profiled_kernel():
    """The row kernel's average duration from the committed rocprofv3 kernel trace of this
    command (a JSON beside its summary), or None if it is absent or was taken on other
    kernel sources."""
    try:
        with open(TRACE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c


# Timing-only events: no system-scope fence (L2 writeback and invalidate) when they are
# recorded, so they neither add that work between the kernels they bracket nor time it.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own launch stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
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


def cpu_baseline(workload: dict, rows: int, min_seconds: float = 10.0) -> dict:
    """The oracle as it stands on the first `rows` rows (count, loss + gradient, mean), in
    1024-row chunks so its float64 gradient buffer stays near 1 GB; whole passes are repeated
    until `min_seconds` have elapsed (at most 20), and the rate is taken over all of them."""
    import numpy as np

    import oracle

    orc = oracle.get()
    V = workload["N"]
    x = workload["x"][:rows]
    t = workload["target"][:rows]
    passes = 0
    t0 = time.perf_counter()
    while True:
        n, _ = orc.xent_count(t, V)
        losses = []
        for r0 in range(0, rows, 1024):
            _, loss = orc.xent_rows(x[r0:r0 + 1024], t[r0:r0 + 1024], V, n, want_grad=True)
            losses.append(loss)
        orc.mean(np.concatenate(losses), n)
        passes += 1
        sec = time.perf_counter() - t0
        if sec >= min_seconds or passes >= 20:
            break
    elt = 2 if workload["dtype"] == "bf16" else 4
    b = xent_bmin(rows, V, int((t != -100).sum()), elt) * passes
    return {"value": float(f"{b / sec / 1e9:.4g}"), "unit": "GB/s", "cores": orc.num_threads(),
            "kind": "oracle", "rows_per_s": round(rows * passes / sec, 1), "seconds": round(sec, 3),
            "sample": f"first {rows} of {workload['M']} rows of the same workload "
                      f"(V={V} {workload['dtype']}): float64 count, loss, gradient and mean, "
                      f"{passes} whole passes"}


def cpu_baseline_softmax(workload: dict, rows: int, min_seconds: float = 10.0) -> dict:
    """The oracle's softmax forward (and, when the workload has dy, its backward on the
    forward's output stored in the workload's dtype) on the first `rows` rows, whole passes
    repeated until `min_seconds` have elapsed; the rate counts the same minimal bytes as
    the GPU line."""
    import numpy as np

    import oracle
    import synth

    orc = oracle.get()
    M, N = workload["M"], workload["N"]
    rows = min(rows, M)
    x = workload["x"][:rows]
    dy = workload["dy"][:rows] if "dy" in workload else None
    bf16 = workload["dtype"] == "bf16"
    elt = 2 if bf16 else 4
    per_pass = rows * N * elt * (2 + (3 if dy is not None else 0))
    passes = 0
    t0 = time.perf_counter()
    while True:
        for r0 in range(0, rows, 256):
            y = orc.softmax_fwd(x[r0:r0 + 256])
            if dy is not None:
                ys = (synth.bf16_bits_from_f32(y.astype(np.float32)) if bf16
                      else y.astype(np.float32))
                orc.softmax_bwd(ys, dy[r0:r0 + 256])
        passes += 1
        sec = time.perf_counter() - t0
        if sec >= min_seconds:
            break
    return {"value": float(f"{per_pass * passes / sec / 1e9:.4g}"), "unit": "GB/s",
            "cores": orc.num_threads(), "kind": "oracle",
            "rows_per_s": round(rows * passes / sec, 1), "seconds": round(sec, 3),
            "sample": f"first {rows} of {M} rows of the same workload (N={N} "
                      f"{workload['dtype']}): float64 softmax forward"
                      + (", its output stored in the dtype, and the backward"
                         if dy is not None else "")
                      + f", {passes} whole passes"}


def _cpu_passes(one_pass, min_seconds: float):
    """Run `one_pass` until `min_seconds` have elapsed (at least once); (passes, seconds)."""
    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        passes += 1
        sec = time.perf_counter() - t0
        if sec >= min_seconds:
            return passes, sec


def _cpu_line(bytes_per_pass: int, rows: int, passes: int, sec: float, cores: int,
              sample: str) -> dict:
    return {"value": float(f"{bytes_per_pass * passes / sec / 1e9:.4g}"), "unit": "GB/s",
            "cores": cores, "kind": "oracle", "rows_per_s": round(rows * passes / sec, 1),
            "seconds": round(sec, 3), "sample": f"{sample}, {passes} whole passes"}


def cpu_baseline_element_mul(workload: dict, rows: int, scale: float,
                             min_seconds: float = 10.0) -> dict:
    """The oracle's element_mul (x times the row's upstream gradient) on the first `rows` rows
    of the matrix, 256 rows at a time; the rate counts the GPU line's minimal bytes."""
    import oracle

    orc = oracle.get()
    M, V = workload["M"], workload["N"]
    rows = min(rows, M)
    x = workload["x"][:rows]

    def one_pass():
        for r0 in range(0, rows, 256):
            orc.element_mul(x[r0:r0 + 256], scale)

    passes, sec = _cpu_passes(one_pass, min_seconds)
    return _cpu_line(2 * rows * V * 2, rows, passes, sec, orc.num_threads(),
                     f"first {rows} of {M} rows of the same matrix (V={V} bf16): float64 "
                     f"element_mul by {scale}")


def cpu_baseline_nll(workload: dict, idx, rows: int, min_seconds: float = 10.0) -> dict:
    """The oracle's negative log-softmax with the gathered loss on the first `rows` rows."""
    import oracle

    orc = oracle.get()
    M, N = workload["M"], workload["N"]
    rows = min(rows, M)
    x = workload["x"][:rows]

    def one_pass():
        for r0 in range(0, rows, 256):
            orc.nll_fwd(x[r0:r0 + 256], idx[r0:r0 + 256])

    passes, sec = _cpu_passes(one_pass, min_seconds)
    return _cpu_line(2 * rows * N * 2 + 12 * rows, rows, passes, sec, orc.num_threads(),
                     f"first {rows} of {M} rows of the same matrix (N={N} bf16): float64 "
                     "-log softmax and the gathered loss")


def cpu_baseline_layernorm(workload: dict, rows: int, min_seconds: float = 10.0) -> dict:
    """The oracle's layer norm forward, then its backward, on the first `rows` rows, 1024 rows
    at a time (dw, db summed per piece); the rate counts the GPU line's minimal bytes."""
    import oracle

    orc = oracle.get()
    M, N = workload["M"], workload["N"]
    rows = min(rows, M)
    x, dy, w, b, eps = workload["x"][:rows], workload["dy"][:rows], workload["w"], workload["b"], \
        workload["eps"]
    elt = 2 if workload["dtype"] == "bf16" else 4

    def one_pass():
        for r0 in range(0, rows, 1024):
            orc.layernorm_fwd(x[r0:r0 + 1024], w, b, eps)
            orc.layernorm_bwd(dy[r0:r0 + 1024], x[r0:r0 + 1024], w, eps)

    passes, sec = _cpu_passes(one_pass, min_seconds)
    per_pass = (2 * rows * N * elt + 2 * N * elt + 8 * rows) + \
        (3 * rows * N * elt + N * elt + 8 * rows + 2 * N * elt)
    return _cpu_line(per_pass, rows, passes, sec, orc.num_threads(),
                     f"first {rows} of {M} rows of the same workload (N={N} "
                     f"{workload['dtype']}): float64 layer norm forward, then backward")


def cpu_baseline_bsr(workload: dict, maps: int, min_seconds: float = 10.0) -> dict:
    """The oracle's block-sparse softmax backward on the first `maps` attention maps, one map at
    a time; the rate counts the GPU line's minimal bytes for those maps."""
    import oracle

    orc = oracle.get()
    Z = workload["Z"]
    maps = max(1, min(maps, Z))
    y, dy, lut = workload["y"], workload["dy"], workload["lut"]
    elt = 2 if workload["dtype"] == "bf16" else 4

    def one_pass():
        for z in range(maps):
            orc.bsr_softmax_bwd(y[z:z + 1], dy[z:z + 1], lut, workload["n_brows"],
                                workload["block"], workload["scale"])

    passes, sec = _cpu_passes(one_pass, min_seconds)
    listed = int(workload["layout"].sum()) * maps * workload["block"] ** 2
    rows = maps * workload["n_brows"] * workload["block"]
    return _cpu_line(3 * listed * elt + lut.size * 4, rows, passes, sec, orc.num_threads(),
                     f"first {maps} of {Z} maps of the same workload ({workload['seq']}^2 in "
                     f"{workload['block']}-blocks, {workload['dtype']}): float64 block-sparse "
                     "softmax backward")


def _device_matrix(torch, a, dev):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def _timed(ev, steps, warmup, launch):
    """Warm up, then time `steps` launches back to back, with the row kernel of each timed
    step bracketed by its own pair of events."""
    import torch

    import cross_entropy_reductions_amd as xr

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    starts = [ev.create() for _ in range(steps)]
    stops = [ev.create() for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        xr.set_profile_events(starts[i], stops[i])
        launch(warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    xr.set_profile_events(None, None)
    ms = [ev.elapsed_ms(a, b) for a, b in zip(starts, stops)]
    for e in starts + stops:
        ev.destroy(e)
    return wall, ms


# Launch shapes of the row kernels (threads, 16-byte vectors per thread): one row operand,
# and two (the softmax backward).
FWD_SHAPES = [(64, 4), (64, 8), (64, 16), (128, 8), (128, 16), (256, 8), (256, 16), (512, 8),
              (512, 16), (1024, 16)]
BWD_SHAPES = [(64, 4), (64, 8), (128, 8), (256, 8), (512, 8), (1024, 8)]


def probe_shapes(nv: int, two_inputs: bool):
    """(threads, vpt, split): the row-kernel shapes that hold a row of nv 16-byte vectors in
    1-32 chunks of at least 64 vectors, each chunk filling more than half of the shape."""
    out = []
    for S in (1, 2, 4, 8, 16, 32):
        chunk = -(-nv // S)
        if chunk < 64:
            break
        for t, v in (BWD_SHAPES if two_inputs else FWD_SHAPES):
            if chunk <= t * v < 2 * chunk:
                out.append((t, v, S))
    return out


def ceiling(args, kernel_ms: float, nbytes: int, shape, shapes, launch_probe) -> dict:
    """The memory-ceiling probe (xr_probe_rows: the row kernels' loads and stores, none of
    their arithmetic) over the same rows and buffers: timed in the kernel's own launch shape
    and in every shape of `shapes`, the same way as the kernel (HIP events around each
    launch). Returns the probe's figures and the kernel's time as a fraction of them."""
    res = {}
    best = None
    for sh in dict.fromkeys([tuple(shape)] + [tuple(x) for x in shapes]):
        _, ms = _timed(HipEvents(), args.steps, args.warmup, lambda i, sh=sh: launch_probe(i, *sh))
        avg = statistics.mean(ms)
        if sh == tuple(shape):
            res["same_shape"] = {"shape": list(sh), "ms_avg": round(avg, 5),
                                 "GBps": round(nbytes / avg / 1e6, 1)}
        if best is None or avg < best[1]:
            best = (sh, avg)
    res["best"] = {"shape": list(best[0]), "ms_avg": round(best[1], 5),
                   "GBps": round(nbytes / best[1] / 1e6, 1)}
    res["kernel_frac_of_same_shape"] = round(res["same_shape"]["ms_avg"] / kernel_ms, 4)
    res["kernel_frac_of_best"] = round(best[1] / kernel_ms, 4)
    return res


def run_xent(args, name: str) -> dict:
    import torch

    import cross_entropy_reductions_amd as xr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    w = synth.WORKLOADS[name](**({"M": args.rows} if args.rows else {}))
    M, V = w["M"], w["N"]
    t = torch.from_numpy(w["target"]).to(dev)
    x0 = _device_matrix(torch, w["x"], dev)
    n_keep = int((w["target"] != -100).sum())
    elt = 2 if w["dtype"] == "bf16" else 4
    print(f"[bench] {name} ready in {time.perf_counter() - t_gen:.1f}s: M={M} V={V} "
          f"n={n_keep}", file=sys.stderr, flush=True)

    steps, warmup = args.steps, args.warmup
    copies = [x0.clone() for _ in range(warmup + steps)]
    del x0
    row_loss = torch.empty(M, dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    counts = torch.empty(3, dtype=torch.int32, device=dev)
    dt = copies[0].dtype
    ws = torch.empty(max(256, xr.xent_workspace_bytes(M, V, dt)), dtype=torch.uint8, device=dev)

    scale = None
    if args.grad_scale is not None:
        scale = torch.tensor([args.grad_scale], dtype=torch.float32, device=dev)

    def launch(i):
        xr.xent_fwd_bwd(copies[i][:, :V], t, -100, row_loss=row_loss, mean_loss=mean,
                        counts=counts, workspace=ws, reduction=args.reduction,
                        grad_scale=scale)

    wall, kernel_ms = _timed(HipEvents(), steps, warmup, launch)
    c = counts.cpu().tolist()
    assert c[0] == n_keep and c[2] == 0, f"unexpected counts {c}"
    bmin = xent_bmin(M, V, n_keep, elt)
    p = xr.plan("xent", M, V, dt)
    out = _line(args, name, bmin, M, wall, kernel_ms, ROW_KERNEL,
                {"M": M, "V": V, "n_non_ignore": n_keep, "bytes_min": bmin, "path": p["path"],
                 "threads": p["threads"], "split": p["split"], "grid": p["grid"],
                 "reduction": args.reduction, "grad_scale": args.grad_scale},
                w["dtype"])
    if name == "c4" and args.reduction == "mean" and args.grad_scale is None and not args.rows:
        out["roofline"]["traffic"] = measured_traffic()
        prof = profiled_kernel()
        if prof is not None:
            ms = prof["kernel_ms_avg"]
            out["roofline"]["profiled"] = {
                "kernel_ms_avg": ms, "achieved": round(bmin / ms / 1e6, 1),
                "frac": round(bmin / ms / 1e6 / PEAK_HBM_GBS, 4), "calls": prof["calls"],
                "source": "profiles/xent_c4_kernel_trace.md"}
    if getattr(args, "ceiling", False) and args.grad_scale is None and args.reduction == "mean":
        import cross_entropy_reductions_amd as xr_

        nv = V * elt // 16

        def probe(i, t_, v_, s_):
            x = copies[i][:, :V]
            xr_.probe_rows(x, x, threads=t_, vpt=v_, split=s_, target=t)

        out["roofline"]["ceiling"] = ceiling(
            args, out["roofline"]["kernel_ms_avg"], bmin,
            (p["threads"], p["vec_per_thread"], p["split"]), probe_shapes(nv, False), probe)
        if not args.rows:
            n_c = len(copies)
            out["roofline"]["ceiling"]["copy"] = copy_ceiling(
                args, out["roofline"]["kernel_ms_avg"], bmin,
                2 * copies[0].numel() * copies[0].element_size(),
                lambda i, g, t_: xr_.probe_copy(copies[(i + 1) % n_c], copies[i % n_c],
                                                workgroups=g, threads=t_),
                launch_in_place=lambda i, g, t_: xr_.probe_copy(copies[i], copies[i],
                                                                workgroups=g, threads=t_))
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, min(args.cpu_rows, M))
    return out


# Launches of the plain copy of the ceiling: (threads, 16-byte vectors per thread), the grid
# following from the size; (0, 0) is the runtime's device-to-device copy (one input only).
COPY_LAUNCHES = [(0, 0)] + [(256, v) for v in (1, 2, 4, 8, 32, 128)] + [(512, v) for v in (1, 2)]


def copy_ceiling(args, kernel_ms: float, bmin: int, nbytes: int, launch_copy,
                 two_inputs: bool = False, launch_in_place=None) -> dict:
    """The plain copy of a kernel's traffic, nothing else (xr_probe_copy): one read and one
    write of every byte (or two reads per write with two inputs) through the runtime's
    device-to-device copy and a grid-stride copy kernel over a range of grids, timed like the
    row kernel (HIP events around each launch; launch_copy(i, workgroups, threads) rotates
    through the benchmark's buffers). nbytes: bytes read plus written by one launch. Returns
    each launch's rate and the row kernel's rate over the fastest copy's. For a kernel that
    overwrites its input, launch_in_place(i, workgroups, threads) times the copy kernel in
    place as well (every vector written back where it was read), reported under "in_place"."""
    nvec = nbytes // (3 if two_inputs else 2) // 16

    def sweep(launch, with_memcpy):
        launches, best = {}, None
        for t_, v in COPY_LAUNCHES:
            if t_ == 0 and not with_memcpy:
                continue
            g = 0 if t_ == 0 else max(1, min(-(-nvec // (t_ * v)), 2 ** 31 - 1))
            _, ms = _timed(HipEvents(), args.steps, args.warmup,
                           lambda i, g=g, t_=t_: launch(i, g, t_ or 256))
            avg = statistics.mean(ms)
            key = "memcpy" if g == 0 else f"{g}x{t_}"
            launches[key] = {"ms_avg": round(avg, 5), "GBps": round(nbytes / avg / 1e6, 1)}
            if best is None or avg < best[1]:
                best = (key, avg)
        return {"launches": launches,
                "best": {"launch": best[0], "GBps": round(nbytes / best[1] / 1e6, 1)},
                "kernel_rate_over_copy": round((bmin / kernel_ms) / (nbytes / best[1]), 4)}

    res = {"bytes_moved": nbytes, "inputs": 2 if two_inputs else 1}
    res.update(sweep(launch_copy, not two_inputs))
    if launch_in_place is not None:
        res["in_place"] = sweep(launch_in_place, False)
    return res


def run_element_mul(args, name: str) -> dict:
    """The backward's element_mul over the c4 matrix: every row read and written once."""
    import torch

    import cross_entropy_reductions_amd as xr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.xent_c4()
    M, V = w["M"], w["N"]
    x0 = _device_matrix(torch, w["x"], dev)
    copies = [x0.clone() for _ in range(args.warmup + args.steps)]
    del x0
    scale = torch.tensor([0.5], dtype=torch.float32, device=dev)

    def launch(i):
        xr.element_mul(copies[i], scale)

    wall, kernel_ms = _timed(HipEvents(), args.steps, args.warmup, launch)
    bmin = 2 * M * V * 2 + 4
    out = _line(args, name, bmin, M, wall, kernel_ms, "element_mul_kernel",
                {"M": M, "V": V, "bytes_min": bmin, "threads": 1024, "vec_per_thread": 8},
                "bf16")
    if getattr(args, "ceiling", False):
        n_c = len(copies)
        out["roofline"]["ceiling"] = {"copy": copy_ceiling(
            args, out["roofline"]["kernel_ms_avg"], bmin, 2 * M * V * 2,
            lambda i, g, t_: xr.probe_copy(copies[(i + 1) % n_c], copies[i % n_c], workgroups=g,
                                           threads=t_),
            launch_in_place=lambda i, g, t_: xr.probe_copy(copies[i], copies[i], workgroups=g,
                                                           threads=t_))}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_element_mul(w, args.cpu_rows, 0.5)
    return out


def run_nll(args, name: str) -> dict:
    """-log softmax of the c4 logits into a separate output, plus the gathered losses."""
    import numpy as np
    import torch

    import cross_entropy_reductions_amd as xr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.xent_c4()
    M, N = w["M"], w["N"]
    # one device copy of known size before the timed region (it calibrates HBM counters)
    x = _device_matrix(torch, w["x"], dev).clone()
    idx = torch.from_numpy(w["target"]).clamp(min=0).to(dev)
    out = torch.empty_like(x)
    loss = torch.empty(M, dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, int(xr.lib.xr_nll_fwd_workspace_bytes(M, N, xr.BF16))),
                     dtype=torch.uint8, device=dev)

    def launch(i):
        xr.nll_fwd(x, idx, out, loss, workspace=ws)

    wall, kernel_ms = _timed(HipEvents(), args.steps, args.warmup, launch)
    bmin = 2 * M * N * 2 + 12 * M
    p = xr.plan("nll_fwd", M, N, x.dtype)
    res = _line(args, name, bmin, M, wall, kernel_ms, "softmax_fwd_kernel (negative log)",
                {"M": M, "N": N, "bytes_min": bmin, "path": p["path"], "threads": p["threads"],
                 "vec_per_thread": p["vec_per_thread"], "split": p["split"], "grid": p["grid"]},
                "bf16")
    if getattr(args, "ceiling", False):
        res["roofline"]["ceiling"] = {"copy": copy_ceiling(
            args, res["roofline"]["kernel_ms_avg"], bmin, 2 * M * N * 2,
            lambda i, g, t_: xr.probe_copy(out, x, workgroups=g, threads=t_))}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline_nll(w, np.clip(w["target"], 0, None), args.cpu_rows)
    return res


def run_layernorm(args, name: str) -> dict:
    """Forward then backward on the same rows; inputs rotated over >= 1 GB of copies."""
    import torch

    import cross_entropy_reductions_amd as xr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.layernorm_ln()
    M, N = wl["M"], wl["N"]
    x = _device_matrix(torch, wl["x"], dev)
    dy = _device_matrix(torch, wl["dy"], dev)
    w = _device_matrix(torch, wl["w"], dev)
    b = _device_matrix(torch, wl["b"], dev)
    elt = x.element_size()
    per_set = 5 * M * N * elt
    nsets = max(2, -(-(1 << 30) // per_set))
    xs = [x.clone() for _ in range(nsets)]
    dys = [dy.clone() for _ in range(nsets)]
    ys = [torch.empty_like(x) for _ in range(nsets)]
    dxs = [torch.empty_like(x) for _ in range(nsets)]
    mean = torch.empty(M, dtype=torch.float32, device=dev)
    rstd = torch.empty(M, dtype=torch.float32, device=dev)
    dw = torch.empty(N, dtype=x.dtype, device=dev)
    db = torch.empty(N, dtype=x.dtype, device=dev)
    ws = torch.empty(max(16, xr.layernorm_bwd_workspace_bytes(M, N, x.dtype)), dtype=torch.uint8,
                     device=dev)
    ev = HipEvents()
    bwd_events = [(ev.create(), ev.create()) for _ in range(args.warmup + args.steps)]

    def launch(i):
        j = i % nsets
        xr.layernorm_fwd(xs[j], w, b, wl["eps"], out=ys[j], mean=mean, rstd=rstd)
        xr.set_profile_events(*bwd_events[i])
        xr.layernorm_bwd(dys[j], xs[j], w, mean, rstd, dx=dxs[j], dw=dw, db=db, workspace=ws)

    wall, fwd_ms = _timed(ev, args.steps, args.warmup, launch)
    bwd_ms = [ev.elapsed_ms(a, b_) for a, b_ in bwd_events[args.warmup:]]
    for a, b_ in bwd_events:
        ev.destroy(a)
        ev.destroy(b_)
    b_fwd = 2 * M * N * elt + 2 * N * elt + 8 * M
    b_bwd = 3 * M * N * elt + N * elt + 8 * M + 2 * N * elt
    out = _line(args, name, b_fwd + b_bwd, M, wall, fwd_ms, "ln_fwd_kernel",
                {"M": M, "N": N, "bytes_min": b_fwd + b_bwd, "input_sets": nsets,
                 "workspace_bytes": ws.numel()}, "bf16", kernel_bytes=b_fwd)
    kavg = statistics.mean(bwd_ms)
    out["roofline_bwd"] = {"bound": "hbm", "achieved": round(b_bwd / kavg / 1e6, 1),
                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(b_bwd / kavg / 1e6 / PEAK_HBM_GBS, 4),
                           "kernel": "ln_bwd_kernel (stage 1)", "kernel_ms_avg": round(kavg, 5)}
    if getattr(args, "ceiling", False):
        mat = M * N * elt
        out["roofline"]["ceiling"] = {"copy": copy_ceiling(
            args, out["roofline"]["kernel_ms_avg"], b_fwd, 2 * mat,
            lambda i, g, t_: xr.probe_copy(ys[i % nsets], xs[i % nsets], workgroups=g,
                                           threads=t_))}
        out["roofline_bwd"]["ceiling"] = {"copy": copy_ceiling(
            args, kavg, b_bwd, 3 * mat,
            lambda i, g, t_: xr.probe_copy(dxs[i % nsets], xs[i % nsets], dys[i % nsets],
                                           workgroups=g, threads=t_), two_inputs=True)}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_layernorm(wl, args.cpu_rows)
    return out


def run_bsr(args, name: str) -> dict:
    """In-place block-sparse backward; inputs rotated over >= 1 GB of copies."""
    import torch

    import cross_entropy_reductions_amd as xr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.bsr_softmax()
    y = _device_matrix(torch, w["y"], dev)
    d = _device_matrix(torch, w["dy"], dev)
    lut = torch.from_numpy(w["lut"]).to(dev)
    elt = y.element_size()
    per_set = 2 * y.numel() * elt
    nsets = max(2, -(-(1 << 30) // per_set))
    ys = [y.clone() for _ in range(nsets)]
    ds = [d.clone() for _ in range(nsets)]

    def launch(i):
        j = i % nsets
        xr.bsr_softmax_bwd(ys[j], ds[j], lut, w["n_brows"], w["n_blocks"], w["block"], w["scale"])

    wall, kernel_ms = _timed(HipEvents(), args.steps, args.warmup, launch)
    listed = int(w["layout"].sum()) * w["Z"] * w["block"] ** 2
    bmin = 3 * listed * elt + lut.numel() * 4
    rows = w["Z"] * w["n_brows"] * w["block"]
    out = _line(args, name, bmin, rows, wall, kernel_ms, "bsr_softmax_bwd_kernel",
                {"Z": w["Z"], "seq": w["seq"], "block": w["block"], "n_blocks": w["n_blocks"],
                 "bytes_min": bmin, "input_sets": nsets}, "bf16")
    if getattr(args, "ceiling", False):
        # y and dy read, the result written to another buffer of the same size
        out["roofline"]["ceiling"] = {"copy": copy_ceiling(
            args, out["roofline"]["kernel_ms_avg"], bmin, 3 * y.numel() * elt,
            lambda i, g, t_: xr.probe_copy(ds[(i + 1) % nsets], ys[i % nsets], ds[i % nsets],
                                           workgroups=g, threads=t_), two_inputs=True)}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_bsr(w, max(1, args.cpu_rows * w["Z"] // 16384))
    return out


def run_softmax(args, name: str) -> dict:
    import torch

    import cross_entropy_reductions_amd as xr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[name](**({"M": args.rows} if args.rows else {}))
    M, N = w["M"], w["N"]
    x = _device_matrix(torch, w["x"], dev)
    elt = x.element_size()
    bwd = "dy" in w
    dy = _device_matrix(torch, w["dy"], dev) if bwd else None
    per_set = (4 if bwd else 2) * M * N * elt
    nsets = max(2, -(-(1 << 30) // per_set))  # >= 1 GB of distinct inputs and outputs
    xs = [x.clone() for _ in range(nsets)]
    dys = [dy.clone() for _ in range(nsets)] if bwd else None
    ys = [torch.empty_like(x) for _ in range(nsets)]
    dxs = [torch.empty_like(x) for _ in range(nsets)] if bwd else None
    # one workspace for both directions, allocated before the timed region
    ws = torch.empty(max(256, xr.softmax_workspace_bytes(M, N, x.dtype)), dtype=torch.uint8,
                     device=dev)
    ev = HipEvents()
    bwd_events = [(ev.create(), ev.create()) for _ in range(args.warmup + args.steps)]

    def launch(i):
        j = i % nsets
        xr.softmax_fwd(xs[j], ys[j], workspace=ws)  # bracketed by the events _timed installs
        if bwd:
            xr.set_profile_events(*bwd_events[i])
            xr.softmax_bwd(ys[j], dys[j], dxs[j], workspace=ws)

    wall, fwd_ms = _timed(ev, args.steps, args.warmup, launch)
    bwd_ms = [ev.elapsed_ms(a, b) for a, b in bwd_events[args.warmup:]] if bwd else []
    for a, b in bwd_events:
        ev.destroy(a)
        ev.destroy(b)
    b_fwd = 2 * M * N * elt
    b_bwd = 3 * M * N * elt if bwd else 0
    p = xr.plan("softmax_fwd_ws", M, N, x.dtype)
    out = _line(args, name, b_fwd + b_bwd, M, wall, fwd_ms,
                "softmax_split_kernel" if p["split"] > 1 else "softmax_fwd_kernel",
                {"M": M, "N": N, "bytes_min": b_fwd + b_bwd, "path": p["path"],
                 "threads": p["threads"], "split": p["split"], "grid": p["grid"],
                 "load_priority": p["load_priority"], "input_sets": nsets},
                w["dtype"], kernel_bytes=b_fwd)
    if bwd:
        kavg = statistics.mean(bwd_ms)
        out["roofline_bwd"] = {"bound": "hbm", "achieved": round(b_bwd / kavg / 1e6, 1),
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(b_bwd / kavg / 1e6 / PEAK_HBM_GBS, 4),
                               "kernel": "softmax_bwd_split_kernel"
                               if xr.plan("softmax_bwd_ws", M, N, x.dtype)["split"] > 1
                               else "softmax_bwd_kernel", "kernel_ms_avg": round(kavg, 5),
                               "kernel_ms_min": round(min(bwd_ms), 5), "bytes": b_bwd}
    if getattr(args, "ceiling", False) and name != "c2":
        out["roofline"]["ceiling"] = {"copy": copy_ceiling(
            args, out["roofline"]["kernel_ms_avg"], b_fwd, b_fwd,
            lambda i, g, t_: xr.probe_copy(ys[i % nsets], xs[i % nsets], workgroups=g,
                                           threads=t_))}
        if bwd:
            out["roofline_bwd"]["ceiling"] = {"copy": copy_ceiling(
                args, out["roofline_bwd"]["kernel_ms_avg"], b_bwd, b_bwd,
                lambda i, g, t_: xr.probe_copy(dxs[i % nsets], ys[i % nsets], dys[i % nsets],
                                               workgroups=g, threads=t_), two_inputs=True)}
    if getattr(args, "ceiling", False) and name == "c2":
        nv = N * elt // 16

        def probe_fwd(i, t_, v_, s_):
            j = i % nsets
            xr.probe_rows(ys[j], xs[j], threads=t_, vpt=v_, split=s_)

        def probe_bwd(i, t_, v_, s_):
            j = i % nsets
            xr.probe_rows(dxs[j], ys[j], dys[j], threads=t_, vpt=v_, split=s_)

        out["roofline"]["ceiling"] = ceiling(
            args, out["roofline"]["kernel_ms_avg"], b_fwd,
            (p["threads"], p["vec_per_thread"], p["split"]), probe_shapes(nv, False), probe_fwd)
        pb = xr.plan("softmax_bwd_ws", M, N, x.dtype)
        out["roofline_bwd"]["ceiling"] = ceiling(
            args, out["roofline_bwd"]["kernel_ms_avg"], b_bwd,
            (pb["threads"], pb["vec_per_thread"], pb["split"]), probe_shapes(nv, True), probe_bwd)
        if not args.rows:
            out["roofline"]["ceiling"]["copy"] = copy_ceiling(
                args, out["roofline"]["kernel_ms_avg"], b_fwd, b_fwd,
                lambda i, g, t_: xr.probe_copy(ys[i % nsets], xs[i % nsets], workgroups=g,
                                               threads=t_))
            out["roofline_bwd"]["ceiling"]["copy"] = copy_ceiling(
                args, out["roofline_bwd"]["kernel_ms_avg"], b_bwd, b_bwd,
                lambda i, g, t_: xr.probe_copy(dxs[i % nsets], ys[i % nsets], dys[i % nsets],
                                               workgroups=g, threads=t_), two_inputs=True)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_softmax(w, args.cpu_rows)
    return out


def _line(args, name, bmin, M, wall, kernel_ms, kernel, config, dtype, kernel_bytes=None):
    steps = args.steps
    gbs = bmin / (wall / steps) / 1e9
    kavg = statistics.mean(kernel_ms)
    kb = bmin if kernel_bytes is None else kernel_bytes
    kgbs = kb / (kavg / 1e3) / 1e9
    metric = ("achieved HBM GB/s (% of peak) and rows/s for fused xent fwd+bwd, V=128256 bf16"
              if name == "c4" else f"achieved HBM GB/s (% of peak) and rows/s, {name}")
    return {
        "metric": metric,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{name}: {DESCRIPTIONS[name]}" +
                   (f" (rows overridden: M={M}; a scaling check, not the configuration)"
                    if args.rows else ""), **config},
        "pct_of_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "rows_per_s": round(M / (wall / steps), 1),
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": kernel, "kernel_ms_avg": round(kavg, 5),
                     "kernel_ms_min": round(min(kernel_ms), 5)},
    }


EXTRAS = ("c2", "c3", "c5")


def run_extras(args) -> dict:
    """The other configurations the 75 % target covers, timed the same way in the same
    process after the headline: per kernel, its minimal bytes, average and fastest launch
    (HIP events), achieved GB/s and fraction of 8 TB/s, and the whole step."""
    import copy

    import torch

    out = {}
    prof = profiled_kernel()
    profiled = {w: {k: {key: v[key] for key in ("kernel_ms_avg", "achieved_GBps", "frac", "calls")}
                    for k, v in ks.items()}
                for w, ks in (prof or {}).get("other_configs", {}).items()}
    for name in EXTRAS:
        torch.cuda.empty_cache()
        a = copy.copy(args)
        a.no_cpu, a.rows, a.reduction, a.grad_scale = True, 0, "mean", None
        a.ceiling = not args.no_ceiling
        line = run_softmax(a, name) if name == "c2" else run_xent(a, name)
        kernels = [("softmax_fwd" if name == "c2" else "xent", line["roofline"])]
        if "roofline_bwd" in line:
            kernels.append(("softmax_bwd", line["roofline_bwd"]))
        bmin = line["config"]["bytes_min"]
        out[name] = {
            "workload": line["config"]["workload"], "bytes_min": bmin,
            "ms_per_step": line["ms_per_step"], "step_GBps": line["value"],
            "kernels": {
                k: {"kernel": r["kernel"], "kernel_ms_avg": r["kernel_ms_avg"],
                    "kernel_ms_min": r.get("kernel_ms_min"), "achieved_GBps": r["achieved"],
                    "frac": r["frac"], **({"ceiling": r["ceiling"]} if "ceiling" in r else {}),
                    **({"profiled": profiled[name][k]}
                       if name in profiled and k in profiled[name] else {})}
                for k, r in kernels}}
        print(f"[bench] {name}: " + ", ".join(
            f"{k} {v['achieved_GBps']} GB/s ({100 * v['frac']:.1f} %)"
            for k, v in out[name]["kernels"].items()), file=sys.stderr, flush=True)
    return out


# Counter summaries: per workload, the matrix the benchmark copies before its timed region
# (bytes of one copy), and the kernels to summarise with their minimal bytes per launch.
LN_M, LN_N = 16384, 8192
VOCAB_M, VOCAB_N = 4096, 128256
FEW_M, FEW_N = 16, 1 << 20
COUNTER_WORKLOADS = {
    "c4": (C4_M * C4_V * 2, [(ROW_KERNEL, xent_bmin(C4_M, C4_V, C4_KEEP, 2))]),
    "c3": (8192 * 32000 * 2, [(ROW_KERNEL, xent_bmin(8192, 32000, 7373, 2))]),
    "c5": (2048 * 256064 * 4, [(ROW_KERNEL, xent_bmin(2048, 256000, 2048, 4))]),
    "c2": (4096 * 4096 * 2, [("softmax_fwd_kernel", 2 * 4096 * 4096 * 2),
                             ("softmax_bwd_kernel", 3 * 4096 * 4096 * 2)]),
    "c4-mul": (C4_M * C4_V * 2, [("element_mul_kernel", 2 * C4_M * C4_V * 2 + 4)]),
    "c4-nll": (C4_M * C4_V * 2, [("softmax_split_kernel", 2 * C4_M * C4_V * 2 + 12 * C4_M)]),
    # layer norm: the backward's stage 1 also writes one row of fp32 column sums per workgroup
    # (not counted here: they are the price of a deterministic dw / db)
    "ln": (LN_M * LN_N * 2, [("ln_fwd_kernel", 2 * LN_M * LN_N * 2 + 2 * LN_N * 2 + 8 * LN_M),
                             ("ln_bwd_kernel", 3 * LN_M * LN_N * 2 + LN_N * 2 + 8 * LN_M)]),
    "sm-vocab": (VOCAB_M * VOCAB_N * 2,
                 [("softmax_split_kernel", 2 * VOCAB_M * VOCAB_N * 2),
                  ("softmax_bwd_split_kernel", 3 * VOCAB_M * VOCAB_N * 2)]),
    "sm-few": (FEW_M * FEW_N * 4, [("softmax_split_kernel", 2 * FEW_M * FEW_N * 4),
                                   ("softmax_bwd_split_kernel", 3 * FEW_M * FEW_N * 4)]),
}


def counter_workload(name: str):
    """(bytes of the copied matrix, [(kernel, minimal bytes per launch)]) of a workload."""
    if name != "bsr":
        return COUNTER_WORKLOADS[name]
    import synth
    w = synth.bsr_softmax(Z=1)  # the layout only: Z, seq and block are the workload's
    Z, seq, block = 32, w["seq"], w["block"]
    listed = int(w["layout"].sum()) * Z * block * block
    stored = Z * w["n_blocks"] * block * block * 2
    return stored, [("bsr_softmax_bwd_kernel", 3 * listed * 2 + w["lut"].size * 4)]


def summarize_counters(fetch_csv: str, write_csv: str, workload: str = "c4") -> dict:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of a workload's row kernel(s) from a run of
    `bench.py --workload <workload>`, each scaled by what the same counter reads for the
    runtime's device copies of the workload's input matrix (the copies bench.py makes before
    its timed region: one known read and one known write of the whole matrix). For c4 the
    result is what bench.py reports as roofline.traffic."""
    matrix, kernels = counter_workload(workload)

    def per_kernel(path):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name", "")
                key = COPY_KERNEL if COPY_KERNEL in name else next(
                    (k for k, _ in kernels if k in name), None)
                if key is not None:
                    vals.setdefault(key, []).append(float(row["Counter_Value"]) * 1024.0)
        return vals

    f, w = per_kernel(fetch_csv), per_kernel(write_csv)
    # the matrix copies, not the runtime's small ones (a copy's FETCH_SIZE reads about half
    # its bytes, so the cut sits well below that)
    copy_f = [v for v in f[COPY_KERNEL] if v > 0.25 * matrix]
    copy_w = [v for v in w[COPY_KERNEL] if v > 0.25 * matrix]
    scale_f = matrix / statistics.median(copy_f)
    scale_w = matrix / statistics.median(copy_w)
    out = {}
    for name, bmin in kernels:
        fetch = statistics.median(f[name]) * scale_f
        write = statistics.median(w[name]) * scale_w
        out[name] = {"kernel": name, "kernel_source_hash": kernel_source_hash(),
                     "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
                     "traffic_bytes_per_launch": round(fetch + write), "bytes_min": bmin,
                     "traffic_over_bytes_min": round((fetch + write) / bmin, 4),
                     "copy_scale_fetch": round(scale_f, 4), "copy_scale_write": round(scale_w, 4),
                     "dispatches": {"row_kernel": len(f[name]), "copy": len(copy_f)}}
    return out[ROW_KERNEL] if workload == "c4" else {"workload": workload, "kernels": out}


def traced_launches():
    """Every traced kernel of the default run: (name in the summary, kernel name prefix and
    dtype template argument, workgroup size, work-items, minimal bytes), from the library's
    plans on a modelled 256-CU device (plans of rows this many do not depend on occupancy)."""
    import torch

    import cross_entropy_reductions_amd as xr

    def xent(M, V, keep, dt, elt):
        p = xr.plan_model("xent", M, V, dt, 256, 2)
        return (f"{ROW_KERNEL}<{1 if dt == torch.bfloat16 else 0}, {p['threads']},", p["threads"],
                p["grid_total"] * p["threads"], xent_bmin(M, V, keep, elt))

    def soft(op, kernel, nbytes):
        p = xr.plan_model(op, 4096, 4096, torch.bfloat16, 256, 2)
        return (f"{kernel}<1, {p['threads']},", p["threads"], p["grid_total"] * p["threads"],
                nbytes)

    return {"c4": {"xent": xent(C4_M, C4_V, C4_KEEP, torch.bfloat16, 2)},
            "c3": {"xent": xent(8192, 32000, 7373, torch.bfloat16, 2)},
            "c5": {"xent": xent(2048, 256000, 2048, torch.float32, 4)},
            "c2": {"softmax_fwd": soft("softmax_fwd_ws", "softmax_fwd_kernel", 2 * 4096 * 4096 * 2),
                   "softmax_bwd": soft("softmax_bwd_ws", "softmax_bwd_kernel", 3 * 4096 * 4096 * 2)}}


def summarize_trace(trace_csv: str, steps: int) -> dict:
    """Each benchmarked kernel's average duration from a rocprofv3 --kernel-trace CSV of the
    default command: its launches in its plan's launch shape (told apart from the same
    kernel's launches on the other workloads by dtype, workgroup and grid size), the last
    `steps` of them in launch order being the timed steps. The headline's figures sit at the
    top level, the others under other_configs, all with the kernel-source hash."""
    want = traced_launches()
    launches = {(w, k): [] for w, ks in want.items() for k in ks}
    with open(trace_csv) as f:
        for row in csv.DictReader(f):
            for (w, k), lst in launches.items():
                prefix, threads, items, _ = want[w][k]
                if prefix in row["Kernel_Name"] and int(row["Workgroup_Size_X"]) == threads \
                        and int(row["Grid_Size_X"]) == items:
                    lst.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"])))

    def fig(w, k):
        ns = [e - s for s, e in sorted(launches[(w, k)])[-steps:]]
        ms = statistics.mean(ns) / 1e6
        b = want[w][k][3]
        return {"kernel_ms_avg": round(ms, 5), "kernel_ms_min": round(min(ns) / 1e6, 5),
                "calls": len(ns), "launches_traced": len(launches[(w, k)]), "bytes_min": b,
                "achieved_GBps": round(b / ms / 1e6, 1),
                "frac": round(b / ms / 1e6 / PEAK_HBM_GBS, 4)}

    out = {"kernel": ROW_KERNEL, "kernel_source_hash": kernel_source_hash(), **fig("c4", "xent")}
    out["other_configs"] = {w: {k: fig(w, k) for k in ks if launches[(w, k)]}
                            for w, ks in want.items() if w != "c4"}
    return out



def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=16384)
    ap.add_argument("--workload", default="c4", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--rows", type=int, default=0,
                    help="c1..c5: run the workload with this many rows instead (scaling checks)")
    ap.add_argument("--reduction", default="mean", choices=["mean", "sum", "none"])
    ap.add_argument("--grad-scale", type=float, default=None,
                    help="upstream gradient folded into the cross-entropy gradient write")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="the headline kernel's average from a rocprofv3 kernel trace")
    ap.add_argument("--no-extras", action="store_true",
                    help="default run: skip timing the other configurations after c4")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the memory-ceiling probes timed beside each kernel")
    args = ap.parse_args()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(*args.summarize_counters, workload=args.workload),
                         indent=1))
        return 0
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace, args.steps), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (--gpus {args.gpus} "
              "requested).", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.steps + args.warmup > 40:
        print("need 1 <= steps and steps + warmup <= 40 (one copy of the logits per step)",
              file=sys.stderr)
        return 2
    args.ceiling = args.workload != "c1" and not (args.no_ceiling or args.rows)
    if args.workload in ("c1", "c2", "sm-vocab", "sm-few"):
        out = run_softmax(args, args.workload)
    elif args.workload == "c4-mul":
        out = run_element_mul(args, args.workload)
    elif args.workload == "c4-nll":
        out = run_nll(args, args.workload)
    elif args.workload == "ln":
        out = run_layernorm(args, args.workload)
    elif args.workload == "bsr":
        out = run_bsr(args, args.workload)
    else:
        out = run_xent(args, args.workload)
        if args.workload == "c4" and not (args.no_extras or args.rows or args.grad_scale is not None
                                          or args.reduction != "mean"):
            out["other_configs"] = run_extras(args)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
