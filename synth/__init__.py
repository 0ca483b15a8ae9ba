"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out in memory. It holds
none of the softmax / cross-entropy arithmetic: neither the oracle nor the GPU
library imports anything from it, and it imports neither of them.

Every workload is drawn with numpy's PCG64 in a fixed order. Matrices are drawn
in 1024-row chunks; chunk ``c`` of a workload seeded ``seed`` has its own
generator ``PCG64(SeedSequence([seed, c]))``, so chunks can be drawn on several
host threads and still give the same bytes. Everything else (targets, ignored
rows, special rows) comes from ``PCG64(seed)`` after the matrix. Float draws are
float32 ``standard_normal`` values scaled in float32; bf16 matrices are the
round-to-nearest-even bf16 of those float32 values, held as ``uint16`` bit
patterns. The oracle and the GPU receive the same bytes.

Workloads (the shapes of the softmax / fused cross-entropy benchmarks):

====  =====================================================================
c1    softmax forward fp32, 128 x 1000, x = 3 N(0,1), contiguous
c2    softmax forward + backward bf16, 4096 x 4096, x = N(0,1), dy = N(0,1)
c3    fused cross-entropy bf16, 8192 x 32000 (B=4, T=2048), x = 2 N(0,1),
      int64 targets uniform in [0, V), floor(10 % M) rows set to -100
c4    fused cross-entropy bf16, 16384 x 128256, x = N(0,1) plus +20 at 4
      distinct uniform columns per row, targets uniform, floor(5 % M) ignored
c5    fused cross-entropy fp32, 2048 x 256000 in a row pitch of 256064 whose
      padding holds quiet NaN (0x7FC00000), x = 8 N(0,1); floor(1 % M) rows are
      all-equal (a constant 8 N(0,1) draw), floor(1 % M) rows have half their
      entries at -inf with a finite target; no ignored rows
====  =====================================================================
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

IGNORE_INDEX = -100
CHUNK_ROWS = 1024
NAN_PAD_BITS = np.uint32(0x7FC00000)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); NaN stays a quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16))
    r = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _chunk_rng(seed: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, chunk])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux hosts
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_chunks(out: np.ndarray, ncols: int, seed: int, make_chunk) -> None:
    """out[r0:r1, :ncols] = make_chunk(chunk_rng, rows) for every 1024-row chunk, in parallel."""
    M = out.shape[0]
    starts = list(range(0, M, CHUNK_ROWS))

    def work(ci: int) -> None:
        r0 = starts[ci]
        r1 = min(M, r0 + CHUNK_ROWS)
        out[r0:r1, :ncols] = make_chunk(_chunk_rng(seed, ci), r1 - r0)

    if len(starts) == 1:
        work(0)
        return
    with ThreadPoolExecutor(max_workers=_threads()) as pool:
        list(pool.map(work, range(len(starts))))


def _ignored_rows(rng: np.random.Generator, M: int, frac: float) -> np.ndarray:
    k = int(np.floor(frac * M))
    return rng.permutation(M)[:k]


def softmax_c1(M: int = 128, N: int = 1000, seed: int = 1001) -> dict:
    """c1: fp32 softmax forward input, x = 3 N(0,1), contiguous rows."""
    x = np.empty((M, N), dtype=np.float32)
    _fill_chunks(x, N, seed, lambda rng, rows: _normal(rng, (rows, N), 3.0))
    return {"name": "c1", "op": "softmax_fwd", "dtype": "f32", "M": M, "N": N, "x": x}


def softmax_c2(M: int = 4096, N: int = 4096, seed: int = 1002) -> dict:
    """c2: bf16 softmax forward + backward inputs, x and dy = N(0,1) (dy uses seed + 100)."""
    x = np.empty((M, N), dtype=np.uint16)
    dy = np.empty((M, N), dtype=np.uint16)
    _fill_chunks(x, N, seed, lambda rng, rows: bf16_bits_from_f32(_normal(rng, (rows, N), 1.0)))
    _fill_chunks(dy, N, seed + 100,
                 lambda rng, rows: bf16_bits_from_f32(_normal(rng, (rows, N), 1.0)))
    return {"name": "c2", "op": "softmax_fwd_bwd", "dtype": "bf16", "M": M, "N": N, "x": x,
            "dy": dy}


def softmax_long(M: int = 4096, N: int = 128256, dtype: str = "bf16", seed: int = 1008,
                 name: str = "sm-vocab") -> dict:
    """Softmax forward + backward over long rows: x and dy = N(0,1) (dy uses seed + 100), in
    bf16 (bit patterns) or fp32. Defaults: 4096 rows as wide as a 128256-entry vocabulary."""
    conv = bf16_bits_from_f32 if dtype == "bf16" else (lambda a: a)
    et = np.uint16 if dtype == "bf16" else np.float32
    x = np.empty((M, N), dtype=et)
    dy = np.empty((M, N), dtype=et)
    _fill_chunks(x, N, seed, lambda rng, rows: conv(_normal(rng, (rows, N), 1.0)))
    _fill_chunks(dy, N, seed + 100, lambda rng, rows: conv(_normal(rng, (rows, N), 1.0)))
    return {"name": name, "op": "softmax_fwd_bwd", "dtype": dtype, "M": M, "N": N, "x": x,
            "dy": dy}


def softmax_few(M: int = 16, N: int = 1 << 20, seed: int = 1009) -> dict:
    """Softmax forward + backward with too few rows to fill the GPU one row per workgroup:
    16 fp32 rows of 2^20 entries, x and dy = N(0,1)."""
    return softmax_long(M, N, "f32", seed, "sm-few")


def xent_c3(M: int = 8192, V: int = 32000, seed: int = 1003) -> dict:
    """c3: bf16 logits 2 N(0,1), uniform int64 targets, floor(10 % M) rows ignored."""
    x = np.empty((M, V), dtype=np.uint16)
    _fill_chunks(x, V, seed, lambda rng, rows: bf16_bits_from_f32(_normal(rng, (rows, V), 2.0)))
    rng = np.random.Generator(np.random.PCG64(seed))
    t = rng.integers(0, V, M, dtype=np.int64)
    t[_ignored_rows(rng, M, 0.10)] = IGNORE_INDEX
    return {"name": "c3", "op": "xent", "dtype": "bf16", "M": M, "N": V, "x": x, "target": t,
            "ignore_index": IGNORE_INDEX}


def xent_c4(M: int = 16384, V: int = 128256, seed: int = 1004, spikes: int = 4,
            spike: float = 20.0) -> dict:
    """c4: bf16 logits N(0,1) + spikes of +20 at 4 distinct columns per row, 5 % ignored.

    Within a chunk the normals are drawn first, then each row's spike columns
    (``choice(V, 4, replace=False)``) in row order; the spikes are added in
    float32 before the single rounding to bf16.
    """
    def chunk(rng, rows):
        blk = _normal(rng, (rows, V), 1.0)
        for r in range(rows):
            blk[r, rng.choice(V, spikes, replace=False)] += np.float32(spike)
        return bf16_bits_from_f32(blk)

    x = np.empty((M, V), dtype=np.uint16)
    _fill_chunks(x, V, seed, chunk)
    rng = np.random.Generator(np.random.PCG64(seed))
    t = rng.integers(0, V, M, dtype=np.int64)
    t[_ignored_rows(rng, M, 0.05)] = IGNORE_INDEX
    return {"name": "c4", "op": "xent", "dtype": "bf16", "M": M, "N": V, "x": x, "target": t,
            "ignore_index": IGNORE_INDEX}


def xent_c5(M: int = 2048, V: int = 256000, pad: int = 64, seed: int = 1005) -> dict:
    """c5: fp32 logits 8 N(0,1) in a NaN-padded pitch of V+64, special rows, no ignores."""
    ld = V + pad
    x = np.empty((M, ld), dtype=np.float32)
    x[:, V:].view(np.uint32)[...] = NAN_PAD_BITS
    _fill_chunks(x, V, seed, lambda rng, rows: _normal(rng, (rows, V), 8.0))
    rng = np.random.Generator(np.random.PCG64(seed))
    t = rng.integers(0, V, M, dtype=np.int64)
    k = int(np.floor(0.01 * M))
    sp = rng.permutation(M)[:2 * k]
    equal_rows, half_inf_rows = sp[:k], sp[k:2 * k]
    for r in equal_rows:
        x[r, :V] = np.float32(8.0) * rng.standard_normal(dtype=np.float32)
    for r in half_inf_rows:
        cols = rng.permutation(V)[: V // 2]
        x[r, cols] = -np.inf
        if not np.isfinite(x[r, t[r]]):
            finite = np.flatnonzero(np.isfinite(x[r, :V]))
            t[r] = finite[rng.integers(0, finite.shape[0])]
    return {"name": "c5", "op": "xent", "dtype": "f32", "M": M, "N": V, "ld": ld, "x": x,
            "target": t, "ignore_index": IGNORE_INDEX, "equal_rows": np.sort(equal_rows),
            "half_inf_rows": np.sort(half_inf_rows)}


def layernorm_ln(M: int = 16384, N: int = 8192, seed: int = 1006, dtype: str = "bf16") -> dict:
    """Layer norm forward + backward inputs: token rows of an 8192-wide hidden state.

    x = 2 N(0,1) + a per-row offset N(0,1) (rows do not have mean 0), w = 1 + 0.1 N(0,1),
    b = 0.1 N(0,1), dy = N(0,1) (seed + 100), eps = 1e-5."""
    shape_dt = np.uint16 if dtype == "bf16" else np.float32
    conv = bf16_bits_from_f32 if dtype == "bf16" else (lambda a: a)

    def rows_x(rng, rows):
        a = _normal(rng, (rows, N), 2.0)
        a += _normal(rng, (rows, 1), 1.0)
        return conv(a)

    x = np.empty((M, N), dtype=shape_dt)
    dy = np.empty((M, N), dtype=shape_dt)
    _fill_chunks(x, N, seed, rows_x)
    _fill_chunks(dy, N, seed + 100, lambda rng, rows: conv(_normal(rng, (rows, N), 1.0)))
    rng = np.random.Generator(np.random.PCG64(seed + 200))
    w = conv(1.0 + _normal(rng, (N,), 0.1))
    b = conv(_normal(rng, (N,), 0.1))
    return {"op": "layernorm", "M": M, "N": N, "dtype": dtype, "x": x, "dy": dy, "w": w, "b": b,
            "eps": 1e-5, "seed": seed}


def bsr_layout(n_brows: int, local: int, stride: int) -> dict:
    """A causal block-sparse layout and its look-up table.

    Block (r, c) is present when c <= r and either r - c < local (a local window) or
    c % stride == stride - 1 (global columns). Present blocks are numbered in row-major
    order: that number is the block's index in the block storage. The table holds two
    words (size, offset) per block-row, then four words per present block at word
    `offset + 4 k`: (block index, block-row, block-column, 0); the backward reads the first."""
    layout = np.zeros((n_brows, n_brows), dtype=bool)
    for r in range(n_brows):
        for c in range(r + 1):
            layout[r, c] = (r - c < local) or (c % stride == stride - 1)
    rows, cols = np.nonzero(layout)
    n_blocks = rows.size
    lut = np.zeros(2 * n_brows + 4 * n_blocks, dtype=np.int32)
    k = 0
    for r in range(n_brows):
        cs = np.flatnonzero(layout[r])
        lut[2 * r] = cs.size
        lut[2 * r + 1] = 2 * n_brows + 4 * k
        for c in cs:
            lut[2 * n_brows + 4 * k: 2 * n_brows + 4 * k + 4] = (k, r, c, 0)
            k += 1
    return {"layout": layout, "lut": lut, "n_blocks": int(n_blocks), "n_brows": n_brows}


def bsr_softmax(Z: int = 32, seq: int = 4096, block: int = 64, local: int = 4, stride: int = 8,
                seed: int = 1007, dtype: str = "bf16") -> dict:
    """Block-sparse softmax backward inputs: Z = batch x heads attention maps of seq x seq in
    block x block blocks under bsr_layout(seq / block, local, stride). y is positive with
    mean 1/(row length) (a softmax output's scale), dy = N(0,1) (seed + 100)."""
    lay = bsr_layout(seq // block, local, stride)
    per_z = lay["n_blocks"] * block * block
    mean_len = float(lay["layout"].sum(axis=1).mean() * block)
    shape_dt = np.uint16 if dtype == "bf16" else np.float32
    conv = bf16_bits_from_f32 if dtype == "bf16" else (lambda a: a)
    y = np.empty((Z, per_z), dtype=shape_dt)
    dy = np.empty((Z, per_z), dtype=shape_dt)
    for z in range(Z):
        rng = _chunk_rng(seed, z)
        y[z] = conv(rng.random(per_z, dtype=np.float32) * np.float32(2.0 / mean_len))
        dy[z] = conv(_normal(_chunk_rng(seed + 100, z), (per_z,), 1.0))
    return {"op": "bsr_softmax_bwd", "Z": Z, "seq": seq, "block": block, "y": y, "dy": dy,
            "scale": 0.125, "dtype": dtype, **lay}


WORKLOADS = {"c1": softmax_c1, "c2": softmax_c2, "c3": xent_c3, "c4": xent_c4, "c5": xent_c5,
             "sm-vocab": softmax_long, "sm-few": softmax_few}


def random_rows(seed: int, M: int, N: int, ld: int | None = None, dtype: str = "f32",
                scale: float = 1.0, pad_nan: bool = True) -> np.ndarray:
    """A generic (M, ld) matrix of scale*N(0,1) rows; padding columns hold quiet NaN."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ld = N if ld is None else ld
    vals = _normal(rng, (M, N), scale)
    if dtype == "bf16":
        out = np.empty((M, ld), dtype=np.uint16)
        out[:, N:] = np.uint16(0x7FC0) if pad_nan else 0
        out[:, :N] = bf16_bits_from_f32(vals)
    elif dtype == "f32":
        out = np.empty((M, ld), dtype=np.float32)
        out[:, N:].view(np.uint32)[...] = NAN_PAD_BITS if pad_nan else 0
        out[:, :N] = vals
    else:
        raise ValueError(dtype)
    return out


def random_targets(seed: int, M: int, V: int, ignore_frac: float = 0.0,
                   ignore_index: int = IGNORE_INDEX) -> np.ndarray:
    """Uniform int64 targets in [0, V) with floor(ignore_frac * M) rows set to ignore_index."""
    rng = np.random.Generator(np.random.PCG64(seed))
    t = rng.integers(0, V, M, dtype=np.int64)
    t[_ignored_rows(rng, M, ignore_frac)] = ignore_index
    return t
