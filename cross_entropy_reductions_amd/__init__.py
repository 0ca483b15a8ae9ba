"""Row softmax, softmax backward and fused cross-entropy on AMD MI355X (gfx950).

A thin ctypes binding over ``libxr.so`` (``include/xr.h``): every function here
checks and marshals its torch tensors into the C ABI call of the same name
(``softmax_fwd`` -> ``xr_softmax_fwd``, ``softmax_bwd`` -> ``xr_softmax_bwd``,
``xent_fwd_bwd`` -> ``xr_xent_fwd_bwd``, ...). All of the computation runs in the
library's HIP kernels; PyTorch only provides device memory and the current stream.

There is no fallback: importing this package raises if ``libxr.so`` has not been
built (``python cross_entropy_reductions_amd/build.py``), and every call raises on a
non-OK status.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libxr.so")

if not os.path.exists(LIBRARY):
    raise ImportError(
        f"{LIBRARY} is missing: build it with `python cross_entropy_reductions_amd/build.py`")

lib = ctypes.CDLL(LIBRARY)

_i64, _i32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t

lib.xr_softmax_fwd.argtypes = [_p, _i64, _p, _i64, _i64, _i64, ctypes.c_int, _p]
lib.xr_softmax_fwd.restype = ctypes.c_int
lib.xr_softmax_bwd.argtypes = [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, ctypes.c_int, _p]
lib.xr_softmax_bwd.restype = ctypes.c_int
lib.xr_xent_workspace_bytes.argtypes = [_i64, _i64, ctypes.c_int]
lib.xr_xent_workspace_bytes.restype = _sz
lib.xr_xent_fwd_bwd.argtypes = [_p, _i64, _p, _i64, _i64, _i64, ctypes.c_int, _p, _p, _p, _p,
                                _sz, _p]
lib.xr_xent_fwd_bwd.restype = ctypes.c_int
lib.xr_status_string.argtypes = [ctypes.c_int]
lib.xr_status_string.restype = ctypes.c_char_p
lib.xr_version.argtypes = []
lib.xr_version.restype = _i32


class XrPlan(ctypes.Structure):
    _fields_ = [("path", _i32), ("threads", _i32), ("vec_per_thread", _i32), ("split", _i32),
                ("grid", _i32), ("cooperative", _i32), ("chunk_vecs", _i64)]


lib.xr_plan.argtypes = [_i32, _i64, _i64, ctypes.c_int, _i32, ctypes.POINTER(XrPlan)]
lib.xr_plan.restype = ctypes.c_int
lib.xr_set_option.argtypes = [ctypes.c_int, _i64]
lib.xr_set_option.restype = ctypes.c_int
lib.xr_set_profile_events.argtypes = [_p, _p]
lib.xr_set_profile_events.restype = ctypes.c_int

# Names exported by include/xr.h (checked against the library by the tests).
C_SYMBOLS = ("xr_softmax_fwd", "xr_softmax_bwd", "xr_xent_workspace_bytes", "xr_xent_fwd_bwd",
             "xr_status_string", "xr_version", "xr_plan", "xr_set_option",
             "xr_set_profile_events")

F32, BF16 = 0, 1
OK = 0
PATHS = {1: "resident", 2: "split", 3: "stream"}
OPS = {"softmax_fwd": 0, "softmax_bwd": 1, "xent": 2}
OPTIONS = {"path": 1, "split": 2, "threads": 3, "grid": 4, "load_policy": 5}

_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


class XrError(RuntimeError):
    """A non-OK status from libxr."""

    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {status_string(status)} (status {status})")


def status_string(status: int) -> str:
    return lib.xr_status_string(int(status)).decode()


def version() -> int:
    return int(lib.xr_version())


def _check(func: str, status: int) -> None:
    if status != OK:
        raise XrError(func, status)


def _stream(t: torch.Tensor, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _matrix(t: torch.Tensor, name: str):
    """(pointer, row stride, rows, cols, dtype code) of a 2-D device matrix."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on a HIP device")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D (rows, columns)")
    if t.dtype not in _DTYPES:
        raise TypeError(f"{name}: dtype {t.dtype} is not supported (float32 or bfloat16)")
    M, N = t.shape
    if N > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    ld = t.stride(0) if M > 1 else max(N, 1)
    return t.data_ptr(), ld, M, N, _DTYPES[t.dtype]


def softmax_fwd(x: torch.Tensor, out: torch.Tensor | None = None, *, stream=None) -> torch.Tensor:
    """Row softmax of x into ``out`` (a new tensor like x, or x itself for in place)."""
    px, ldx, M, N, dt = _matrix(x, "x")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    py, ldy, M2, N2, dt2 = _matrix(out, "out")
    if (M2, N2, dt2) != (M, N, dt) or out.device != x.device:
        raise ValueError("out must match x in shape, dtype and device")
    _check("xr_softmax_fwd", lib.xr_softmax_fwd(py, ldy, px, ldx, M, N, dt, _stream(x, stream)))
    return out


def softmax_bwd(y: torch.Tensor, dy: torch.Tensor, out: torch.Tensor | None = None, *,
                stream=None) -> torch.Tensor:
    """dx = y * (dy - sum(y * dy)) per row, into ``out`` (new, or exactly y or dy)."""
    py, ldy, M, N, dt = _matrix(y, "y")
    pd, ldd, M2, N2, dt2 = _matrix(dy, "dy")
    if (M2, N2, dt2) != (M, N, dt) or dy.device != y.device:
        raise ValueError("dy must match y in shape, dtype and device")
    if out is None:
        out = torch.empty_like(y, memory_format=torch.contiguous_format)
    px, ldx, M3, N3, dt3 = _matrix(out, "out")
    if (M3, N3, dt3) != (M, N, dt) or out.device != y.device:
        raise ValueError("out must match y in shape, dtype and device")
    _check("xr_softmax_bwd",
           lib.xr_softmax_bwd(px, ldx, py, ldy, pd, ldd, M, N, dt, _stream(y, stream)))
    return out


def xent_workspace_bytes(M: int, V: int, dtype: torch.dtype) -> int:
    """Device workspace bytes xent_fwd_bwd needs (on the current device)."""
    return int(lib.xr_xent_workspace_bytes(int(M), int(V), _DTYPES[dtype]))


def xent_fwd_bwd(logits: torch.Tensor, target: torch.Tensor, ignore_index: int = -100, *,
                 row_loss: torch.Tensor | None = None, mean_loss: torch.Tensor | None = None,
                 counts: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None):
    """Fused cross-entropy: overwrites ``logits`` with the gradient of the mean loss.

    Returns ``(mean_loss, row_loss, counts)``: a 1-element fp32 tensor, the fp32 row
    losses and int32 ``[n_non_ignore, n_bad_target, error_flags]``, all on the device
    (nothing is synchronised).
    """
    pl, ld, M, V, dt = _matrix(logits, "logits")
    dev = logits.device
    if not isinstance(target, torch.Tensor) or target.dtype != torch.int64 or target.device != dev:
        raise TypeError("target must be an int64 tensor on the logits' device")
    if target.dim() != 1 or target.shape[0] != M or (M > 1 and target.stride(0) != 1):
        raise ValueError("target must be a contiguous 1-D tensor of one entry per row")
    if row_loss is None:
        row_loss = torch.empty(M, dtype=torch.float32, device=dev)
    if mean_loss is None:
        mean_loss = torch.empty(1, dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(3, dtype=torch.int32, device=dev)
    for t, name, dtp, n in ((row_loss, "row_loss", torch.float32, M),
                            (mean_loss, "mean_loss", torch.float32, 1),
                            (counts, "counts", torch.int32, 3)):
        if t.dtype != dtp or t.device != dev or t.numel() < n or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtp} tensor of >= {n} entries")
    need = xent_workspace_bytes(M, V, logits.dtype) if M >= 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("xr_xent_fwd_bwd",
           lib.xr_xent_fwd_bwd(pl, ld, target.data_ptr(), M, V, int(ignore_index), dt,
                               row_loss.data_ptr(), mean_loss.data_ptr(), counts.data_ptr(),
                               workspace.data_ptr(), ws_bytes, _stream(logits, stream)))
    return mean_loss, row_loss, counts


def plan(op: str, M: int, N: int, dtype: torch.dtype, aligned: int = 2) -> dict:
    """How the library carries out a call of these sizes on the current device.

    aligned: 2 = rows start on 16-byte boundaries (contiguous tensors), 1 = operands share
    their row alignment, 0 = they do not (see xr_plan in include/xr.h)."""
    out = XrPlan()
    _check("xr_plan", lib.xr_plan(OPS[op], int(M), int(N), _DTYPES[dtype], int(aligned),
                                  ctypes.byref(out)))
    return {"path": PATHS.get(out.path, str(out.path)), "threads": out.threads,
            "vec_per_thread": out.vec_per_thread, "split": out.split, "grid": out.grid,
            "cooperative": bool(out.cooperative), "chunk_vecs": out.chunk_vecs}


def set_option(name: str, value: int) -> None:
    """Process-wide override for tests and benchmarks (0 restores the automatic choice)."""
    _check("xr_set_option", lib.xr_set_option(OPTIONS[name], int(value)))


def set_profile_events(start, stop) -> None:
    """Record raw hipEvent_t handles (ints or None) around each call's row kernel."""
    _check("xr_set_profile_events",
           lib.xr_set_profile_events(None if start is None else ctypes.c_void_p(start),
                                     None if stop is None else ctypes.c_void_p(stop)))


def reset_options() -> None:
    for name in OPTIONS:
        set_option(name, 0)
