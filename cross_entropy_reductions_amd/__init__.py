"""Row softmax, softmax backward and fused cross-entropy on AMD MI355X (gfx950).

A thin ctypes binding over ``libxr.so`` (``include/xr.h``): every function here
checks and marshals its torch tensors into the C ABI call of the same name
(``softmax_fwd`` -> ``xr_softmax_fwd_ex``, ``softmax_bwd`` -> ``xr_softmax_bwd_ex``,
``nll_fwd`` -> ``xr_nll_fwd``,
``xent_fwd_bwd`` -> ``xr_xent_fwd_bwd_ex``, ``element_mul`` -> ``xr_element_mul``, ...).
All of the computation runs in the library's HIP kernels; PyTorch only provides device
memory and the current stream. ``CrossEntropyFunction`` / ``cross_entropy`` wrap the
fused cross-entropy as a ``torch.autograd.Function`` the way the Liger-Kernel
``cross_entropy.py`` page's ``LigerCrossEntropyFunction`` does: the forward leaves the
gradient in the logits' memory, the backward scales it by the upstream gradient.

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
lib.xr_softmax_workspace_bytes.argtypes = [_i64, _i64, ctypes.c_int]
lib.xr_softmax_workspace_bytes.restype = _sz
lib.xr_softmax_fwd_ex.argtypes = [_p, _i64, _p, _i64, _i64, _i64, ctypes.c_int, _p, _sz, _p]
lib.xr_softmax_fwd_ex.restype = ctypes.c_int
lib.xr_softmax_bwd_ex.argtypes = [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, ctypes.c_int, _p,
                                  _sz, _p]
lib.xr_softmax_bwd_ex.restype = ctypes.c_int
lib.xr_nll_fwd.argtypes = [_p, _i64, _p, _i64, _p, _p, _i64, _i64, ctypes.c_int, _p, _sz, _p]
lib.xr_nll_fwd_workspace_bytes.argtypes = [_i64, _i64, ctypes.c_int]
lib.xr_nll_fwd_workspace_bytes.restype = _sz
lib.xr_nll_fwd.restype = ctypes.c_int
lib.xr_bsr_softmax_bwd.argtypes = [_p, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _i32,
                                   ctypes.c_float, ctypes.c_int, _p]
lib.xr_bsr_softmax_bwd.restype = ctypes.c_int
lib.xr_layernorm_fwd.argtypes = [_p, _i64, _p, _i64, _p, _p, _p, _p, _i64, _i64, ctypes.c_float,
                                 ctypes.c_int, _p]
lib.xr_layernorm_fwd.restype = ctypes.c_int
lib.xr_layernorm_bwd_workspace_bytes.argtypes = [_i64, _i64, ctypes.c_int]
lib.xr_layernorm_bwd_workspace_bytes.restype = _sz
lib.xr_layernorm_bwd.argtypes = [_p, _i64, _p, _i64, _p, _i64, _p, _p, _p, _p, _p, _i64, _i64,
                                 ctypes.c_int, _p, _sz, _p]
lib.xr_layernorm_bwd.restype = ctypes.c_int
lib.xr_xent_workspace_bytes.argtypes = [_i64, _i64, ctypes.c_int]
lib.xr_xent_workspace_bytes.restype = _sz
lib.xr_xent_fwd_bwd.argtypes = [_p, _i64, _p, _i64, _i64, _i64, ctypes.c_int, _p, _p, _p, _p,
                                _sz, _p]
lib.xr_xent_fwd_bwd.restype = ctypes.c_int
lib.xr_xent_fwd_bwd_ex.argtypes = [_p, _i64, _p, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                   _p, _i64, _p, _p, _p, _p, _sz, _p]
lib.xr_xent_fwd_bwd_ex.restype = ctypes.c_int
lib.xr_element_mul.argtypes = [_p, _i64, _i64, _i64, ctypes.c_int, _p, _i64, _p]
lib.xr_element_mul.restype = ctypes.c_int
lib.xr_xent_fwd_bwd_noalloc.argtypes = [_p, _i64, _p, _i64, _i64, _i64, ctypes.c_int,
                                        ctypes.c_int, _p, _i64, _p, _p, _p, _p]
lib.xr_xent_fwd_bwd_noalloc.restype = ctypes.c_int
lib.xr_probe_rows.argtypes = [_p, _i64, _p, _p, _i64, _i64, _i64, ctypes.c_int, _i32, _i32, _i32,
                              _p, _i64, _p]
lib.xr_probe_rows.restype = ctypes.c_int
lib.xr_probe_copy.argtypes = [_p, _p, _p, _i64, _i32, _i32, _p]
lib.xr_probe_copy.restype = ctypes.c_int
lib.xr_workspace_status.argtypes = [_p, _sz, _p, _p]
lib.xr_workspace_status.restype = ctypes.c_int
lib.xr_status_string.argtypes = [ctypes.c_int]
lib.xr_status_string.restype = ctypes.c_char_p
lib.xr_version.argtypes = []
lib.xr_version.restype = _i32


class XrPlan(ctypes.Structure):
    _fields_ = [("path", _i32), ("threads", _i32), ("vec_per_thread", _i32), ("split", _i32),
                ("grid", _i32), ("cooperative", _i32), ("chunk_vecs", _i64),
                ("group_rows", _i32), ("load_priority", _i32), ("grid_total", _i64)]


lib.xr_plan.argtypes = [_i32, _i64, _i64, ctypes.c_int, _i32, ctypes.POINTER(XrPlan)]
lib.xr_plan.restype = ctypes.c_int
lib.xr_plan_model.argtypes = [_i32, _i64, _i64, ctypes.c_int, _i32, _i32, _i32,
                              ctypes.POINTER(XrPlan)]
lib.xr_plan_model.restype = ctypes.c_int
lib.xr_set_option.argtypes = [ctypes.c_int, _i64]
lib.xr_set_option.restype = ctypes.c_int
lib.xr_set_profile_events.argtypes = [_p, _p]
lib.xr_set_profile_events.restype = ctypes.c_int

# Names exported by include/xr.h (checked against the library by the tests).
C_SYMBOLS = ("xr_softmax_fwd", "xr_softmax_bwd", "xr_softmax_workspace_bytes",
             "xr_softmax_fwd_ex", "xr_softmax_bwd_ex", "xr_bsr_softmax_bwd", "xr_nll_fwd",
             "xr_nll_fwd_workspace_bytes",
             "xr_layernorm_fwd",
             "xr_layernorm_bwd_workspace_bytes", "xr_layernorm_bwd", "xr_xent_workspace_bytes",
             "xr_xent_fwd_bwd",
             "xr_xent_fwd_bwd_ex", "xr_xent_fwd_bwd_noalloc", "xr_element_mul",
             "xr_workspace_status", "xr_probe_rows", "xr_probe_copy",
             "xr_status_string", "xr_version", "xr_plan", "xr_plan_model", "xr_set_option",
             "xr_set_profile_events")

F32, BF16 = 0, 1
OK = 0
PATHS = {1: "resident", 2: "split", 3: "stream"}
OPS = {"softmax_fwd": 0, "softmax_bwd": 1, "xent": 2, "nll_fwd": 3, "softmax_fwd_ws": 4,
       "softmax_bwd_ws": 5}
OPTIONS = {"path": 1, "split": 2, "threads": 3, "grid": 4, "load_policy": 5, "no_wait": 6,
           "groups": 7}
REDUCTIONS = {"mean": 0, "sum": 1, "none": 2}

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


def softmax_workspace_bytes(M: int, N: int, dtype: torch.dtype) -> int:
    """Workspace bytes the softmax forward and backward need to split rows of this size."""
    return int(lib.xr_softmax_workspace_bytes(int(M), int(N), _DTYPES[dtype]))


def _softmax_ws(workspace, M: int, N: int, dt: int, dev):
    """(pointer, bytes) of a softmax workspace: a given tensor, a new one when None, or
    (None, 0) when False (rows handled whole)."""
    if workspace is False:
        return None, 0
    if workspace is None:
        need = int(lib.xr_softmax_workspace_bytes(M, N, dt)) if M > 0 else 0
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if not isinstance(workspace, torch.Tensor) or workspace.device != dev or \
            not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous tensor on the operands' device")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def softmax_fwd(x: torch.Tensor, out: torch.Tensor | None = None, *, workspace=None,
                stream=None) -> torch.Tensor:
    """Row softmax of x into ``out`` (a new tensor like x, or x itself for in place).
    ``workspace``: a device tensor of softmax_workspace_bytes() bytes, None to allocate one
    here, or False to keep every row in one workgroup (no split rows)."""
    px, ldx, M, N, dt = _matrix(x, "x")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    py, ldy, M2, N2, dt2 = _matrix(out, "out")
    if (M2, N2, dt2) != (M, N, dt) or out.device != x.device:
        raise ValueError("out must match x in shape, dtype and device")
    pw, nw = _softmax_ws(workspace, M, N, dt, x.device)
    _check("xr_softmax_fwd_ex", lib.xr_softmax_fwd_ex(py, ldy, px, ldx, M, N, dt, pw, nw,
                                                      _stream(x, stream)))
    return out


def softmax_bwd(y: torch.Tensor, dy: torch.Tensor, out: torch.Tensor | None = None, *,
                workspace=None, stream=None) -> torch.Tensor:
    """dx = y * (dy - sum(y * dy)) per row, into ``out`` (new, or exactly y or dy).
    ``workspace`` as for softmax_fwd."""
    py, ldy, M, N, dt = _matrix(y, "y")
    pd, ldd, M2, N2, dt2 = _matrix(dy, "dy")
    if (M2, N2, dt2) != (M, N, dt) or dy.device != y.device:
        raise ValueError("dy must match y in shape, dtype and device")
    if out is None:
        out = torch.empty_like(y, memory_format=torch.contiguous_format)
    px, ldx, M3, N3, dt3 = _matrix(out, "out")
    if (M3, N3, dt3) != (M, N, dt) or out.device != y.device:
        raise ValueError("out must match y in shape, dtype and device")
    pw, nw = _softmax_ws(workspace, M, N, dt, y.device)
    _check("xr_softmax_bwd_ex",
           lib.xr_softmax_bwd_ex(px, ldx, py, ldy, pd, ldd, M, N, dt, pw, nw, _stream(y, stream)))
    return out


class SoftmaxFunction(torch.autograd.Function):
    """Softmax over the last dimension as a torch.autograd.Function, the way the Triton
    fused-softmax kernels of the "python sum function examples" page pair a forward with
    the fused `_backward`: the forward saves y, the backward computes y * (dy - sum(y * dy))
    per row. Rows are split over workgroups through a workspace when that pays."""

    @staticmethod
    def forward(ctx, x):
        x2 = x.reshape(-1, x.shape[-1])
        if x2.shape[-1] > 1 and x2.stride(-1) != 1:
            x2 = x2.contiguous()
        y = softmax_fwd(x2)
        ctx.save_for_backward(y)
        return y.reshape(x.shape)

    @staticmethod
    def backward(ctx, dy):
        (y,) = ctx.saved_tensors
        dy2 = dy.reshape(-1, dy.shape[-1])
        if dy2.shape[-1] > 1 and dy2.stride(-1) != 1:
            dy2 = dy2.contiguous()
        return softmax_bwd(y, dy2).reshape(dy.shape)


def softmax(x: torch.Tensor) -> torch.Tensor:
    """Autograd-aware softmax over the last dimension (``SoftmaxFunction``)."""
    return SoftmaxFunction.apply(x)


def bsr_softmax_bwd(y: torch.Tensor, dx: torch.Tensor, lut: torch.Tensor, n_brows: int,
                    n_blocks: int, block: int, scale: float = 1.0, *, stream=None) -> torch.Tensor:
    """Block-sparse softmax backward in place: dx (Z, stride) holds the incoming gradient and
    receives y * (dx - sum(y * dx)) * scale along every table row (see xr_bsr_softmax_bwd
    in include/xr.h for the table layout). Returns dx."""
    for t, name in ((y, "y"), (dx, "dx")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != 2 or t.dtype not in _DTYPES:
            raise TypeError(f"{name} must be a 2-D float32 or bfloat16 device tensor (Z, stride)")
        if t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must have unit stride along its last dimension")
    if y.dtype != dx.dtype or y.device != dx.device or y.shape[0] != dx.shape[0]:
        raise ValueError("y and dx must share dtype, device and batch count")
    if not isinstance(lut, torch.Tensor) or lut.dtype != torch.int32 or lut.device != dx.device \
            or lut.dim() != 1 or not lut.is_contiguous():
        raise TypeError("lut must be a contiguous 1-D int32 tensor on dx's device")
    per = int(n_blocks) * int(block) * int(block)
    if y.shape[1] < per or dx.shape[1] < per:
        raise ValueError("y and dx rows must hold n_blocks * block^2 elements")
    Z = dx.shape[0]
    sy = y.stride(0) if Z > 1 else y.shape[1]
    sd = dx.stride(0) if Z > 1 else dx.shape[1]
    _check("xr_bsr_softmax_bwd",
           lib.xr_bsr_softmax_bwd(y.data_ptr(), sy, dx.data_ptr(), sd, Z, lut.data_ptr(),
                                  lut.numel(), int(n_brows), int(n_blocks), int(block),
                                  float(scale), _DTYPES[dx.dtype], _stream(dx, stream)))
    return dx


def nll_fwd(x: torch.Tensor, idx: torch.Tensor, out: torch.Tensor | None = None,
            loss: torch.Tensor | None = None, *, workspace: torch.Tensor | None = None,
            stream=None):
    """-log softmax of each row of x into ``out`` (new, or x itself), and the fp32 loss
    ``out[i, idx[i]]`` as stored (NaN for an index outside the row). Returns (out, loss).
    A workspace (allocated here when not given) lets long rows be split over workgroups."""
    px, ldx, M, N, dt = _matrix(x, "x")
    if not isinstance(idx, torch.Tensor) or idx.dtype != torch.int64 or idx.device != x.device:
        raise TypeError("idx must be an int64 tensor on x's device")
    if idx.dim() != 1 or idx.shape[0] != M or (M > 1 and idx.stride(0) != 1):
        raise ValueError("idx must be a contiguous 1-D tensor of one entry per row")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    po, ldo, M2, N2, dt2 = _matrix(out, "out")
    if (M2, N2, dt2) != (M, N, dt) or out.device != x.device:
        raise ValueError("out must match x in shape, dtype and device")
    if loss is None:
        loss = torch.empty(M, dtype=torch.float32, device=x.device)
    if loss.dtype != torch.float32 or loss.device != x.device or loss.numel() < M or \
            not loss.is_contiguous():
        raise ValueError("loss must be a contiguous float32 tensor of one entry per row")
    if workspace is None:
        need = int(lib.xr_nll_fwd_workspace_bytes(M, N, dt)) if M > 0 else 0
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check("xr_nll_fwd", lib.xr_nll_fwd(po, ldo, px, ldx, idx.data_ptr(), loss.data_ptr(), M, N,
                                        dt, workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(x, stream)))
    return out, loss


def _vector(t: torch.Tensor, name: str, N: int, dt: int, dev) -> int:
    if not isinstance(t, torch.Tensor) or t.device != dev or _DTYPES.get(t.dtype) != dt:
        raise TypeError(f"{name} must be a tensor of the input's dtype on its device")
    if t.dim() != 1 or t.shape[0] != N or (N > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous 1-D tensor of N entries")
    return t.data_ptr()


def layernorm_fwd(x: torch.Tensor, w: torch.Tensor, b: torch.Tensor, eps: float = 1e-5,
                  out: torch.Tensor | None = None, mean: torch.Tensor | None = None,
                  rstd: torch.Tensor | None = None, *, stream=None):
    """Layer norm of each row of x: returns (y, mean, rstd); y may be x itself."""
    px, ldx, M, N, dt = _matrix(x, "x")
    pw = _vector(w, "w", N, dt, x.device)
    pb = _vector(b, "b", N, dt, x.device)
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    py, ldy, M2, N2, dt2 = _matrix(out, "out")
    if (M2, N2, dt2) != (M, N, dt) or out.device != x.device:
        raise ValueError("out must match x in shape, dtype and device")
    if mean is None:
        mean = torch.empty(M, dtype=torch.float32, device=x.device)
    if rstd is None:
        rstd = torch.empty(M, dtype=torch.float32, device=x.device)
    for t, name in ((mean, "mean"), (rstd, "rstd")):
        if t.dtype != torch.float32 or t.device != x.device or t.numel() < M or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of one entry per row")
    _check("xr_layernorm_fwd",
           lib.xr_layernorm_fwd(py, ldy, px, ldx, pw, pb, mean.data_ptr(), rstd.data_ptr(), M, N,
                                float(eps), dt, _stream(x, stream)))
    return out, mean, rstd


def layernorm_bwd_workspace_bytes(M: int, N: int, dtype: torch.dtype) -> int:
    return int(lib.xr_layernorm_bwd_workspace_bytes(int(M), int(N), _DTYPES[dtype]))


def layernorm_bwd(dy: torch.Tensor, x: torch.Tensor, w: torch.Tensor, mean: torch.Tensor,
                  rstd: torch.Tensor, dx: torch.Tensor | None = None,
                  dw: torch.Tensor | None = None, db: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, *, stream=None):
    """Layer norm backward: returns (dx, dw, db); dx may be dy or x itself."""
    pd, ldd, M, N, dt = _matrix(dy, "dy")
    px, ldx, M2, N2, dt2 = _matrix(x, "x")
    if (M2, N2, dt2) != (M, N, dt) or x.device != dy.device:
        raise ValueError("x must match dy in shape, dtype and device")
    pw = _vector(w, "w", N, dt, dy.device)
    for t, name in ((mean, "mean"), (rstd, "rstd")):
        if t.dtype != torch.float32 or t.device != dy.device or t.numel() < M or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of one entry per row")
    if dx is None:
        dx = torch.empty_like(dy, memory_format=torch.contiguous_format)
    pdx, lddx, M3, N3, dt3 = _matrix(dx, "dx")
    if (M3, N3, dt3) != (M, N, dt) or dx.device != dy.device:
        raise ValueError("dx must match dy in shape, dtype and device")
    if dw is None:
        dw = torch.empty(N, dtype=dy.dtype, device=dy.device)
    if db is None:
        db = torch.empty(N, dtype=dy.dtype, device=dy.device)
    pdw = _vector(dw, "dw", N, dt, dy.device)
    pdb = _vector(db, "db", N, dt, dy.device)
    need = layernorm_bwd_workspace_bytes(M, N, dy.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dy.device)
    _check("xr_layernorm_bwd",
           lib.xr_layernorm_bwd(pdx, lddx, pd, ldd, px, ldx, pw, mean.data_ptr(), rstd.data_ptr(),
                                pdw, pdb, M, N, dt, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream(dy, stream)))
    return dx, dw, db


class LayerNormFunction(torch.autograd.Function):
    """Layer norm over the last dimension as a torch.autograd.Function (the shape of the
    Triton LayerNorm tutorial's LayerNorm class): the forward saves x, w, mean and rstd;
    the backward runs the two-stage dw / db reduction."""

    @staticmethod
    def forward(ctx, x, normalized_shape, weight, bias, eps=1e-5):
        x2 = x.reshape(-1, x.shape[-1])
        y, mean, rstd = layernorm_fwd(x2, weight, bias, eps)
        ctx.save_for_backward(x2, weight, mean, rstd)
        return y.reshape(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, w, mean, rstd = ctx.saved_tensors
        dy2 = dy.reshape(-1, dy.shape[-1])
        if dy2.stride(-1) != 1:
            dy2 = dy2.contiguous()
        dx, dw, db = layernorm_bwd(dy2, x2, w, mean, rstd)
        return dx.reshape(dy.shape), None, dw, db, None


def layer_norm(x: torch.Tensor, weight: torch.Tensor, bias: torch.Tensor,
               eps: float = 1e-5) -> torch.Tensor:
    """Autograd-aware layer norm over the last dimension."""
    return LayerNormFunction.apply(x, (x.shape[-1],), weight, bias, eps)


def xent_workspace_bytes(M: int, V: int, dtype: torch.dtype) -> int:
    """Device workspace bytes xent_fwd_bwd needs (on the current device)."""
    return int(lib.xr_xent_workspace_bytes(int(M), int(V), _DTYPES[dtype]))


def _scale_arg(scale, M: int, dev, name: str):
    """(pointer, stride) of an upstream-gradient argument: None, a number, or a float32
    device tensor holding one value (any shape with one element) or one value per row."""
    if scale is None:
        return None, 0, None
    if not isinstance(scale, torch.Tensor):
        scale = torch.tensor([float(scale)], dtype=torch.float32, device=dev)
    if scale.dtype != torch.float32 or scale.device != dev:
        raise TypeError(f"{name} must be a float32 tensor on the logits' device")
    if scale.numel() == 1:
        return scale.data_ptr(), 0, scale
    if scale.dim() != 1 or scale.shape[0] != M:
        raise ValueError(f"{name} must hold one value, or one value per row")
    return scale.data_ptr(), scale.stride(0), scale


def xent_fwd_bwd(logits: torch.Tensor, target: torch.Tensor, ignore_index: int = -100, *,
                 reduction: str = "mean", grad_scale=None,
                 row_loss: torch.Tensor | None = None, mean_loss: torch.Tensor | None = None,
                 counts: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 stream=None):
    """Fused cross-entropy: overwrites ``logits`` with the gradient of the reduced loss.

    ``reduction`` is "mean" (the pages' kernel), "sum" or "none"; ``grad_scale`` is the
    upstream gradient folded into the gradient write (None for 1, a number, or a float32
    device tensor of one value or one value per row). Returns ``(loss, row_loss, counts)``:
    the reduced loss as a 1-element fp32 tensor (the row losses themselves for "none"),
    the fp32 row losses and int32 ``[n_non_ignore, n_bad_target, error_flags]``, all on the
    device (nothing is synchronised). ``row_loss=False`` (mean and sum only) keeps the row
    losses in the workspace instead; row_loss is then returned as None.
    """
    pl, ld, M, V, dt = _matrix(logits, "logits")
    dev = logits.device
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    if not isinstance(target, torch.Tensor) or target.dtype != torch.int64 or target.device != dev:
        raise TypeError("target must be an int64 tensor on the logits' device")
    if target.dim() != 1 or target.shape[0] != M or (M > 1 and target.stride(0) != 1):
        raise ValueError("target must be a contiguous 1-D tensor of one entry per row")
    if row_loss is False and reduction == "none":
        raise ValueError('the row losses are the result of reduction="none"')
    if row_loss is None:
        row_loss = torch.empty(M, dtype=torch.float32, device=dev)
    if mean_loss is None and reduction != "none":
        mean_loss = torch.empty(1, dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(3, dtype=torch.int32, device=dev)
    outs = [(counts, "counts", torch.int32, 3)]
    if row_loss is not False:
        outs.append((row_loss, "row_loss", torch.float32, M))
    if reduction != "none":
        outs.append((mean_loss, "mean_loss", torch.float32, 1))
    for t, name, dtp, n in outs:
        if t.dtype != dtp or t.device != dev or t.numel() < n or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtp} tensor of >= {n} entries")
    ps, sstride, _keep = _scale_arg(grad_scale, M, dev, "grad_scale")
    need = xent_workspace_bytes(M, V, logits.dtype) if M >= 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("xr_xent_fwd_bwd_ex",
           lib.xr_xent_fwd_bwd_ex(pl, ld, target.data_ptr(), M, V, int(ignore_index), dt,
                                  REDUCTIONS[reduction], ps, sstride,
                                  None if row_loss is False else row_loss.data_ptr(),
                                  None if reduction == "none" else mean_loss.data_ptr(),
                                  counts.data_ptr(), workspace.data_ptr(), ws_bytes,
                                  _stream(logits, stream)))
    if row_loss is False:
        row_loss = None
    return (row_loss if reduction == "none" else mean_loss), row_loss, counts


def probe_rows(out: torch.Tensor, in0: torch.Tensor, in1: torch.Tensor | None = None, *,
               threads: int, vpt: int, split: int, target: torch.Tensor | None = None,
               ignore_index: int = -100, stream=None) -> torch.Tensor:
    """The memory-ceiling probe (xr_probe_rows): the row kernels' loads and stores over these
    rows in the given launch shape, with none of their arithmetic. Returns out."""
    po, ldo, M, N, dt = _matrix(out, "out")
    p0, ld0, M0, N0, dt0 = _matrix(in0, "in0")
    if (M0, N0, dt0) != (M, N, dt):
        raise ValueError("in0 must match out in shape and dtype")
    p1 = None
    if in1 is not None:
        p1, ld1, M1, N1, dt1 = _matrix(in1, "in1")
        if (M1, N1, dt1, ld1) != (M, N, dt, ld0):
            raise ValueError("in1 must match in0 in shape, dtype and row stride")
    pt = None if target is None else target.data_ptr()
    _check("xr_probe_rows", lib.xr_probe_rows(po, ldo, p0, p1, ld0, M, N, dt, int(threads),
                                              int(vpt), int(split), pt, int(ignore_index),
                                              _stream(out, stream)))
    return out


def probe_copy(out: torch.Tensor, src: torch.Tensor, src1: torch.Tensor | None = None, *,
               workgroups: int, threads: int = 256, stream=None) -> torch.Tensor:
    """The copy ceiling (xr_probe_copy): src's bytes (src ^ src1's with a second input) into
    out, by a grid-stride kernel of ``workgroups`` workgroups of ``threads`` threads, or by
    the runtime's device-to-device copy when ``workgroups`` is 0. ``src`` being ``out`` (the
    same memory) is the kernel's stream in place, every vector read and written back. Returns
    out."""
    for t, name in ((out, "out"), (src, "src"), (src1, "src1")):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    for t in (out, src1):
        if t is not None and t.numel() * t.element_size() != nbytes:
            raise ValueError("out, src and src1 must hold the same number of bytes")
    _check("xr_probe_copy", lib.xr_probe_copy(out.data_ptr(), src.data_ptr(),
                                              None if src1 is None else src1.data_ptr(), nbytes,
                                              int(workgroups), int(threads),
                                              _stream(out, stream)))
    return out


def workspace_status(workspace: torch.Tensor, *, stream=None) -> torch.Tensor:
    """The status word the last call left in ``workspace`` (0, or bit 0 when a split row's
    exchange timed out), copied on the device into a new 1-element int32 tensor (nothing is
    synchronised)."""
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or \
            not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous device tensor")
    out = torch.empty(1, dtype=torch.int32, device=workspace.device)
    _check("xr_workspace_status",
           lib.xr_workspace_status(workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), out.data_ptr(),
                                   _stream(workspace, stream)))
    return out


def element_mul(x: torch.Tensor, grad_output, *, stream=None) -> torch.Tensor:
    """x[i, :] *= grad_output[i] in place (one value for all rows, or one per row; rows
    whose value is exactly 1.0 are left untouched without being read). Returns x."""
    px, ld, M, N, dt = _matrix(x, "x")
    pg, gstride, _keep = _scale_arg(grad_output, M, x.device, "grad_output")
    if pg is None:
        raise ValueError("grad_output is required")
    _check("xr_element_mul", lib.xr_element_mul(px, ld, M, N, dt, pg, gstride, _stream(x, stream)))
    return x


class CrossEntropyFunction(torch.autograd.Function):
    """Cross-entropy whose forward computes the loss and, in the same pass, the gradient,
    stored in the logits' own memory (the logits are overwritten); the backward multiplies
    that stored gradient by the upstream gradient (``element_mul``; skipped on the device
    for rows whose upstream value is exactly 1.0). As on the Liger-Kernel page, the logits
    tensor passed in must not be needed afterwards by anything else. The forward returns
    the loss and the call's int32 counts ``[n_non_ignore, n_bad_target, error_flags]`` (on
    the device, not differentiable)."""

    @staticmethod
    def forward(ctx, logits, target, ignore_index=-100, reduction="mean"):
        loss, _, counts = xent_fwd_bwd(logits, target, ignore_index, reduction=reduction)
        ctx.reduction = reduction
        ctx.save_for_backward(logits.detach())
        ctx.mark_non_differentiable(counts)
        return (loss.reshape(()) if reduction != "none" else loss), counts

    @staticmethod
    def backward(ctx, grad_output, _grad_counts=None):
        (grad,) = ctx.saved_tensors
        g = grad_output
        if g.dtype != torch.float32:
            g = g.float()
        if g.dim() > 1 or (g.dim() == 1 and g.shape[0] != grad.shape[0]):
            raise ValueError("unexpected upstream gradient shape")
        element_mul(grad, g.reshape(-1) if g.dim() == 0 else g)
        return grad, None, None, None


def cross_entropy(logits: torch.Tensor, target: torch.Tensor, ignore_index: int = -100,
                  reduction: str = "mean", return_counts: bool = False):
    """Autograd-aware fused cross-entropy (``CrossEntropyFunction``); logits are consumed.
    With ``return_counts``, also the int32 device tensor ``[n_non_ignore, n_bad_target,
    error_flags]`` (bit 0 of error_flags: a split row's exchange timed out), read without a
    host synchronisation."""
    loss, counts = CrossEntropyFunction.apply(logits, target, ignore_index, reduction)
    return (loss, counts) if return_counts else loss


def plan(op: str, M: int, N: int, dtype: torch.dtype, aligned: int = 2) -> dict:
    """How the library carries out a call of these sizes on the current device.

    aligned: 2 = rows start on 16-byte boundaries (contiguous tensors), 1 = operands share
    their row alignment, 0 = they do not (see xr_plan in include/xr.h)."""
    out = XrPlan()
    _check("xr_plan", lib.xr_plan(OPS[op], int(M), int(N), _DTYPES[dtype], int(aligned),
                                  ctypes.byref(out)))
    return _plan_dict(out)


def _plan_dict(out: XrPlan) -> dict:
    return {"path": PATHS.get(out.path, str(out.path)), "threads": out.threads,
            "vec_per_thread": out.vec_per_thread, "split": out.split, "grid": out.grid,
            "cooperative": bool(out.cooperative), "chunk_vecs": out.chunk_vecs,
            "group_rows": out.group_rows, "load_priority": bool(out.load_priority),
            "grid_total": out.grid_total}


def plan_model(op: str, M: int, N: int, dtype: torch.dtype, compute_units: int,
               blocks_per_cu: int, aligned: int = 2) -> dict:
    """plan() for a modelled device (no GPU needed): compute_units compute units holding
    blocks_per_cu workgroups of the planned shape each (see xr_plan_model in include/xr.h)."""
    out = XrPlan()
    _check("xr_plan_model", lib.xr_plan_model(OPS[op], int(M), int(N), _DTYPES[dtype],
                                              int(aligned), int(compute_units),
                                              int(blocks_per_cu), ctypes.byref(out)))
    return _plan_dict(out)


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
