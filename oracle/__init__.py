"""Float64 CPU oracle for the row-softmax family (ctypes wrapper over xr_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package. The product path (``cross_entropy_reductions_amd``) never imports it
and shares no code with it.

What each function computes, and the passage it follows:

* ``softmax_fwd`` -- safe softmax of each row (page "python sum function
  examples", Triton kernels ``softmax_kernel`` / ``_softmax``).
* ``softmax_bwd`` -- ``dx = y * (dy - sum(y * dy))`` per row (same page,
  kernel ``_backward``, block-sparse scale taken as 1).
* ``bsr_softmax_bwd`` -- the block-sparse softmax backward of the same page's
  ``_backward`` kernel, rows gathered through its look-up table.
* ``nll_fwd`` -- negative log-softmax rows and the loss gathered at one index
  per row, as stored in the output type (same page, kernel ``_forward``).
* ``layernorm_fwd``, ``layernorm_bwd`` -- layer norm (the Triton LayerNorm
  tutorial page, from its prose and the paper it cites; its code is cut off):
  y = (x - mean) * rstd * w + b per row, and the derivative of that definition,
  dw and db summed over the rows.
* ``xent_count``, ``xent_rows``, ``mean``, ``xent`` -- Liger-Kernel
  ``cross_entropy.py``: ``liger_cross_entropy_kernel`` steps 1-6 (ignore
  early-out, loss ``m + log d - x_y``, gradient ``(softmax - onehot)/n``) and
  ``LigerCrossEntropyFunction.forward`` (``n`` counts non-ignored targets, mean
  loss ``sum(loss)/n``). ``reduction="sum"`` / ``"none"`` and the upstream
  gradient ``scale`` follow the definition of the loss that page links to
  (its kernel documents only the mean).
* ``element_mul`` -- the backward's ``element_mul`` kernel on the same page:
  every element of a stored gradient row times the upstream gradient.

Inputs are host numpy arrays holding exactly the bytes the GPU receives:
``uint16`` arrays carry bf16 bit patterns, ``float32`` arrays carry fp32.
A 2-D array of shape ``(M, ld)`` is read as M rows of row stride ``ld``, of
which the first ``N`` (or ``V``) columns are the row; the rest is padding that
is never read. Outputs are float64.

Every function here is pinned by ``tests/test_oracle_pins.py`` (invariants,
closed forms, finite differences, independent library routines) and the pins
are shown to catch planted mistakes by ``tests/test_oracle_mutants.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "xr_oracle.c")
LIBRARY = os.path.join(_HERE, "libxr_oracle.so")

F32, BF16 = 0, 1
REDUCTIONS = {"mean": 0, "sum": 1, "none": 2}

_c_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def compile_library(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc (C99, OpenMP, -O2, IEEE semantics kept)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


class Oracle:
    """One loaded copy of the oracle library (tests may load planted-mistake builds)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            compile_library(output=path)
        lib = ctypes.CDLL(path)
        lib.xro_softmax_fwd.argtypes = [_p, _c_i64, _c_i64, _c_i64, ctypes.c_int, _p]
        lib.xro_softmax_fwd.restype = None
        lib.xro_softmax_bwd.argtypes = [_p, _c_i64, _p, _c_i64, _c_i64, _c_i64, ctypes.c_int, _p]
        lib.xro_softmax_bwd.restype = None
        lib.xro_nll_fwd.argtypes = [_p, _c_i64, _p, _c_i64, _c_i64, ctypes.c_int, _p, _p]
        lib.xro_nll_fwd.restype = None
        lib.xro_bsr_softmax_bwd.argtypes = [_p, _p, _c_i64, _c_i64, _p, _c_i64, _c_i64,
                                            ctypes.c_double, ctypes.c_int, _p]
        lib.xro_bsr_softmax_bwd.restype = None
        lib.xro_layernorm_fwd.argtypes = [_p, _c_i64, _p, _p, _c_i64, _c_i64, ctypes.c_double,
                                          ctypes.c_int, _p, _p, _p]
        lib.xro_layernorm_fwd.restype = None
        lib.xro_layernorm_bwd.argtypes = [_p, _c_i64, _p, _c_i64, _p, _c_i64, _c_i64,
                                          ctypes.c_double, ctypes.c_int, _p, _p, _p]
        lib.xro_layernorm_bwd.restype = None
        lib.xro_xent_count.argtypes = [_p, _c_i64, _c_i64, _c_i64, _p]
        lib.xro_xent_count.restype = None
        lib.xro_xent_rows.argtypes = [_p, _c_i64, _p, _p, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                      _c_i64, _p, _p]
        lib.xro_xent_rows.restype = None
        lib.xro_xent_rows_ex.argtypes = [_p, _c_i64, _p, _p, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                         ctypes.c_int, _c_i64, _p, _c_i64, _p, _p]
        lib.xro_xent_rows_ex.restype = None
        lib.xro_sum.argtypes = [_p, _c_i64]
        lib.xro_sum.restype = ctypes.c_double
        lib.xro_element_mul.argtypes = [_p, _c_i64, _c_i64, _c_i64, ctypes.c_int, _p, _c_i64, _p]
        lib.xro_element_mul.restype = None
        lib.xro_mean.argtypes = [_p, _c_i64, _c_i64]
        lib.xro_mean.restype = ctypes.c_double
        lib.xro_num_threads.argtypes = []
        lib.xro_num_threads.restype = ctypes.c_int
        lib.xro_set_num_threads.argtypes = [ctypes.c_int]
        lib.xro_set_num_threads.restype = None
        self.lib = lib
        self.path = path

    # -- helpers -------------------------------------------------------------
    @staticmethod
    def _matrix(a: np.ndarray):
        """(pointer, row stride, rows, dtype code) of a 2-D uint16/float32 array."""
        if a.ndim != 2:
            raise ValueError("expected a 2-D array")
        if a.dtype == np.uint16:
            code = BF16
        elif a.dtype == np.float32:
            code = F32
        else:
            raise TypeError(f"unsupported dtype {a.dtype}: uint16 (bf16 bits) or float32")
        if a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
            raise ValueError("rows must be unit-stride in their last dimension")
        ld = a.strides[0] // a.itemsize
        return a.ctypes.data, ld, a.shape[0], code

    def num_threads(self) -> int:
        return int(self.lib.xro_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.xro_set_num_threads(int(n))

    # -- operations ----------------------------------------------------------
    def softmax_fwd(self, x: np.ndarray, n_cols: int | None = None) -> np.ndarray:
        ptr, ld, M, code = self._matrix(x)
        N = x.shape[1] if n_cols is None else int(n_cols)
        if not 0 < N <= x.shape[1]:
            raise ValueError("n_cols out of range")
        y = np.full((M, N), np.nan, dtype=np.float64)
        self.lib.xro_softmax_fwd(ptr, ld, M, N, code, y.ctypes.data)
        return y

    def softmax_bwd(self, y: np.ndarray, dy: np.ndarray, n_cols: int | None = None) -> np.ndarray:
        py, ldy, M, code = self._matrix(y)
        pd, ldd, M2, code2 = self._matrix(dy)
        if M != M2 or code != code2:
            raise ValueError("y and dy must have the same rows and dtype")
        N = y.shape[1] if n_cols is None else int(n_cols)
        if not 0 < N <= min(y.shape[1], dy.shape[1]):
            raise ValueError("n_cols out of range")
        dx = np.full((M, N), np.nan, dtype=np.float64)
        self.lib.xro_softmax_bwd(py, ldy, pd, ldd, M, N, code, dx.ctypes.data)
        return dx

    def nll_fwd(self, x: np.ndarray, idx: np.ndarray, n_cols: int | None = None):
        """(-log softmax rows [M, N] as float64, loss [M]: the output element at idx[i] rounded
        to x's type, NaN where idx[i] is outside [0, N))."""
        ptr, ld, M, code = self._matrix(x)
        N = x.shape[1] if n_cols is None else int(n_cols)
        if not 0 < N <= x.shape[1]:
            raise ValueError("n_cols out of range")
        ix = np.ascontiguousarray(idx, dtype=np.int64)
        if ix.shape != (M,):
            raise ValueError("idx must hold one index per row")
        # -1 is no value of -log p: an entry left unwritten fails every check of the output,
        # and a read past a row's end (another row's first entry, written or not) is never
        # the NaN that an index outside the row gives
        out = np.full((M, N), -1.0, dtype=np.float64)
        loss = np.full(M, np.nan, dtype=np.float64)
        self.lib.xro_nll_fwd(ptr, ld, ix.ctypes.data, M, N, code, out.ctypes.data,
                             loss.ctypes.data)
        return out, loss

    def _vector(self, a: np.ndarray, code: int, N: int, name: str) -> np.ndarray:
        a = np.ascontiguousarray(a)
        if a.ndim != 1 or a.shape[0] < N or (BF16 if a.dtype == np.uint16 else F32) != code or \
                a.dtype not in (np.uint16, np.float32):
            raise ValueError(f"{name} must be a 1-D array of >= N entries in x's type")
        return a

    def layernorm_fwd(self, x: np.ndarray, w: np.ndarray, b: np.ndarray, eps: float,
                      n_cols: int | None = None):
        """(y [M, N], mean [M], rstd [M]) as float64."""
        ptr, ld, M, code = self._matrix(x)
        N = x.shape[1] if n_cols is None else int(n_cols)
        if not 0 < N <= x.shape[1]:
            raise ValueError("n_cols out of range")
        w = self._vector(w, code, N, "w")
        b = self._vector(b, code, N, "b")
        y = np.full((M, N), np.nan, dtype=np.float64)
        mean = np.full(M, np.nan, dtype=np.float64)
        rstd = np.full(M, np.nan, dtype=np.float64)
        self.lib.xro_layernorm_fwd(ptr, ld, w.ctypes.data, b.ctypes.data, M, N, float(eps), code,
                                   y.ctypes.data, mean.ctypes.data, rstd.ctypes.data)
        return y, mean, rstd

    def layernorm_bwd(self, dy: np.ndarray, x: np.ndarray, w: np.ndarray, eps: float,
                      n_cols: int | None = None):
        """(dx [M, N], dw [N], db [N]) as float64."""
        pd, ldd, M, code = self._matrix(dy)
        px, ldx, M2, code2 = self._matrix(x)
        if M != M2 or code != code2:
            raise ValueError("dy and x must have the same rows and type")
        N = x.shape[1] if n_cols is None else int(n_cols)
        if not 0 < N <= min(x.shape[1], dy.shape[1]):
            raise ValueError("n_cols out of range")
        w = self._vector(w, code, N, "w")
        dx = np.full((M, N), np.nan, dtype=np.float64)
        dw = np.full(N, np.nan, dtype=np.float64)
        db = np.full(N, np.nan, dtype=np.float64)
        self.lib.xro_layernorm_bwd(pd, ldd, px, ldx, w.ctypes.data, M, N, float(eps), code,
                                   dx.ctypes.data, dw.ctypes.data, db.ctypes.data)
        return dx, dw, db

    def bsr_softmax_bwd(self, y: np.ndarray, dy: np.ndarray, lut: np.ndarray, n_brows: int,
                        block: int, scale: float = 1.0) -> np.ndarray:
        """y, dy: (Z, stride_z) arrays of blocks (uint16 bf16 bits or float32); lut: int32.
        Returns dy as float64 with the listed rows replaced by y * (dy - sum(y dy)) * scale."""
        py, sz, Z, code = self._matrix(y)
        pd, sz2, Z2, code2 = self._matrix(dy)
        if (sz, Z, code) != (sz2, Z2, code2):
            raise ValueError("y and dy must have the same layout and type")
        lt = np.ascontiguousarray(lut, dtype=np.int32)
        out = _widen_bits(dy).copy()
        self.lib.xro_bsr_softmax_bwd(py, pd, sz, Z, lt.ctypes.data, int(n_brows), int(block),
                                     float(scale), code, out.ctypes.data)
        return out

    def xent_count(self, target: np.ndarray, V: int, ignore_index: int = -100):
        t = np.ascontiguousarray(target, dtype=np.int64)
        counts = np.zeros(2, dtype=np.int64)
        self.lib.xro_xent_count(t.ctypes.data, t.shape[0], int(V), int(ignore_index),
                                counts.ctypes.data)
        return int(counts[0]), int(counts[1])

    @staticmethod
    def _scale(scale, M: int):
        """(array, stride) of an upstream gradient: None, a number, or one value per row."""
        if scale is None:
            return None, 0
        a = np.ascontiguousarray(np.atleast_1d(np.asarray(scale, dtype=np.float64)))
        if a.ndim != 1 or a.shape[0] not in (1, M):
            raise ValueError("scale must be a number or hold one value per row")
        return a, (1 if a.shape[0] == M and M != 1 else 0)

    def xent_rows(self, logits: np.ndarray, target: np.ndarray, V: int, n: int,
                  ignore_index: int = -100, rows=None, want_grad: bool = True,
                  reduction: str = "mean", scale=None):
        """(grad [len(rows), V] or None, loss [len(rows)]) for the given rows.

        reduction selects whose gradient is written (mean: of sum(loss)/n, sum: of
        sum(loss), none: of each row's loss); scale is the upstream gradient (a number, or
        one value per row of ``logits``), None meaning 1."""
        ptr, ld, M, code = self._matrix(logits)
        if not 0 < V <= logits.shape[1]:
            raise ValueError("V out of range")
        t = np.ascontiguousarray(target, dtype=np.int64)
        if t.shape[0] != M:
            raise ValueError("target length must equal the number of rows")
        if rows is None:
            ridx, nr = None, M
        else:
            ridx = np.ascontiguousarray(rows, dtype=np.int64)
            if ridx.size and (ridx.min() < 0 or ridx.max() >= M):
                raise ValueError("row index out of range")
            nr = ridx.shape[0]
        sc, sstride = self._scale(scale, M)
        # Outputs start as NaN, so an element the library never writes cannot pass as a value.
        grad = np.full((nr, V), np.nan, dtype=np.float64) if want_grad else None
        loss = np.full(nr, np.nan, dtype=np.float64)
        self.lib.xro_xent_rows_ex(ptr, ld, t.ctypes.data,
                                  None if ridx is None else ridx.ctypes.data, nr, int(V),
                                  int(ignore_index), code, REDUCTIONS[reduction], int(n),
                                  None if sc is None else sc.ctypes.data, sstride,
                                  None if grad is None else grad.ctypes.data, loss.ctypes.data)
        return grad, loss

    def mean(self, loss: np.ndarray, n: int) -> float:
        lo = np.ascontiguousarray(loss, dtype=np.float64)
        return float(self.lib.xro_mean(lo.ctypes.data, lo.shape[0], int(n)))

    def sum(self, loss: np.ndarray) -> float:
        lo = np.ascontiguousarray(loss, dtype=np.float64)
        return float(self.lib.xro_sum(lo.ctypes.data, lo.shape[0]))

    def xent(self, logits: np.ndarray, target: np.ndarray, V: int, ignore_index: int = -100,
             want_grad: bool = True, reduction: str = "mean", scale=None):
        """(grad or None, row losses, reduced loss, (n_non_ignore, n_bad)).

        The reduced loss is the mean for "mean", the sum for "sum" and None for "none"."""
        n, bad = self.xent_count(target, V, ignore_index)
        grad, loss = self.xent_rows(logits, target, V, n, ignore_index, None, want_grad,
                                    reduction, scale)
        red = {"mean": lambda: self.mean(loss, n), "sum": lambda: self.sum(loss),
               "none": lambda: None}[reduction]()
        return grad, loss, red, (n, bad)

    def element_mul(self, x: np.ndarray, scale, n_cols: int | None = None) -> np.ndarray:
        """x[i, :V] * scale_i as float64 [M, V]; scale is a number or one value per row."""
        ptr, ld, M, code = self._matrix(x)
        V = x.shape[1] if n_cols is None else int(n_cols)
        if not 0 < V <= x.shape[1]:
            raise ValueError("n_cols out of range")
        sc, sstride = self._scale(scale, M)
        if sc is None:
            raise ValueError("element_mul needs a scale")
        out = np.full((M, V), np.nan, dtype=np.float64)
        self.lib.xro_element_mul(ptr, ld, M, V, code, sc.ctypes.data, sstride, out.ctypes.data)
        return out


def _widen_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits or float32 values as float64 (exact)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from xr_oracle.c (compiled on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
