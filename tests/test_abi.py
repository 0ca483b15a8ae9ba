"""The C-ABI library on the CPU: it loads, exports every entry point include/xr.h declares,
and rejects bad arguments before touching a device. No call here can enqueue anything, with
or without a GPU: the pointers are made-up addresses, so every call either fails a check or
has nothing to do (M == 0)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xr.h")


@pytest.fixture(scope="module")
def xr():
    import cross_entropy_reductions_amd as xr
    return xr


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xr_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("xr_softmax_fwd", "xr_softmax_bwd", "xr_xent_fwd_bwd", "xr_xent_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(xr):
    for name in declared_functions():
        assert hasattr(xr.lib, name), f"{name} declared in xr.h but not exported"
    assert set(declared_functions()) == set(xr.C_SYMBOLS)


def test_status_strings_and_version(xr):
    assert xr.status_string(0) == "ok"
    for code in range(1, 13):
        assert xr.status_string(code) != "unknown status"
    assert xr.status_string(99) == "unknown status"
    assert xr.version() == 10400


XR_OK, XR_ERR_NULL, XR_ERR_SHAPE, XR_ERR_STRIDE, XR_ERR_DTYPE, XR_ERR_ALIAS = 0, 1, 2, 3, 4, 5
XR_ERR_WORKSPACE, XR_ERR_ALIGN, XR_ERR_DEVICE, XR_ERR_OPTION, XR_ERR_VALUE = 6, 7, 8, 10, 11


def test_softmax_argument_errors(xr):
    f = xr.lib.xr_softmax_fwd
    P = ctypes.c_void_p(0x10000)
    Q = ctypes.c_void_p(0x20000)
    assert f(P, 10, Q, 10, 4, 10, 2, None) == XR_ERR_DTYPE
    assert f(P, 10, Q, 10, -1, 10, 0, None) == XR_ERR_SHAPE
    assert f(P, 10, Q, 10, 4, 0, 0, None) == XR_ERR_SHAPE
    assert f(P, 9, Q, 10, 4, 10, 0, None) == XR_ERR_STRIDE
    assert f(P, 10, Q, 9, 4, 10, 0, None) == XR_ERR_STRIDE
    assert f(None, 10, Q, 10, 4, 10, 0, None) == XR_ERR_NULL
    assert f(P, 10, None, 10, 4, 10, 0, None) == XR_ERR_NULL
    assert f(ctypes.c_void_p(0x10002), 10, Q, 10, 4, 10, 0, None) == XR_ERR_ALIGN
    assert f(ctypes.c_void_p(0x10001), 10, Q, 10, 4, 10, 1, None) == XR_ERR_ALIGN
    # partial overlap: y starts 4 elements into x
    assert f(ctypes.c_void_p(0x10010), 10, P, 10, 4, 10, 0, None) == XR_ERR_ALIAS
    assert f(P, 10, Q, 10, 0, 10, 0, None) == XR_OK  # M == 0: nothing to do


def test_softmax_bwd_argument_errors(xr):
    f = xr.lib.xr_softmax_bwd
    A, B, C = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000))
    assert f(A, 8, B, 8, C, 8, 2, 8, 7, None) == XR_ERR_DTYPE
    assert f(A, 8, B, 8, C, 7, 2, 8, 0, None) == XR_ERR_STRIDE
    assert f(A, 8, None, 8, C, 8, 2, 8, 0, None) == XR_ERR_NULL
    assert f(ctypes.c_void_p(0x20004), 8, B, 8, C, 8, 2, 8, 0, None) == XR_ERR_ALIAS
    assert f(ctypes.c_void_p(0x30008), 8, B, 8, C, 8, 2, 8, 0, None) == XR_ERR_ALIAS


def test_softmax_ex_argument_errors(xr):
    f, g = xr.lib.xr_softmax_fwd_ex, xr.lib.xr_softmax_bwd_ex
    A, B, C, W = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x50000))
    # the checks of the calls without a workspace come first, unchanged
    assert f(A, 10, B, 10, 4, 10, 2, W, 4096, None) == XR_ERR_DTYPE
    assert f(A, 9, B, 10, 4, 10, 0, W, 4096, None) == XR_ERR_STRIDE
    assert f(None, 10, B, 10, 4, 10, 0, W, 4096, None) == XR_ERR_NULL
    assert f(ctypes.c_void_p(0x10010), 10, A, 10, 4, 10, 0, W, 4096, None) == XR_ERR_ALIAS
    assert g(A, 8, B, 8, C, 7, 2, 8, 0, W, 4096, None) == XR_ERR_STRIDE
    assert g(ctypes.c_void_p(0x30008), 8, B, 8, C, 8, 2, 8, 0, W, 4096, None) == XR_ERR_ALIAS
    # a workspace not on an 8-byte boundary
    assert f(A, 10, B, 10, 4, 10, 0, ctypes.c_void_p(0x50004), 4096, None) == XR_ERR_ALIGN
    assert g(A, 8, B, 8, C, 8, 2, 8, 1, ctypes.c_void_p(0x50002), 4096, None) == XR_ERR_ALIGN
    # M == 0: nothing to do, with or without a workspace
    assert f(A, 10, B, 10, 0, 10, 0, W, 4096, None) == XR_OK
    assert g(A, 8, B, 8, C, 8, 0, 8, 0, None, 0, None) == XR_OK
    assert xr.lib.xr_softmax_workspace_bytes(4, 0, 0) == 0
    assert xr.lib.xr_softmax_workspace_bytes(-1, 8, 0) == 0
    assert xr.lib.xr_softmax_workspace_bytes(4, 8, 9) == 0


def test_xent_argument_errors(xr):
    f = xr.lib.xr_xent_fwd_bwd
    L, T, R, Mn, W = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000, 0x50000))
    assert f(L, 8, T, 2, 8, -100, 3, R, Mn, None, W, 4096, None) == XR_ERR_DTYPE
    assert f(L, 8, T, -2, 8, -100, 0, R, Mn, None, W, 4096, None) == XR_ERR_SHAPE
    assert f(L, 8, T, 2, 0, -100, 0, R, Mn, None, W, 4096, None) == XR_ERR_SHAPE
    assert f(L, 7, T, 2, 8, -100, 0, R, Mn, None, W, 4096, None) == XR_ERR_STRIDE
    assert f(L, 8, T, 2, 8, -100, 0, R, None, None, W, 4096, None) == XR_ERR_NULL
    assert f(L, 8, T, 2, 8, -100, 0, R, Mn, None, None, 4096, None) == XR_ERR_NULL
    assert f(None, 8, T, 2, 8, -100, 0, R, Mn, None, W, 4096, None) == XR_ERR_NULL
    assert f(L, 8, None, 2, 8, -100, 0, R, Mn, None, W, 4096, None) == XR_ERR_NULL
    assert f(L, 8, ctypes.c_void_p(0x20004), 2, 8, -100, 0, R, Mn, None, W, 4096, None) == XR_ERR_ALIGN
    assert f(ctypes.c_void_p(0x10002), 8, T, 2, 8, -100, 0, R, Mn, None, W, 4096, None) == XR_ERR_ALIGN


def test_xent_ex_argument_errors(xr):
    f = xr.lib.xr_xent_fwd_bwd_ex
    L, T, R, Mn, W, S = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000,
                                                       0x50000, 0x60000))
    assert f(L, 8, T, 2, 8, -100, 0, 3, None, 0, R, Mn, None, W, 4096, None) == XR_ERR_VALUE
    assert f(L, 8, T, 2, 8, -100, 0, -1, None, 0, R, Mn, None, W, 4096, None) == XR_ERR_VALUE
    assert f(L, 8, T, 2, 8, -100, 0, 0, S, -1, R, Mn, None, W, 4096, None) == XR_ERR_VALUE
    assert f(L, 8, T, 2, 8, -100, 5, 0, None, 0, R, Mn, None, W, 4096, None) == XR_ERR_DTYPE
    # mean and sum need the loss output; none does not
    assert f(L, 8, T, 2, 8, -100, 0, 0, None, 0, R, None, None, W, 4096, None) == XR_ERR_NULL
    assert f(L, 8, T, 2, 8, -100, 0, 1, None, 0, R, None, None, W, 4096, None) == XR_ERR_NULL
    assert f(L, 8, T, 2, 8, -100, 0, 2, None, 0, None, None, None, W, 4096, None) == XR_ERR_NULL
    assert f(L, 8, T, 2, 8, -100, 0, 2, ctypes.c_void_p(0x60002), 1, R, None, None, W, 4096,
             None) == XR_ERR_ALIGN


def test_xent_overlap_errors(xr):
    """No written buffer of the cross-entropy (logits, row losses, loss, counts, workspace)
    may overlap another buffer of the call; the check runs before anything is enqueued."""
    f = xr.lib.xr_xent_fwd_bwd_ex
    L, T, R, Mn, C, W, S = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000, 0x400000,
                                                          0x500000, 0x600000, 0x700000))
    M, V = 4, 1000  # logits span 0x100000 + 4 * 1000 * 2 bytes (bf16)
    inside = ctypes.c_void_p(0x100000 + 4000)
    ok_args = dict(L=L, T=T, R=R, Mn=Mn, C=C, W=W, S=S)

    def call(wsb=4096, **kw):
        a = {**ok_args, **kw}
        return f(a["L"], V, a["T"], M, V, -100, 1, 0, a["S"], 1, a["R"], a["Mn"], a["C"], a["W"],
                 wsb, None)
    for name in ("T", "R", "Mn", "C", "W", "S"):  # each one moved inside the logits
        assert call(**{name: inside}) == XR_ERR_ALIAS, name
    # the workspace over the row losses, the counts over the mean, the loss over the targets
    assert call(W=ctypes.c_void_p(0x300000 - 64)) == XR_ERR_ALIAS
    assert call(C=ctypes.c_void_p(0x400000 + 0)) == XR_ERR_ALIAS
    assert call(Mn=ctypes.c_void_p(0x200000 + 8)) == XR_ERR_ALIAS
    # Calls that pass the overlap checks stop at the next ones, before anything is enqueued:
    # without a device at the device query, with one at the 8-byte workspace (these
    # addresses are not device memory: a launch on them would fault a GPU).
    # Read-only buffers may overlap each other (targets and upstream gradient) ...
    assert call(wsb=8, S=ctypes.c_void_p(0x200000)) in (XR_ERR_DEVICE, XR_ERR_WORKSPACE)
    # ... and exactly adjacent spans do not overlap.
    assert call(wsb=8, R=ctypes.c_void_p(0x100000 + 8000)) in (XR_ERR_DEVICE, XR_ERR_WORKSPACE)


def test_xent_row_loss_may_be_null(xr):
    """row_loss may be NULL for the mean and sum (kept in the workspace), not for none (the
    row losses are its result)."""
    f = xr.lib.xr_xent_fwd_bwd_ex
    L, T, Mn, W = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x400000, 0x600000))
    assert f(L, 8, T, 2, 8, -100, 0, 2, None, 0, None, None, None, W, 4096, None) == XR_ERR_NULL
    for red in (0, 1):  # past the argument checks, stopped before anything is enqueued (above)
        assert f(L, 8, T, 2, 8, -100, 0, red, None, 0, None, Mn, None, W, 8, None) in \
            (XR_ERR_DEVICE, XR_ERR_WORKSPACE)


def test_workspace_status_argument_errors(xr):
    f = xr.lib.xr_workspace_status
    W, S = ctypes.c_void_p(0x600000), ctypes.c_void_p(0x700000)
    assert f(None, 4096, S, None) == XR_ERR_NULL
    assert f(W, 4096, None, None) == XR_ERR_NULL
    assert f(ctypes.c_void_p(0x600004), 4096, S, None) == XR_ERR_ALIGN
    assert f(W, 4096, ctypes.c_void_p(0x700002), None) == XR_ERR_ALIGN
    assert f(W, 64, S, None) == 6  # XR_ERR_WORKSPACE: smaller than the counts block
    assert f(W, 4096, ctypes.c_void_p(0x600008), None) == XR_ERR_ALIAS


def test_probe_argument_errors(xr):
    f = xr.lib.xr_probe_rows
    O, A, B = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000))
    # (out, ld_out, in0, in1, ld_in, M, N, dtype, threads, vpt, split, target, ignore, stream)
    assert f(O, 64, A, None, 64, 4, 64, 3, 64, 4, 1, None, -100, None) == XR_ERR_DTYPE
    assert f(O, 64, A, None, 64, 4, 64, 0, 64, 4, 0, None, -100, None) == XR_ERR_SHAPE
    assert f(O, 63, A, None, 64, 4, 64, 0, 64, 4, 1, None, -100, None) == XR_ERR_STRIDE
    assert f(None, 64, A, None, 64, 4, 64, 0, 64, 4, 1, None, -100, None) == XR_ERR_NULL
    assert f(O, 64, A, None, 64, 4, 62, 0, 64, 4, 1, None, -100, None) == XR_ERR_ALIGN
    assert f(ctypes.c_void_p(0x100004), 64, A, None, 64, 4, 64, 0, 64, 4, 1, None, -100,
             None) == XR_ERR_ALIGN
    assert f(O, 64, A, None, 64, 4, 64, 0, 96, 4, 1, None, -100, None) == XR_ERR_SHAPE
    assert f(O, 64, A, B, 64, 4, 64, 0, 64, 16, 1, None, -100, None) == XR_ERR_SHAPE
    assert f(O, 64, A, None, 64, 0, 64, 0, 64, 4, 1, None, -100, None) == XR_OK


def test_probe_copy_argument_errors(xr):
    f = xr.lib.xr_probe_copy
    O, A, B = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000))
    # (out, in, in1, bytes, workgroups, threads, stream)
    assert f(O, A, None, -16, 64, 256, None) == XR_ERR_SHAPE
    assert f(O, A, None, 4096, -1, 256, None) == XR_ERR_SHAPE
    assert f(O, A, B, 0, 64, 256, None) == XR_OK           # nothing to copy: nothing enqueued
    assert f(None, A, None, 4096, 64, 256, None) == XR_ERR_NULL
    assert f(O, None, B, 4096, 0, 256, None) == XR_ERR_NULL
    assert f(ctypes.c_void_p(0x100008), A, None, 4096, 64, 256, None) == XR_ERR_ALIGN
    assert f(O, A, ctypes.c_void_p(0x300004), 4096, 64, 256, None) == XR_ERR_ALIGN
    assert f(O, A, None, 4100, 64, 256, None) == XR_ERR_ALIGN
    assert f(O, ctypes.c_void_p(0x100800), None, 4096, 64, 256, None) == XR_ERR_ALIAS
    assert f(O, A, ctypes.c_void_p(0x100800), 4096, 64, 256, None) == XR_ERR_ALIAS
    assert f(O, ctypes.c_void_p(0x100800), None, 4096, 0, 256, None) == XR_ERR_ALIAS
    assert f(O, A, B, 4096, 0, 256, None) == XR_ERR_VALUE   # the runtime's copy has one input
    assert f(O, A, B, 4096, 64, 128, None) == XR_ERR_SHAPE  # not a copy-kernel workgroup size
    # in place (out == in exactly): the copy kernel only, with one input
    assert f(O, O, None, 4096, 0, 256, None) == XR_ERR_ALIAS
    assert f(O, O, B, 4096, 64, 256, None) == XR_ERR_VALUE
    assert f(O, O, ctypes.c_void_p(0x100800), 4096, 64, 256, None) == XR_ERR_ALIAS
    assert f(O, O, None, 4096, 64, 128, None) == XR_ERR_SHAPE


def test_element_mul_argument_errors(xr):
    f = xr.lib.xr_element_mul
    X, G = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x90000)
    assert f(X, 8, 4, 8, 2, G, 0, None) == XR_ERR_DTYPE
    assert f(X, 8, 4, 8, 0, G, -1, None) == XR_ERR_VALUE
    assert f(X, 8, -1, 8, 0, G, 0, None) == XR_ERR_SHAPE
    assert f(X, 8, 4, 0, 0, G, 0, None) == XR_ERR_SHAPE
    assert f(X, 7, 4, 8, 0, G, 0, None) == XR_ERR_STRIDE
    assert f(None, 8, 4, 8, 0, G, 0, None) == XR_ERR_NULL
    assert f(X, 8, 4, 8, 0, None, 0, None) == XR_ERR_NULL
    assert f(ctypes.c_void_p(0x10001), 8, 4, 8, 1, G, 0, None) == XR_ERR_ALIGN
    assert f(X, 8, 4, 8, 0, ctypes.c_void_p(0x90002), 0, None) == XR_ERR_ALIGN
    # the factors may not lie inside the matrix they scale
    assert f(X, 8, 4, 8, 0, ctypes.c_void_p(0x10010), 0, None) == XR_ERR_ALIAS
    assert f(X, 8, 0, 8, 0, None, 0, None) == XR_OK  # M == 0: nothing to do


def test_options(xr):
    o = xr.lib.xr_set_option
    assert o(1, 4) == XR_ERR_OPTION and o(2, 1) == XR_ERR_OPTION and o(3, 96) == XR_ERR_OPTION
    assert o(4, -2) == XR_ERR_OPTION and o(99, 0) == XR_ERR_OPTION
    assert o(5, 3) == XR_ERR_OPTION and o(6, 2) == XR_ERR_OPTION and o(6, -1) == XR_ERR_OPTION
    assert o(7, 3) == XR_ERR_OPTION and o(7, -1) == XR_ERR_OPTION
    for opt, val in ((1, 3), (2, 4), (3, 256), (4, -1), (5, 2), (6, 1), (7, 2), (7, 1)):
        assert o(opt, val) == XR_OK
    xr.reset_options()


def test_plan_argument_errors(xr):
    out = xr.XrPlan()
    assert xr.lib.xr_plan(0, 4, 8, 0, 1, None) == XR_ERR_NULL
    assert xr.lib.xr_plan(6, 4, 8, 0, 1, ctypes.byref(out)) == XR_ERR_SHAPE
    assert xr.lib.xr_plan(-1, 4, 8, 0, 1, ctypes.byref(out)) == XR_ERR_SHAPE
    assert xr.lib.xr_plan(0, 4, 8, 5, 1, ctypes.byref(out)) == XR_ERR_DTYPE


def test_nll_argument_errors(xr):
    f = xr.lib.xr_nll_fwd
    Y, X, I, L, W = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000, 0x50000))
    assert f(Y, 8, X, 8, I, L, 4, 8, 2, None, 0, None) == XR_ERR_DTYPE
    assert f(Y, 8, X, 8, I, L, -1, 8, 0, None, 0, None) == XR_ERR_SHAPE
    assert f(Y, 7, X, 8, I, L, 4, 8, 0, None, 0, None) == XR_ERR_STRIDE
    assert f(Y, 8, X, 8, None, L, 4, 8, 0, None, 0, None) == XR_ERR_NULL
    assert f(Y, 8, X, 8, I, None, 4, 8, 0, None, 0, None) == XR_ERR_NULL
    assert f(Y, 8, X, 8, ctypes.c_void_p(0x30004), L, 4, 8, 0, None, 0, None) == XR_ERR_ALIGN
    assert f(Y, 8, X, 8, I, L, 4, 8, 0, ctypes.c_void_p(0x50004), 4096, None) == XR_ERR_ALIGN
    assert f(ctypes.c_void_p(0x10010), 8, ctypes.c_void_p(0x10000), 8, I, L, 4, 8, 0, None, 0,
             None) == XR_ERR_ALIAS
    # the losses may not land inside the output or the input
    assert f(Y, 8, X, 8, I, ctypes.c_void_p(0x10010), 4, 8, 0, None, 0, None) == XR_ERR_ALIAS
    assert f(Y, 8, X, 8, I, ctypes.c_void_p(0x20010), 4, 8, 0, None, 0, None) == XR_ERR_ALIAS
    assert f(Y, 8, X, 8, I, L, 0, 8, 0, W, 4096, None) == XR_OK
    assert xr.lib.xr_nll_fwd_workspace_bytes(4, 0, 0) == 0


def test_layernorm_argument_errors(xr):
    f = xr.lib.xr_layernorm_fwd
    Y, X, W, B, Mn, R = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000,
                                                       0x50000, 0x60000))
    assert f(Y, 8, X, 8, W, B, Mn, R, 4, 8, ctypes.c_float(1e-5), 2, None) == XR_ERR_DTYPE
    assert f(Y, 8, X, 8, W, B, Mn, R, 4, 8, ctypes.c_float(-1.0), 0, None) == XR_ERR_VALUE
    assert f(Y, 8, X, 8, W, B, Mn, R, 4, 8, ctypes.c_float(float("nan")), 0, None) == XR_ERR_VALUE
    assert f(Y, 7, X, 8, W, B, Mn, R, 4, 8, ctypes.c_float(1e-5), 0, None) == XR_ERR_STRIDE
    assert f(Y, 8, X, 8, None, B, Mn, R, 4, 8, ctypes.c_float(1e-5), 0, None) == XR_ERR_NULL
    assert f(Y, 8, X, 8, W, B, Mn, ctypes.c_void_p(0x60002), 4, 8, ctypes.c_float(1e-5), 0,
             None) == XR_ERR_ALIGN
    assert f(Y, 8, X, 8, W, B, ctypes.c_void_p(0x10008), R, 4, 8, ctypes.c_float(1e-5), 0,
             None) == XR_ERR_ALIAS
    assert f(Y, 8, X, 8, W, B, Mn, R, 0, 8, ctypes.c_float(1e-5), 0, None) == XR_OK
    g = xr.lib.xr_layernorm_bwd
    DX, DY, DW, DB, WS = (ctypes.c_void_p(a) for a in (0x70000, 0x80000, 0x90000, 0xA0000,
                                                        0xB0000))
    assert g(DX, 8, DY, 8, X, 8, W, Mn, R, DW, DB, 4, 8, 3, WS, 1 << 20, None) == XR_ERR_DTYPE
    assert g(DX, 8, DY, 7, X, 8, W, Mn, R, DW, DB, 4, 8, 0, WS, 1 << 20, None) == XR_ERR_STRIDE
    assert g(DX, 8, DY, 8, X, 8, W, Mn, R, None, DB, 4, 8, 0, WS, 1 << 20, None) == XR_ERR_NULL
    assert g(DX, 8, DY, 8, X, 8, W, Mn, R, DW, DB, 4, 8, 0, None, 1 << 20, None) == XR_ERR_NULL
    assert g(DX, 8, DY, 8, X, 8, W, Mn, R, DW, DB, 4, 8, 0, ctypes.c_void_p(0xB0008), 1 << 20,
             None) == XR_ERR_ALIGN
    assert g(DX, 8, DY, 8, X, 8, W, Mn, R, DW, ctypes.c_void_p(0x90010), 4, 8, 0, WS, 1 << 20,
             None) == XR_ERR_ALIAS
    assert g(ctypes.c_void_p(0x80010), 8, DY, 8, X, 8, W, Mn, R, DW, DB, 4, 8, 0, WS, 1 << 20,
             None) == XR_ERR_ALIAS


def test_bsr_argument_errors(xr):
    f = xr.lib.xr_bsr_softmax_bwd
    Y, D, L = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000))
    one = ctypes.c_float(1.0)
    assert f(Y, 4096, D, 4096, 2, L, 20, 4, 4, 32, one, 2, None) == XR_ERR_DTYPE
    assert f(Y, 4096, D, 4096, 2, L, 20, 4, 4, 48, one, 0, None) == XR_ERR_SHAPE  # not a power of 2
    assert f(Y, 4096, D, 4096, 2, L, 20, 4, 4, 2, one, 1, None) == XR_ERR_SHAPE   # below a vector
    assert f(Y, 4096, D, 4096, 2, L, 7, 4, 4, 32, one, 0, None) == XR_ERR_SHAPE   # table too short
    assert f(Y, 4095, D, 4096, 2, L, 20, 4, 4, 32, one, 0, None) == XR_ERR_STRIDE
    assert f(Y, 4096, D, 4096, 2, L, 20, 4, 4, 32, ctypes.c_float(float("nan")), 0, None) == XR_ERR_VALUE
    assert f(None, 4096, D, 4096, 2, L, 20, 4, 4, 32, one, 0, None) == XR_ERR_NULL
    assert f(ctypes.c_void_p(0x100008), 4096, D, 4096, 2, L, 20, 4, 4, 32, one, 0, None) == XR_ERR_ALIGN
    assert f(Y, 4096, ctypes.c_void_p(0x100000 + 4096), 4096, 2, L, 20, 4, 4, 32, one, 0,
             None) == XR_ERR_ALIAS
    assert f(Y, 4096, D, 4096, 0, L, 20, 4, 4, 32, one, 0, None) == XR_OK


def test_spans_beyond_the_limit_are_refused(xr):
    """An operand spanning 2^48 bytes or more is refused with XR_ERR_SHAPE before any arithmetic
    on its sizes or addresses (none of these calls gets as far as a device query)."""
    lib = xr.lib
    P, Q, R, S, T = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000, 0x50000))
    big, half = 1 << 24, 1 << 46   # 2^24 x 2^24 bf16 rows: 2^49 bytes
    one = ctypes.c_float(1.0)
    assert lib.xr_softmax_fwd(P, big, Q, big, big, big, 1, None) == XR_ERR_SHAPE
    assert lib.xr_softmax_fwd(P, 1 << 47, Q, 8, 2, 8, 1, None) == XR_ERR_SHAPE  # the stride alone
    # just under the limit the sizes pass; the spans then overlap (nothing is enqueued)
    assert lib.xr_softmax_fwd(P, half, Q, 8, 2, 8, 1, None) == XR_ERR_ALIAS
    # (M - 1) ld + N elements of 2 bytes: 2^48 - 2 bytes passes, 2^48 does not
    assert lib.xr_softmax_fwd(P, half, Q, half, 2, half - 1, 1, None) == XR_ERR_ALIAS
    assert lib.xr_softmax_fwd(P, half, Q, half, 2, half, 1, None) == XR_ERR_SHAPE
    assert lib.xr_softmax_bwd(P, big, Q, big, R, big, big, big, 1, None) == XR_ERR_SHAPE
    assert lib.xr_softmax_fwd_ex(P, big, Q, big, big, big, 1, S, 4096, None) == XR_ERR_SHAPE
    assert lib.xr_nll_fwd(P, big, Q, big, R, S, big, big, 1, None, 0, None) == XR_ERR_SHAPE
    assert lib.xr_xent_fwd_bwd_ex(P, big, Q, big, big, -100, 1, 0, None, 0, R, S, T, T, 4096,
                                  None) == XR_ERR_SHAPE
    # upstream values read at i * stride: (M - 1) * 2^50 floats
    assert lib.xr_xent_fwd_bwd_ex(P, 8, Q, 4, 8, -100, 1, 0, R, 1 << 50, S, T, None, T, 4096,
                                  None) == XR_ERR_SHAPE
    assert lib.xr_element_mul(P, big, big, big, 1, Q, 0, None) == XR_ERR_SHAPE
    assert lib.xr_element_mul(P, 8, 4, 8, 1, Q, 1 << 50, None) == XR_ERR_SHAPE
    assert lib.xr_layernorm_fwd(P, big, Q, big, R, S, T, T, big, big, ctypes.c_float(1e-5), 1,
                                None) == XR_ERR_SHAPE
    assert lib.xr_layernorm_bwd(P, big, Q, big, R, big, S, T, T, S, T, big, big, 1, T, 1 << 20,
                                None) == XR_ERR_SHAPE
    assert lib.xr_probe_rows(P, big, Q, None, big, big, big, 1, 256, 8, 1, None, -100,
                             None) == XR_ERR_SHAPE
    assert lib.xr_probe_copy(P, Q, None, 1 << 48, 64, 256, None) == XR_ERR_SHAPE
    # block-sparse: a block count whose byte product would wrap a 64-bit integer, and a batch
    # count past the limit
    assert lib.xr_bsr_softmax_bwd(P, 4096, Q, 4096, 2, R, 20, 4, 1 << 61, 32, one, 1,
                                  None) == XR_ERR_SHAPE
    assert lib.xr_bsr_softmax_bwd(P, 4096, Q, 4096, 1 << 40, R, 20, 4, 4, 32, one, 1,
                                  None) == XR_ERR_SHAPE
    # plans and workspace queries of such sizes
    out = xr.XrPlan()
    assert lib.xr_plan_model(0, big, big, 1, 1, 256, 8, ctypes.byref(out)) == XR_ERR_SHAPE
    assert lib.xr_plan_model(0, 4, 1 << 48, 0, 1, 256, 8, ctypes.byref(out)) == XR_ERR_SHAPE
    assert lib.xr_plan_model(0, 4, 8, 0, 1, 256, 8, ctypes.byref(out)) == XR_OK
    for q in (lib.xr_softmax_workspace_bytes, lib.xr_xent_workspace_bytes,
              lib.xr_nll_fwd_workspace_bytes):
        assert q(big, big, 1) == 0


def test_header_is_plain_c_and_links(tmp_path, xr):
    """include/xr.h compiles as C99 on its own, and a C program linked against libxr.so
    runs its argument checks (tests/c/abi_check.c)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = os.path.join(ROOT, "tests", "c", "abi_check.c")
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(xr.LIBRARY)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    src, "-o", exe, "-L", libdir, "-lxr", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "ok"
