"""Streams and HIP graphs: every entry point enqueues on the stream it is given, and the
cross-entropy, softmax and layer norm calls can be captured into a HIP graph (they launch
kernels only: no allocation, no memset, no synchronisation). Replays are checked one by
one against the eager results, with the program's own work and synchronisations between
them."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from gpu_util import to_device, to_host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import cross_entropy_reductions_amd as xr
else:  # collected on a machine without a GPU: every test here is skipped
    xr = None
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no HIP device")]


def test_side_stream():
    """Work on a side stream, synchronised only through that stream, gives the default
    stream's results."""
    w = synth.xent_c3(M=512)
    x_ref = to_device(w["x"])
    t = to_device(w["target"])
    mean_ref, rows_ref, _ = xr.xent_fwd_bwd(x_ref, t)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    x = to_device(w["x"])
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        mean, rows, _ = xr.xent_fwd_bwd(x, t)
        y = xr.softmax_fwd(x_ref[:, :1000].contiguous())
    side.synchronize()
    assert torch.equal(x.view(torch.int16), x_ref.view(torch.int16))
    assert torch.equal(rows, rows_ref) and torch.equal(mean, mean_ref)
    assert torch.allclose(y.float().sum(dim=1), torch.ones(512, device="cuda"), atol=2e-2)


def _graph_case(run, inputs, replays=4):
    """Capture run(*inputs) once, replay it `replays` times on fresh copies of the inputs,
    and compare every replay with the eager result bit for bit."""
    eager_in = [a.clone() for a in inputs]
    eager_out = [o.clone() for o in run(*eager_in)]
    torch.cuda.synchronize()
    static_in = [a.clone() for a in inputs]
    # warm up on a side stream (library state such as the device cache), as torch advises
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(*[a.clone() for a in inputs])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static_out = run(*static_in)
    for k in range(replays):
        for dst, src in zip(static_in, inputs):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(static_out, eager_out):
            assert torch.equal(got.view(torch.uint8) if got.dtype != torch.uint8 else got,
                               want.view(torch.uint8) if want.dtype != torch.uint8 else want), \
                f"replay {k}"
        # the program's own eager work between replays
        torch.cuda.synchronize()
        _ = (static_in[0].float() * 2).sum().item()


@pytest.mark.parametrize("M,V", [(256, 32000), (8, 128256)], ids=["rows-whole-or-4-chunks", "split-short-batch"])
def test_graph_xent(M, V):
    x = to_device(synth.random_rows(15000, M, V, dtype="bf16", scale=2.0))
    t = to_device(synth.random_targets(15001, M, V, ignore_frac=0.1))
    ws = torch.empty(max(256, xr.xent_workspace_bytes(M, V, torch.bfloat16)), dtype=torch.uint8,
                     device="cuda")
    row_loss = torch.empty(M, dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    counts = torch.empty(3, dtype=torch.int32, device="cuda")

    def run(xx, tt):
        xr.xent_fwd_bwd(xx, tt, row_loss=row_loss, mean_loss=mean, counts=counts, workspace=ws)
        return [xx, row_loss, mean, counts]

    _graph_case(run, [x, t])


def test_graph_softmax_and_layernorm():
    M, N = 512, 4096
    x = to_device(synth.random_rows(15100, M, N, dtype="bf16", scale=2.0))
    dy = to_device(synth.random_rows(15101, M, N, dtype="bf16", scale=1.0))
    wb = synth.random_rows(15102, 2, N, dtype="bf16", scale=1.0)
    w, b = to_device(np.ascontiguousarray(wb[0])), to_device(np.ascontiguousarray(wb[1]))
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    yl = torch.empty_like(x)
    mean = torch.empty(M, dtype=torch.float32, device="cuda")
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    dxl = torch.empty_like(x)
    dw = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    db = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(16, xr.layernorm_bwd_workspace_bytes(M, N, torch.bfloat16)),
                     dtype=torch.uint8, device="cuda")

    def run(xx, dd):
        xr.softmax_fwd(xx, y)
        xr.softmax_bwd(y, dd, dx)
        xr.layernorm_fwd(xx, w, b, 1e-5, out=yl, mean=mean, rstd=rstd)
        xr.layernorm_bwd(dd, xx, w, mean, rstd, dx=dxl, dw=dw, db=db, workspace=ws)
        return [y, dx, yl, dxl, dw, db]

    _graph_case(run, [x, dy])


def test_graph_softmax_split_rows():
    """The softmax forward and backward over split rows (a workspace slot fill kernel, then
    the row kernel, per call) captured and replayed."""
    M, N = 8, 128256
    x = to_device(synth.random_rows(15200, M, N, dtype="bf16", scale=2.0))
    dy = to_device(synth.random_rows(15201, M, N, dtype="bf16", scale=1.0))
    assert xr.plan("softmax_fwd_ws", M, N, torch.bfloat16)["split"] > 1
    ws = torch.empty(xr.softmax_workspace_bytes(M, N, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty_like(x)
    dx = torch.empty_like(x)

    def run(xx, dd):
        xr.softmax_fwd(xx, y, workspace=ws)
        xr.softmax_bwd(y, dd, dx, workspace=ws)
        return [y, dx]

    _graph_case(run, [x, dy])
