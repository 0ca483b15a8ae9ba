"""xr_xent_fwd_bwd_noalloc (the cross-entropy for callers that cannot allocate: its scratch is
a static device array of the library) against xr_xent_fwd_bwd_ex with a caller's workspace:
the same kernels, so the gradient, the row losses, the reduced loss and the counts must be
bit-identical; two calls in a row, the second smaller, so the second runs on the scratch the
first left behind. Sizes beyond the static array are refused with nothing enqueued."""
from __future__ import annotations

import ctypes

import pytest
import torch

import synth
from gpu_util import to_device

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import cross_entropy_reductions_amd as xr
else:  # collected on a machine without a GPU: every test here is skipped
    xr = None
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no HIP device")]

XR_ERR_TOO_LARGE = 12


def noalloc(x, t, reduction="mean", grad_scale=None, row_loss=True):
    """The no-allocation entry point through the C ABI; returns (loss, row_loss, counts)."""
    M, V = x.shape
    dt = xr.BF16 if x.dtype == torch.bfloat16 else xr.F32
    rl = torch.empty(M, dtype=torch.float32, device=x.device) if row_loss else None
    loss = torch.empty(1, dtype=torch.float32, device=x.device)
    counts = torch.empty(3, dtype=torch.int32, device=x.device)
    ps, stride = (None, 0) if grad_scale is None else (grad_scale.data_ptr(),
                                                       0 if grad_scale.numel() == 1 else 1)
    st = xr.lib.xr_xent_fwd_bwd_noalloc(
        x.data_ptr(), x.stride(0) if M > 1 else V, t.data_ptr(), M, V, -100, dt,
        xr.REDUCTIONS[reduction], ps, stride, None if rl is None else rl.data_ptr(),
        None if reduction == "none" else loss.data_ptr(), counts.data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, (rl if reduction == "none" else loss), rl, counts


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# Each pair: a call, then a smaller one on the scratch the first left behind.
CASES = [
    [(8192, 32000, "bf16", "mean", None), (300, 5003, "bf16", "mean", None)],
    [(64, 128256, "bf16", "sum", 0.5), (9, 128256, "bf16", "mean", None)],
    [(257, 70001, "f32", "none", "rows"), (40, 50000, "f32", "sum", -2.0)],
]


@pytest.mark.parametrize("pair", range(len(CASES)))
def test_noalloc_matches_the_workspace_entry_point(pair):
    for k, (M, V, dtype, reduction, scale) in enumerate(CASES[pair]):
        print(f"no-alloc pair {pair} call {k}: M={M} V={V} {dtype} {reduction} scale={scale}",
              flush=True)
        x_h = synth.random_rows(31000 + 10 * pair + k, M, V, dtype=dtype, scale=2.0)
        t_h = synth.random_targets(31100 + 10 * pair + k, M, V, ignore_frac=0.1)
        t_h[min(2, M - 1)] = V + 3  # an out-of-range target
        t = to_device(t_h)
        if scale == "rows":
            s = to_device(synth.random_rows(31200 + pair, 1, M, dtype="f32", scale=1.5)[0])
        elif scale is not None:
            s = torch.tensor([scale], dtype=torch.float32, device="cuda")
        else:
            s = None
        a, b = to_device(x_h), to_device(x_h)
        la, ra, ca = xr.xent_fwd_bwd(a, t, reduction=reduction, grad_scale=s)
        for with_rows in ((True, False) if reduction != "none" else (True,)):
            b.copy_(to_device(x_h))
            st, lb, rb, cb = noalloc(b, t, reduction, s, row_loss=with_rows)
            assert st == 0, xr.status_string(st)
            torch.cuda.synchronize()
            assert torch.equal(bits(a), bits(b)), "gradient differs"
            assert torch.equal(bits(la), bits(lb)), "reduced loss differs"
            assert torch.equal(ca, cb), "counts differ"
            if with_rows:
                assert torch.equal(bits(ra), bits(rb)), "row losses differ"


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """2^21 rows kept without row_loss need 8 MiB of scratch, more than the array holds:
    refused before anything is enqueued (the logits stay as they were)."""
    M, V = 1 << 21, 1
    x = torch.randn(M, V, dtype=torch.float32, device="cuda")
    before = x.clone()
    t = torch.zeros(M, dtype=torch.int64, device="cuda")
    st, _, _, _ = noalloc(x, t, "mean", None, row_loss=False)
    assert st == XR_ERR_TOO_LARGE, xr.status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(x, before)
    # the same sizes with the caller's row_loss fit: 256 bytes of counts, no split slots
    st, loss, _, counts = noalloc(x, t, "mean", None, row_loss=True)
    assert st == 0, xr.status_string(st)
    torch.cuda.synchronize()
    assert counts.tolist() == [M, 0, 0]
    # one column: loss 0 and gradient 0 in exact arithmetic (fp32 leaves the loss a residue)
    assert abs(float(loss.item())) < 1e-6 and bool((x == 0).all())


def test_noalloc_under_graph_capture():
    """The callers it is for: two calls of different sizes captured into one HIP graph
    (kernels only: nothing to allocate, no memset), replayed three times on fresh copies of
    the inputs with eager work between the replays; every replay equals the eager results
    bit for bit."""
    cases = [(256, 32000, 31300), (8, 128256, 31310)]
    xs, ts, eager = [], [], []
    for M, V, seed in cases:
        x_h = synth.random_rows(seed, M, V, dtype="bf16", scale=2.0)
        t_h = synth.random_targets(seed + 1, M, V, ignore_frac=0.1)
        xs.append(to_device(x_h))
        ts.append(to_device(t_h))
        a = xs[-1].clone()
        st, loss, rows, counts = noalloc(a, ts[-1])
        assert st == 0, xr.status_string(st)
        eager.append([a, loss, rows, counts])
    torch.cuda.synchronize()
    static_x = [x.clone() for x in xs]
    outs = [(torch.empty(1, dtype=torch.float32, device="cuda"),
             torch.empty(M, dtype=torch.float32, device="cuda"),
             torch.empty(3, dtype=torch.int32, device="cuda")) for M, _, _ in cases]
    stream = ctypes.c_void_p

    def run():
        for (M, V, _), x, t, (loss, rows, counts) in zip(cases, static_x, ts, outs):
            st = xr.lib.xr_xent_fwd_bwd_noalloc(
                x.data_ptr(), V, t.data_ptr(), M, V, -100, xr.BF16, xr.REDUCTIONS["mean"], None,
                0, rows.data_ptr(), loss.data_ptr(), counts.data_ptr(),
                stream(torch.cuda.current_stream().cuda_stream))
            assert st == 0, xr.status_string(st)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for k in range(3):
        for dst, src in zip(static_x, xs):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, (loss, rows, counts)) in enumerate(zip(static_x, outs)):
            want = eager[i]
            assert torch.equal(bits(x), bits(want[0])), f"replay {k} case {i}: gradient"
            assert torch.equal(bits(loss), bits(want[1])), f"replay {k} case {i}: loss"
            assert torch.equal(bits(rows), bits(want[2])), f"replay {k} case {i}: row losses"
            assert torch.equal(counts, want[3]), f"replay {k} case {i}: counts"
        _ = (static_x[0].float() * 2).sum().item()  # the program's own work between replays
