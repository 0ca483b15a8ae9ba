"""The memory-ceiling probes move exactly the bytes they claim. xr_probe_rows: every row
copied (or the XOR of two inputs), rows whose target is ignore_index written with zeros and
not read, padding untouched, in every launch shape the benchmark times it in. xr_probe_copy:
every byte copied (or the XOR of two inputs) and nothing written past the end, by the copy
kernel and the runtime's copy."""
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


@pytest.mark.parametrize("M,N,ld,dtype,shape", [
    (33, 4096, 4096, "bf16", (64, 8, 1)), (40, 32000, 32000, "bf16", (128, 8, 4)),
    (17, 128256, 128256, "bf16", (512, 16, 2)), (9, 256000, 256064, "f32", (512, 16, 8)),
    (5, 4096, 4104, "bf16", (64, 4, 2)),
])
def test_probe_copies_rows(M, N, ld, dtype, shape):
    import bench
    t_, v_, s_ = shape
    assert shape in bench.probe_shapes(N * (2 if dtype == "bf16" else 4) // 16, False)
    x_h = synth.random_rows(40000 + N, M, N, ld=ld, dtype=dtype, scale=1.0, pad_nan=ld > N)
    tgt = synth.random_targets(40001 + N, M, N, ignore_frac=0.25)
    x = to_device(x_h)
    out = torch.full_like(x, float("nan"))
    xr.probe_rows(out[:, :N], x[:, :N], threads=t_, vpt=v_, split=s_)
    torch.cuda.synchronize()
    got = to_host(out)
    assert np.array_equal(got[:, :N].view(np.uint8), x_h[:, :N].view(np.uint8)), "copy"
    assert np.all(np.isnan(got[:, N:].astype(np.float32) if dtype == "f32"
                           else synth.f32_from_bf16_bits(got[:, N:]))), "padding touched"
    # in place, ignored rows zeroed
    xr.probe_rows(x[:, :N], x[:, :N], threads=t_, vpt=v_, split=s_, target=to_device(tgt))
    torch.cuda.synchronize()
    got = to_host(x)
    ign = tgt == -100
    assert np.all(got[ign, :N] == 0)
    assert np.array_equal(got[~ign, :N].view(np.uint8), x_h[~ign, :N].view(np.uint8))
    assert np.array_equal(got[:, N:].view(np.uint8), x_h[:, N:].view(np.uint8))


@pytest.mark.parametrize("shape", [(64, 8, 1), (64, 4, 2), (128, 8, 1), (256, 8, 1)])
def test_probe_two_inputs(shape):
    M, N = 64, 4096
    a_h = synth.random_rows(40100, M, N, dtype="bf16")
    b_h = synth.random_rows(40101, M, N, dtype="bf16")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    xr.probe_rows(out, to_device(a_h), to_device(b_h), threads=shape[0], vpt=shape[1],
                  split=shape[2])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out), a_h ^ b_h)


@pytest.mark.parametrize("nbytes,workgroups,threads", [
    (16 * 1000003, 7, 256),        # a ragged tail: fewer vectors than a whole unrolled pass
    (16 * (1 << 20), 1024, 512),   # whole unrolled passes
    (16 * 4099, 4096, 1024),       # more threads than vectors
    (16 * 123457, 0, 0),           # the runtime's device-to-device copy
])
def test_probe_copy_moves_exactly_its_bytes(nbytes, workgroups, threads):
    """xr_probe_copy: every byte of the source copied (or, in place, written back unchanged),
    nothing past the end written."""
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    dst = torch.full((nbytes // 4 + 64,), -7, dtype=torch.int32, device="cuda")
    xr.probe_copy(dst[:nbytes // 4], src, workgroups=workgroups, threads=threads or 256)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes // 4], src), "copy"
    assert bool((dst[nbytes // 4:] == -7).all()), "past the end"
    if workgroups:  # two inputs: their XOR
        src1 = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32,
                             device="cuda")
        xr.probe_copy(dst[:nbytes // 4], src, src1, workgroups=workgroups, threads=threads)
        torch.cuda.synchronize()
        assert torch.equal(dst[:nbytes // 4], src ^ src1), "xor of two inputs"
        assert bool((dst[nbytes // 4:] == -7).all()), "past the end"
        # in place: every vector read and written back unchanged, nothing past the end
        xr.probe_copy(dst[:nbytes // 4], dst[:nbytes // 4], workgroups=workgroups,
                      threads=threads)
        torch.cuda.synchronize()
        assert torch.equal(dst[:nbytes // 4], src ^ src1), "in place"
        assert bool((dst[nbytes // 4:] == -7).all()), "past the end"
