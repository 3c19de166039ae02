"""ssd_chunked_fwd_noalloc (the forward on the library's static scratch, for
callers that cannot allocate) against ssd_chunked_fwd with a caller-allocated
workspace: the same kernels on the same inputs, so the outputs are equal bit
for bit.  Two calls in a row, the second smaller, then a shape past the
scratch's limit, which is refused before anything runs."""

import pytest
import torch

from selective_state_space_amd import inputs as gen
from selective_state_space_amd import ssd

from _gpu import log, upload_fwd

pytestmark = pytest.mark.gpu


def _both(inp, io, L, **kw):
    t = upload_fwd(inp, io)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], L, t["init_state"])
    y1, f1 = ssd.ssd_chunked_fwd(*args, **kw)
    y2, f2 = ssd.ssd_chunked_fwd_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return (y1, f1), (y2, f2)


def test_noalloc_equals_workspace_call_twice_then_smaller():
    # the 370M layer's shape (about 52 MB of workspace), then a smaller ragged
    # shape on the same scratch: the second call must not see the first's data
    w = gen.WORKLOADS[1]
    dims = ssd.fwd_dims(torch.empty(w.batch, w.seqlen, w.nheads, 64, dtype=torch.bfloat16),
                        torch.empty(w.batch, w.seqlen, w.ngroups, w.dstate, dtype=torch.bfloat16))
    need = ssd.ssd_chunked_fwd_workspace_size(dims, w.chunk_size)
    log("noalloc: 370M shape needs %d of %d scratch bytes" % (need, ssd.NOALLOC_SCRATCH_BYTES))
    assert need <= ssd.NOALLOC_SCRATCH_BYTES
    inp = gen.make_fwd(w, 0)
    (y1, f1), (y2, f2) = _both(inp, w.io_dtype, w.chunk_size)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    log("  call 1 (370M shape) bitwise equal")
    small = gen.make_small(2, 3 * 128 + 45, 8, 64, 128, 2, gen.BF16, init_state=True, seed=5)
    (y1, f1), (y2, f2) = _both(small, gen.BF16, 128)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    log("  call 2 (smaller, ragged) bitwise equal")
    # options on the scratch path too: gate and y in the io dtype
    z = torch.randn(small.x.shape, device="cuda").to(torch.bfloat16)
    (y1, f1), (y2, f2) = _both(small, gen.BF16, 64, z=z, y_io_dtype=True)
    assert y2.dtype == torch.bfloat16
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    log("  call 3 (gate, bf16 y) bitwise equal")


def test_noalloc_refuses_shapes_past_the_scratch():
    w = gen.WORKLOADS[2]   # the 2.7B layer: about 0.5 GB of workspace
    x = torch.zeros((w.batch, w.seqlen, w.nheads, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((w.batch, w.seqlen, 1, 128), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((w.batch, w.seqlen, w.nheads), device="cuda")
    A = torch.zeros(w.nheads, device="cuda")
    y = torch.full((w.batch, w.seqlen, w.nheads, 64), 7.0, device="cuda")
    with pytest.raises(ssd.SSDError) as e:
        ssd.ssd_chunked_fwd_noalloc(x, dt, A, B, B, A, 256, None, y=y)
    assert e.value.status == -5 and "scratch" in e.value.detail
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())   # nothing was written
