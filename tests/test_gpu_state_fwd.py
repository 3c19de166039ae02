"""GPU parity of the one-pass chunk_state + state_passing stage (ssd_state_fwd,
bf16 io) against the fp64 chunked reference, against the two separate stages,
and across its three row splits."""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_amd import inputs as gen
from selective_state_space_amd import ssd

from _gpu import assert_bf16_stored, assert_close, host, log, upload_fwd

pytestmark = pytest.mark.gpu

ROWS = [4, 2, 1]


def _state_fwd(t, L, rows, force_path, init=None):
    force_path(str(rows))
    a = ssd.FwdArgs(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], L,
                    t["init_state"] if init is None else init)
    ssd.ssd_chunk_cumsum(a)
    ssd.ssd_state_fwd(a)
    torch.cuda.synchronize()
    return a


@pytest.mark.parametrize("rows", ROWS)
@pytest.mark.parametrize("L", [64, 128, 256])
@pytest.mark.parametrize("N", [64, 128])
def test_state_fwd_against_chunked_reference(rows, L, N, force_path):
    T = 2 * L + 37                     # ragged last chunk
    log("state_fwd rows", rows, "L", L, "N", N, "T", T)
    inp = gen.make_small(2, T, 4, 64, N, 2, gen.BF16, init_state=True, seed=3 * L + N + rows)
    t = upload_fwd(inp, gen.BF16)
    a = _state_fwd(t, L, rows, force_path)
    ref = oracle.chunked_reference(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, L, inp.init_state)
    ws = ssd.workspace_views(a)
    assert_bf16_stored(host(ws["h_prev"]), ref["h_prev"], "h_prev")
    assert_close(host(a.final), ref["final"], gen.BF16, "final")


def test_row_splits_are_bitwise_identical(force_path):
    # a state element sees the same operands in the same order whatever the split
    inp = gen.make_small(3, 700, 8, 64, 128, 2, gen.BF16, init_state=True, seed=71)
    t = upload_fwd(inp, gen.BF16)
    outs = []
    for rows in ROWS:
        a = _state_fwd(t, 256, rows, force_path)
        outs.append((ssd.workspace_views(a)["h_prev"].clone(), a.final.clone()))
    for hp, f in outs[1:]:
        assert torch.equal(hp, outs[0][0]) and torch.equal(f, outs[0][1])


@pytest.mark.parametrize("rows", ROWS)
def test_state_fwd_matches_separate_stages(rows, force_path):
    # same per-chunk products (fp32 accumulation of the same bf16 operands);
    # only the order in which the decayed state joins the sum differs
    inp = gen.make_small(2, 1000, 8, 64, 128, 4, gen.BF16, init_state=True, seed=73)
    t = upload_fwd(inp, gen.BF16)
    a = _state_fwd(t, 256, rows, force_path)
    b = ssd.FwdArgs(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 256, t["init_state"])
    for stage in (ssd.ssd_chunk_cumsum, ssd.ssd_chunk_state, ssd.ssd_state_passing):
        stage(b)
    torch.cuda.synchronize()
    fa, fb = host(a.final), host(b.final)
    assert np.max(np.abs(fa - fb)) <= 1e-5 * np.max(np.abs(fb))
    ha, hb = host(ssd.workspace_views(a)["h_prev"]), host(ssd.workspace_views(b)["h_prev"])
    # bf16 roundings of nearly equal fp32 values differ by at most one ulp
    assert np.all(np.abs(ha - hb) <= 2.0 ** -7 * np.abs(hb) + 1e-30)


def test_zero_init_and_no_final(force_path):
    inp = gen.make_small(1, 300, 4, 64, 128, 1, gen.BF16, init_state=False, seed=79)
    t = upload_fwd(inp, gen.BF16)
    force_path("1")
    a = ssd.FwdArgs(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 128, None,
                    want_final=False)
    assert a.final is None
    ssd.ssd_chunk_cumsum(a)
    ssd.ssd_state_fwd(a)
    torch.cuda.synchronize()
    ref = oracle.chunked_reference(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, 128, None)
    hp = host(ssd.workspace_views(a)["h_prev"])
    assert np.count_nonzero(hp[:, :, 0]) == 0      # the state entering chunk 0 is zero
    assert_bf16_stored(hp, ref["h_prev"], "h_prev")
