"""GPU parity of the decode step (through the C ABI) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_amd import inputs as gen
from selective_state_space_amd import ssd

from _gpu import assert_close, dev_tensor, host, log, row_pairs, upload_fwd

pytestmark = pytest.mark.gpu


def _tdt(io):
    return torch.bfloat16 if io == gen.BF16 else torch.float32


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
@pytest.mark.parametrize("N", [64, 128])
def test_decode_steps_against_oracle(io, N):
    w = gen.Workload("dec", 3, 1, 8, 64, N, 2, 64, io, kind="decode")
    prm = gen.decode_params(w, 1)
    rng = np.random.default_rng(5)
    st0 = (rng.standard_normal((3, 8, 64, N)) * 0.1).astype(np.float32)
    state = dev_tensor(st0)
    ref = st0.astype(np.float64).reshape(24, 64, N).copy()
    A, D = dev_tensor(prm.A), dev_tensor(prm.D)
    ys, yrs = [], []
    for k in range(6):
        s = gen.make_decode_step(w, k, prm, 1)
        y = ssd.ssd_decode_step(state, dev_tensor(s.x_t, _tdt(io)), dev_tensor(s.dt_t),
                                dev_tensor(s.B_t, _tdt(io)), dev_tensor(s.C_t, _tdt(io)), A, D)
        yr = oracle.token_decode(ref, s.x_t, s.dt_t, s.B_t, s.C_t, prm.A, prm.D)
        ys.append(host(y).reshape(24, 64))
        yrs.append(yr)
    torch.cuda.synchronize()
    assert_close(np.stack(ys), np.stack(yrs), io, "decode y (6 steps)")
    assert_close(host(state).reshape(24, 64, N), ref, io, "decode state")


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_decode_degenerate_decay(io):
    # heads from exp(-1000) per token (the state is replaced each step) to no
    # decay (A = 0), and one step with dt = 0 everywhere (the state is kept)
    w = gen.Workload("dec", 2, 1, 8, 64, 128, 2, 64, io, kind="decode")
    prm = gen.decode_params(w, 3)
    prm.A[:] = np.array([-2000.0, -30.0, -1.0, -1e-3, 0.0, 0.0, -1.0, -2000.0], np.float32)
    rng = np.random.default_rng(13)
    st0 = (rng.standard_normal((2, 8, 64, 128)) * 0.1).astype(np.float32)
    state = dev_tensor(st0)
    ref = st0.astype(np.float64).reshape(16, 64, 128).copy()
    A, D = dev_tensor(prm.A), dev_tensor(prm.D)
    ys, yrs = [], []
    for k in range(5):
        s = gen.make_decode_step(w, k, prm, 3)
        if k == 2:
            s.dt_t[:] = 0
        else:
            s.dt_t[:] = 0.5
        y = ssd.ssd_decode_step(state, dev_tensor(s.x_t, _tdt(io)), dev_tensor(s.dt_t),
                                dev_tensor(s.B_t, _tdt(io)), dev_tensor(s.C_t, _tdt(io)), A, D)
        yr = oracle.token_decode(ref, s.x_t, s.dt_t, s.B_t, s.C_t, prm.A, prm.D)
        ys.append(host(y).reshape(16, 64))
        yrs.append(yr)
    torch.cuda.synchronize()
    assert torch.isfinite(state).all()
    assert_close(np.stack(ys), np.stack(yrs), io, "degenerate decay y (5 steps)")
    assert_close(host(state).reshape(16, 64, 128), ref, io, "degenerate decay state")


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_decode_steps_equal_forward(io):
    # T decode steps from h0 == one chunked forward over the same T tokens
    T = 40
    inp = gen.make_small(2, T, 4, 64, 128, 2, io, init_state=True, seed=67)
    t = upload_fwd(inp, io)
    y, fin = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 64,
                                 t["init_state"])
    state = t["init_state"].clone()
    ys = [ssd.ssd_decode_step(state, t["x"][:, k].contiguous(), t["dt"][:, k].contiguous(),
                              t["B"][:, k].contiguous(), t["C"][:, k].contiguous(), t["A"],
                              t["D"]) for k in range(T)]
    torch.cuda.synchronize()
    yd = torch.stack(ys, dim=1)
    yr, fr, _ = oracle.token_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state)
    yr = yr.reshape(2, 4, T, 64).transpose(0, 2, 1, 3)
    assert_close(host(yd), yr, io, "decode y vs oracle")
    assert_close(host(state), fr.reshape(2, 4, 64, 128), io, "decode state vs oracle")
    assert_close(host(yd), host(y), io, "decode y vs GPU forward")


def test_decode_is_deterministic():
    io = gen.BF16
    w = gen.Workload("dec", 4, 1, 16, 64, 128, 4, 64, io, kind="decode")
    prm = gen.decode_params(w, 2)
    s = gen.make_decode_step(w, 0, prm, 2)
    args = (dev_tensor(s.x_t, torch.bfloat16), dev_tensor(s.dt_t),
            dev_tensor(s.B_t, torch.bfloat16), dev_tensor(s.C_t, torch.bfloat16),
            dev_tensor(prm.A), dev_tensor(prm.D))
    st0 = torch.randn(4, 16, 64, 128, device="cuda")
    a, b = st0.clone(), st0.clone()
    ya = ssd.ssd_decode_step(a, *args)
    yb = ssd.ssd_decode_step(b, *args)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ya, yb)


def test_decode_full_size_512_steps():
    w = gen.WORKLOADS[4]
    log("workload", w.name, w.description)
    Bt, H, P, N = w.batch, w.nheads, w.headdim, w.dstate
    prm = gen.decode_params(w, 0)
    state = torch.zeros((Bt, H, P, N), device="cuda")
    A, D = dev_tensor(prm.A), dev_tensor(prm.D)
    pairs = row_pairs(Bt, H, 16)   # every head of 16 batch rows: 2048 of 32768 pairs
    log("  %d (b, h) pairs" % len(pairs))
    ref = np.zeros((len(pairs), P, N))
    ys, yrs = [], []
    for k in range(w.steps):
        s = gen.make_decode_step(w, k, prm, 0)
        y = ssd.ssd_decode_step(state, dev_tensor(s.x_t, torch.bfloat16), dev_tensor(s.dt_t),
                                dev_tensor(s.B_t, torch.bfloat16),
                                dev_tensor(s.C_t, torch.bfloat16), A, D)
        yr = oracle.token_decode(ref, s.x_t, s.dt_t, s.B_t, s.C_t, prm.A, prm.D, pairs=pairs)
        yh = host(y).reshape(Bt * H, P)[pairs]
        ys.append(yh)
        yrs.append(yr)
        if k % 128 == 0:
            log("  step", k)
    torch.cuda.synchronize()
    assert_close(np.stack(ys), np.stack(yrs), w.io_dtype, "decode y, 512 steps")
    del ys, yrs
    fg = host(state).reshape(Bt * H, P, N)[pairs]
    assert_close(fg, ref, w.io_dtype, "decode state after 512 steps")


def test_y_in_io_dtype_is_the_rounded_float32_output():
    # y_t stored in bf16 (ssd_layer_opts.y_io_dtype): the fp32 output of the
    # same step rounded to nearest even, for the plain step, the multi-token
    # call and a 16-bit state
    io = gen.BF16
    w = gen.Workload("dec", 3, 1, 8, 64, 128, 2, 64, io, kind="decode")
    prm = gen.decode_params(w, 5)
    s = gen.make_decode_step(w, 0, prm, 5)
    bf = torch.bfloat16
    args = (dev_tensor(s.x_t, bf), dev_tensor(s.dt_t), dev_tensor(s.B_t, bf),
            dev_tensor(s.C_t, bf), dev_tensor(prm.A), dev_tensor(prm.D))
    st0 = torch.randn(3, 8, 64, 128, device="cuda")
    a, b = st0.clone(), st0.clone()
    y32 = ssd.ssd_decode_step(a, *args)
    y16 = ssd.ssd_decode_step(b, *args, y_io_dtype=True)
    torch.cuda.synchronize()
    assert y16.dtype == bf and torch.equal(y16, y32.to(bf)) and torch.equal(a, b)
    xk, dk, Bk, Ck = (t.unsqueeze(1).repeat(1, 3, *([1] * (t.dim() - 1))) for t in args[:4])
    a, b = st0.clone(), st0.clone()
    m32, _ = ssd.ssd_decode_multi(a, xk, dk, Bk, Ck, args[4], args[5])
    m16, _ = ssd.ssd_decode_multi(b, xk, dk, Bk, Ck, args[4], args[5], y_io_dtype=True)
    torch.cuda.synchronize()
    assert m16.dtype == bf and torch.equal(m16, m32.to(bf)) and torch.equal(a, b)
    a, b = st0.to(bf), st0.to(bf)
    l32 = ssd.ssd_decode_step_lp(a, *args, "bf16")
    l16 = ssd.ssd_decode_step_lp(b, *args, "bf16", y_io_dtype=True)
    torch.cuda.synchronize()
    assert l16.dtype == bf and torch.equal(l16, l32.to(bf)) and torch.equal(a, b)
