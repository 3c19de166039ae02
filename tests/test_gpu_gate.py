"""GPU parity of the optional layer interface (dt + dt_bias, softplus below
20, output gate y * silu(z)) in the chunked forward and the decode step,
through the C ABI, against the fp64 oracle with the same options."""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_amd import inputs as gen
from selective_state_space_amd import ssd

from _gpu import assert_close, compare_all_pairs, dev_tensor, host, log, upload_fwd

pytestmark = pytest.mark.gpu


BIG = 95.0   # e^95 overflows fp32: only the threshold keeps such a step finite


def raw_dt(shape, seed, n_big=0):
    """Pre-softplus steps: softplus(raw + bias) lands in about [3e-3, 0.13];
    n_big tokens of head 0 sit far above the threshold of 20."""
    rng = np.random.default_rng(seed)
    raw = rng.uniform(-6.0, -2.0, shape).astype(np.float32)
    if n_big:
        raw[0, 1:1 + n_big, 0] = BIG
    return raw


def gated_case(io, Bt, T, H, N, G, L, seed, bias=True, softplus=True, gate=True, n_big=0):
    inp = gen.make_small(Bt, T, H, 64, N, G, io, init_state=True, seed=seed)
    if softplus:
        raw = raw_dt(inp.dt.shape, seed + 1, n_big)
        b = np.linspace(-0.5, 0.5, H).astype(np.float32) if bias else None
    else:
        # without softplus the steps are used as given: keep them positive
        raw = inp.dt
        b = np.linspace(0.0, 0.05, H).astype(np.float32) if bias else None
    rng = np.random.default_rng(seed + 2)
    z = rng.normal(0.0, 1.5, inp.x.shape).astype(np.float32) if gate else None
    if gate and io == gen.BF16:
        z = gen.bf16_round(z)
    t = upload_fwd(inp, io)
    dt_t = dev_tensor(raw)
    z_t = None if z is None else dev_tensor(z, torch.bfloat16 if io == gen.BF16 else torch.float32)
    b_t = None if b is None else dev_tensor(b)
    y, fin = ssd.ssd_chunked_fwd(t["x"], dt_t, t["A"], t["B"], t["C"], t["D"], L,
                                 t["init_state"], dt_bias=b_t, dt_softplus=softplus, z=z_t)
    torch.cuda.synchronize()
    yr, fr, _ = oracle.token_fwd(inp.x, raw, inp.A, inp.B, inp.C, inp.D, inp.init_state,
                                 dt_bias=b, dt_softplus=softplus, z=z)
    yr = yr.reshape(Bt, H, T, 64).transpose(0, 2, 1, 3)
    return host(y), yr, host(fin), fr.reshape(Bt, H, 64, N)


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
@pytest.mark.parametrize("L,N", [(64, 64), (128, 128), (256, 128)])
@pytest.mark.parametrize("rows", ["", "0", "fused"])
def test_gated_forward(io, L, N, rows, force_path):
    """rows "" lets the library pick the path (the one-pass state stage for
    bf16); "0" forces the four stages, "fused" the fused pass (bf16 only; fp32
    ignores it)."""
    force_path(rows)
    T = 2 * L + 29
    log("gated forward", io, "L", L, "N", N, "rows", rows or "auto")
    # Steps above the threshold only in fp32: the step preparation is the same
    # for both io types, and a step of 95 would dwarf every other output, while
    # the bf16 bar is relative to their rms.
    y, yr, f, fr = gated_case(io, 2, T, 4, N, 2, L, seed=L + N,
                              n_big=2 if io == gen.F32 else 0)
    assert_close(y, yr, io, "y (gated)")
    assert_close(f, fr, io, "final")


@pytest.mark.parametrize("L,N,H", [(128, 64, 256), (256, 128, 128)])
def test_gated_forward_heads_per_workgroup(L, N, H):
    """Enough heads per group that each chunk_scan workgroup takes two of them
    in turn (the gate's LDS buffer is refilled for the second), with a ragged
    last chunk."""
    T = 2 * L + 29
    log("gated forward, two heads per workgroup: L", L, "N", N, "H", H)
    y, yr, f, fr = gated_case(gen.BF16, 1, T, H, N, 1, L, seed=7 * L + N)
    assert_close(y, yr, gen.BF16, "y (gated)")
    assert_close(f, fr, gen.BF16, "final")


@pytest.mark.parametrize("opt", ["bias", "softplus", "gate"])
def test_each_option_alone(opt):
    kw = dict(bias=opt == "bias", softplus=opt == "softplus", gate=opt == "gate")
    y, yr, f, fr = gated_case(gen.BF16, 2, 300, 8, 128, 2, 128, seed=11, **kw)
    assert_close(y, yr, gen.BF16, "y (%s)" % opt)
    assert_close(f, fr, gen.BF16, "final (%s)" % opt)


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_gated_decode(io):
    Bt, H, P, N, G, steps = 3, 8, 64, 128, 2, 5
    dt_ = torch.bfloat16 if io == gen.BF16 else torch.float32
    rng = np.random.default_rng(21)
    st0 = (rng.normal(0.0, 0.1, (Bt, H, P, N))).astype(np.float32)
    state = dev_tensor(st0)
    ref = st0.astype(np.float64).reshape(Bt * H, P, N).copy()
    A = -np.exp(rng.uniform(0.0, np.log(16.0), H)).astype(np.float32)
    D = rng.normal(0.0, 1.0, H).astype(np.float32)
    bias = np.linspace(-0.3, 0.3, H).astype(np.float32)
    for k in range(steps):
        x = rng.normal(0, 1, (Bt, H, P)).astype(np.float32)
        Bv = (rng.normal(0, 1, (Bt, G, N)) / np.sqrt(N)).astype(np.float32)
        Cv = (rng.normal(0, 1, (Bt, G, N)) / np.sqrt(N)).astype(np.float32)
        z = rng.normal(0, 1.5, (Bt, H, P)).astype(np.float32)
        raw = rng.uniform(-6.0, -2.0, (Bt, H)).astype(np.float32)
        if k == 2:
            raw[0, 0] = BIG                  # far above the softplus threshold
        if io == gen.BF16:
            x, Bv, Cv, z = map(gen.bf16_round, (x, Bv, Cv, z))
        y = ssd.ssd_decode_step(state, dev_tensor(x, dt_), dev_tensor(raw), dev_tensor(Bv, dt_),
                                dev_tensor(Cv, dt_), dev_tensor(A), dev_tensor(D),
                                dt_bias=dev_tensor(bias), dt_softplus=True, z_t=dev_tensor(z, dt_))
        yr = oracle.token_decode(ref, x, raw, Bv, Cv, A, D, dt_bias=bias, dt_softplus=True, z_t=z)
        torch.cuda.synchronize()
        assert_close(host(y).reshape(Bt * H, P), yr, io, "y_t step %d" % k)
    assert_close(host(state).reshape(Bt * H, P, N), ref, io, "state after %d steps" % steps)


def test_gated_full_size_all_pairs():
    """The 2.7B shape with all options, every (b, h) pair."""
    w = gen.WORKLOADS[2]
    inp = gen.make_fwd(w, 0)
    raw = raw_dt(inp.dt.shape, 5)
    b = np.linspace(-0.5, 0.5, w.nheads).astype(np.float32)
    z = gen.bf16_round(np.random.default_rng(8).normal(0, 1.5, inp.x.shape).astype(np.float32))
    t = upload_fwd(inp, w.io_dtype)
    y, fin = ssd.ssd_chunked_fwd(t["x"], dev_tensor(raw), t["A"], t["B"], t["C"], t["D"],
                                 w.chunk_size, t["init_state"], dt_bias=dev_tensor(b),
                                 dt_softplus=True, z=dev_tensor(z, torch.bfloat16))
    torch.cuda.synchronize()
    compare_all_pairs(oracle, inp, y, fin, gen.BF16, "gated 2.7B", dt=raw, dt_bias=b,
                      dt_softplus=True, z=z)
