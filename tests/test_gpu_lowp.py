"""GPU parity of the decode step on a 16-bit state ("Optimizing Nemotron v3
Super in TensorRT-LLM", section 6.5): fp16 (nearest and stochastic), bf16 and
int16 with row scales, through the C ABI, against the oracle.

Both sides start from the same stored state and store with the same rule;
they differ only where the fp32 value that decides a rounding differs in its
last bit (the GPU updates in fp32, the oracle in fp64 rounded to fp32).  So
after one step the stored values must agree bit for bit almost everywhere
and within one unit of the format elsewhere; over several steps y and the
state must stay within the benchmark's tolerance of the oracle."""

import numpy as np
import pytest
import torch

from oracle import state_formats as sf
from selective_state_space_amd import inputs as gen
from selective_state_space_amd import ssd

from _gpu import TOL_BF16, TOL_F32, assert_close, dev_tensor, host, log, row_pairs

pytestmark = pytest.mark.gpu

FORMATS = [("f16", False), ("f16", True), ("bf16", False), ("int16", False)]
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "int16": torch.int16}


def initial_state(fmt, shape, seed):
    """A random state as the format stores it: (device tensor, device scales or
    None, decoded float64 values)."""
    v = np.random.default_rng(seed).normal(0, 0.3, shape)
    vals, extra = sf.encode_state(v, fmt)
    if fmt == "int16":
        codes, dec = extra
        return dev_tensor(codes, torch.int16), dev_tensor(dec), vals
    return dev_tensor(vals.astype(np.float32), TORCH[fmt]), None, vals


def decoded(fmt, st, scale):
    if fmt == "int16":
        return (st.float() * scale[..., None]).double().cpu().numpy()
    return host(st)


def step_inputs(rng, Bt, H, P, N, G, io):
    x = rng.normal(0, 1, (Bt, H, P)).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (Bt, H))).astype(np.float32)
    B = (rng.normal(0, 1, (Bt, G, N)) / np.sqrt(N)).astype(np.float32)
    C = (rng.normal(0, 1, (Bt, G, N)) / np.sqrt(N)).astype(np.float32)
    if io == gen.BF16:
        x, B, C = map(gen.bf16_round, (x, B, C))
    return x, dt, B, C


def unit(fmt, vals, scale_np=None):
    """One unit of the stored format at each value (fp16 / bf16 ulp, or the
    row's decode scale for int16)."""
    a = np.abs(vals)
    if fmt == "f16":
        return sf._ulp16(a)
    if fmt == "bf16":
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)
    return np.broadcast_to(scale_np[..., None], vals.shape)


@pytest.mark.parametrize("fmt,stoch", FORMATS)
@pytest.mark.parametrize("N", [64, 128])
def test_one_step_bits(fmt, stoch, N):
    Bt, H, P, G, io = 3, 8, 64, 2, gen.BF16
    log("lowp one step", fmt, "stochastic" if stoch else "", "N", N)
    st, scale, vals = initial_state(fmt, (Bt, H, P, N), seed=N)
    rng = np.random.default_rng(1)
    A = -np.exp(rng.uniform(0, np.log(16), H)).astype(np.float32)
    D = rng.normal(0, 1, H).astype(np.float32)
    x, dt, B, C = step_inputs(rng, Bt, H, P, N, G, io)
    bf = torch.bfloat16
    y = ssd.ssd_decode_step_lp(st, dev_tensor(x, bf), dev_tensor(dt), dev_tensor(B, bf),
                               dev_tensor(C, bf), dev_tensor(A), dev_tensor(D), fmt, scale=scale,
                               philox_rounds=10 * stoch, seed=0xDEADBEEF12345)
    torch.cuda.synchronize()
    yr, new, extra = sf.decode_step_lowp(vals, x, dt, B, C, A, D, fmt, seed=0xDEADBEEF12345,
                                         philox_rounds=10 * stoch)
    assert_close(host(y), yr, io, "y")
    got = decoded(fmt, st, scale)
    if fmt == "int16":
        codes, dec = extra
        dc = np.abs(st.cpu().numpy().astype(np.int64) - codes.astype(np.int64))
        frac = float(np.mean(dc != 0))
        log("  int16 codes differing: %.2e (max %d)" % (frac, dc.max()))
        assert dc.max() <= 1 and frac < 1e-3
        rs = np.abs(scale.cpu().numpy().astype(np.float64) / dec - 1)
        assert rs.max() <= 2.0 ** -22
    else:
        diff = got != new
        frac = float(np.mean(diff))
        log("  stored values differing: %.2e" % frac)
        assert frac < 1e-3
        assert np.all(np.abs(got - new) <= unit(fmt, new) * (1 + 1e-9))


@pytest.mark.parametrize("fmt,stoch", FORMATS)
def test_degenerate_rows(fmt, stoch):
    # heads 0 and 3 decay by exp(-1000) (the old state vanishes) and have x = 0
    # on rows 0..7 of head 0, so those rows become exactly zero (int16: codes 0
    # and decode scale 0); head 1 has A = 0, head 2 dt = 0 (the state is kept)
    Bt, H, P, N, G, io = 2, 4, 64, 128, 2, gen.BF16
    log("lowp degenerate rows", fmt, "stochastic" if stoch else "")
    st, scale, vals = initial_state(fmt, (Bt, H, P, N), seed=17)
    rng = np.random.default_rng(3)
    A = np.array([-2000.0, 0.0, -1.0, -2000.0], np.float32)
    D = rng.normal(0, 1, H).astype(np.float32)
    x, dt, B, C = step_inputs(rng, Bt, H, P, N, G, io)
    dt[:] = np.array([0.5, 0.5, 0.0, 0.5], np.float32)
    x[:, 0, :8] = 0
    bf = torch.bfloat16
    y = ssd.ssd_decode_step_lp(st, dev_tensor(x, bf), dev_tensor(dt), dev_tensor(B, bf),
                               dev_tensor(C, bf), dev_tensor(A), dev_tensor(D), fmt, scale=scale,
                               philox_rounds=10 * stoch, seed=77)
    torch.cuda.synchronize()
    yr, new, extra = sf.decode_step_lowp(vals, x, dt, B, C, A, D, fmt, seed=77,
                                         philox_rounds=10 * stoch)
    assert_close(host(y), yr, io, "y")
    got = decoded(fmt, st, scale)
    assert np.all(np.isfinite(got))
    assert np.all(got[:, 0, :8] == 0) and np.all(new[:, 0, :8] == 0), "zero rows"
    if fmt == "int16":
        codes, dec = extra
        assert np.all(scale.cpu().numpy()[:, 0, :8] == 0) and np.all(dec[:, 0, :8] == 0)
        dc = np.abs(st.cpu().numpy().astype(np.int64) - codes.astype(np.int64))
        assert dc.max() <= 1 and float(np.mean(dc != 0)) < 1e-3
    else:
        assert float(np.mean(got != new)) < 1e-3
        assert np.all(np.abs(got - new) <= unit(fmt, new) * (1 + 1e-9))


@pytest.mark.parametrize("fmt,stoch", FORMATS)
@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_steps_against_oracle(fmt, stoch, io):
    Bt, H, P, N, G, steps = 2, 8, 64, 128, 2, 6
    log("lowp steps", fmt, "stochastic" if stoch else "", io)
    st, scale, vals = initial_state(fmt, (Bt, H, P, N), seed=7)
    rng = np.random.default_rng(2)
    A = -np.exp(rng.uniform(0, np.log(16), H)).astype(np.float32)
    D = rng.normal(0, 1, H).astype(np.float32)
    bias = np.linspace(-0.2, 0.2, H).astype(np.float32)
    dty = torch.bfloat16 if io == gen.BF16 else torch.float32
    ref = vals
    units = np.zeros_like(vals)      # running sum of the format's unit at each step
    for k in range(steps):
        x, dt, B, C = step_inputs(rng, Bt, H, P, N, G, io)
        raw = np.log(np.expm1(dt.astype(np.float64))).astype(np.float32) - bias
        z = rng.normal(0, 1.5, x.shape).astype(np.float32)
        if io == gen.BF16:
            z = gen.bf16_round(z)
        gate = k % 2 == 1          # every other step with the layer options
        kw = dict(dt_bias=bias, dt_softplus=True, z_t=z) if gate else {}
        y = ssd.ssd_decode_step_lp(
            st, dev_tensor(x, dty), dev_tensor(raw if gate else dt), dev_tensor(B, dty),
            dev_tensor(C, dty), dev_tensor(A), dev_tensor(D), fmt, scale=scale,
            philox_rounds=10 * stoch, seed=1000 + k,
            **{a: (dev_tensor(v, dty) if a == "z_t" else dev_tensor(v) if isinstance(v, np.ndarray)
                   else v) for a, v in kw.items()})
        yr, ref, extra = sf.decode_step_lowp(ref, x, raw if gate else dt, B, C, A, D, fmt,
                                             seed=1000 + k, philox_rounds=10 * stoch, **kw)
        torch.cuda.synchronize()
        # y reads the stored state of the previous step: each element may be
        # off by its accumulated units, which moves y by up to sum_n |C_n| units
        Cg = np.repeat(np.abs(C.astype(np.float64)), H // G, axis=1)       # [Bt,H,N]
        slack = np.einsum("bhn,bhpn->bhp", Cg, units)
        base = (TOL_F32 * np.max(np.abs(yr)) if io == gen.F32
                else TOL_BF16 * np.sqrt(np.mean(yr * yr)))
        d = np.abs(host(y) - yr)
        log("  y step %d: max |diff| / (bar + state slack) = %.3f"
            % (k, float(np.max(d / (base + slack)))))
        assert np.all(d <= base + slack)
        units += unit(fmt, ref, None if extra is None else extra[1])
    # The update is elementwise in the state, so a rounding decided the other
    # way stays in its element, decaying: after S steps each element is within
    # the sum of the S units of its format (the fp32 bar would be below one
    # fp16 unit).
    got = decoded(fmt, st, scale)
    excess = np.abs(got - ref) - units * (1 + 1e-6)
    log("  state: max |diff| / sum of units = %.3f"
        % float(np.max(np.abs(got - ref) / np.maximum(units, 1e-30))))
    assert np.all(excess <= 1e-7 * np.sqrt(np.mean(ref * ref)))


@pytest.mark.parametrize("fmt,stoch", [("f16", True), ("int16", False)])
def test_full_size_rows(fmt, stoch):
    """decode_b256's shape on a 16-bit state, 2 steps, every head of 8 batch
    rows (1024 of 32768 (b, h) pairs)."""
    w = gen.WORKLOADS[4]
    Bt, H, P, N = w.batch, w.nheads, w.headdim, w.dstate
    log("lowp full size", fmt)
    st, scale, vals = initial_state(fmt, (Bt, H, P, N), seed=3)
    prm = gen.decode_params(w, 0)
    pairs = row_pairs(Bt, H, 8)
    ref = vals.reshape(-1, P, N)[pairs]
    del vals
    bf = torch.bfloat16
    for k in range(2):
        s = gen.make_decode_step(w, k, prm, 0)
        y = ssd.ssd_decode_step_lp(st, dev_tensor(s.x_t, bf), dev_tensor(s.dt_t),
                                   dev_tensor(s.B_t, bf), dev_tensor(s.C_t, bf),
                                   dev_tensor(prm.A), dev_tensor(prm.D), fmt, scale=scale,
                                   philox_rounds=10 * stoch, seed=77 + k)
        yr, ref, _ = sf.decode_step_lowp(ref, s.x_t, s.dt_t, s.B_t, s.C_t, prm.A, prm.D, fmt,
                                         seed=77 + k, philox_rounds=10 * stoch, pairs=pairs)
        torch.cuda.synchronize()
        yg = host(y).reshape(-1, P)[pairs]
        assert_close(yg, yr, gen.BF16, "y step %d (8 batch rows)" % k)
    got = decoded(fmt, st, scale).reshape(-1, P, N)[pairs]
    assert_close(got, ref, gen.BF16, "state (8 batch rows)")
