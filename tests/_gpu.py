"""Helpers of the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, compare with the float64 oracle to the stated tolerances.

Tolerances:
* float32 path: normwise  max|gpu - ref| / max|ref| <= 1e-4, separately for
  y and for the final state;
* bf16-input path: max|gpu - ref| <= 2e-2 * rms(ref), separately for y and
  for the final state (rms over the compared elements of the oracle).
"""

import sys

import numpy as np
import torch

from selective_state_space_amd import inputs as gen

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(a, dtype=torch.float32):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dtype).cuda()


def upload_fwd(inp: gen.FwdInputs, io: str):
    dt = torch.bfloat16 if io == gen.BF16 else torch.float32
    return dict(
        x=dev_tensor(inp.x, dt), dt=dev_tensor(inp.dt), A=dev_tensor(inp.A),
        B=dev_tensor(inp.B, dt), C=dev_tensor(inp.C, dt), D=dev_tensor(inp.D),
        init_state=None if inp.init_state is None else dev_tensor(inp.init_state))


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def err_ratio(got, ref, io: str):
    """Error relative to the bar: <= 1 passes."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    d = float(np.max(np.abs(got - ref)))
    if not np.all(np.isfinite(got)):
        return float("inf")
    if io == gen.F32:
        return d / (TOL_F32 * max(float(np.max(np.abs(ref))), 1e-30))
    rms = float(np.sqrt(np.mean(ref * ref)))
    return d / (TOL_BF16 * max(rms, 1e-30))


def assert_close(got, ref, io: str, what: str):
    r = err_ratio(got, ref, io)
    log("  %-28s err/tol = %.4f" % (what, r))
    assert r <= 1.0, "%s: error is %.3fx the tolerance" % (what, r)


def assert_bf16_stored(got, ref, what: str):
    """A bf16 intermediate (h_prev) against its fp64 value: storing an fp32
    value as bf16 (round to nearest even) costs up to 2^-9 of it, so allow
    2^-8 |ref| per element, plus 2e-3 rms(ref) for the fp32 accumulation."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    rms = float(np.sqrt(np.mean(ref * ref)))
    excess = np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)
    r = float(np.max(excess)) / max(2e-3 * rms, 1e-30)
    log("  %-28s err/tol = %.4f (bf16 storage bound)" % (what, max(r, 0.0)))
    assert r <= 1.0, "%s: error is %.3fx the bf16 storage bound" % (what, r)
