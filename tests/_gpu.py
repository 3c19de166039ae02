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


class Bar:
    """Accumulates max|gpu - ref|, max|ref| and sum(ref^2) over batches of
    compared elements, so a full-size output is checked against the bar with
    the rms of every element without holding all of it in float64 at once."""

    def __init__(self, io: str, what: str):
        self.io, self.what = io, what
        self.maxd = 0.0
        self.maxr = 0.0
        self.ss = 0.0
        self.n = 0
        self.finite = True

    def add(self, got, ref):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        if ref.size == 0:
            return
        self.finite = self.finite and bool(np.all(np.isfinite(got)))
        self.maxd = max(self.maxd, float(np.max(np.abs(got - ref))))
        self.maxr = max(self.maxr, float(np.max(np.abs(ref))))
        self.ss += float(np.sum(ref * ref))
        self.n += ref.size

    def ratio(self):
        if not self.finite:
            return float("inf")
        if self.n == 0:
            return 0.0
        if self.io == gen.F32:
            return self.maxd / (TOL_F32 * max(self.maxr, 1e-30))
        rms = (self.ss / self.n) ** 0.5
        return self.maxd / (TOL_BF16 * max(rms, 1e-30))

    def check(self, extra=""):
        r = self.ratio()
        log("  %-28s err/tol = %.4f over %d elements%s" % (self.what, r, self.n, extra))
        assert r <= 1.0, "%s: error is %.3fx the tolerance" % (self.what, r)


def row_pairs(Bt: int, H: int, nrows: int, seed: int = 0):
    """Every head of ``nrows`` batch rows (the first, the last and random others),
    as flat (b, h) pair indices b*H + h."""
    rng = np.random.default_rng(seed)
    rows = {0, Bt - 1}
    while len(rows) < min(nrows, Bt):
        rows.add(int(rng.integers(Bt)))
    return [b * H + h for b in sorted(rows) for h in range(H)]


def compare_all_pairs(oracle, inp, y, fin, io: str, name: str, pairs_per_batch: int = 64,
                      y_io: bool = False, dt=None, **opts):
    """Every (b, h) pair of a forward against the float64 oracle, streamed in
    batches of pairs: y (float32, or io dtype when y_io) and the final state
    to the bar of ``io``.  With y_io, y is also held per element to its own
    bf16 rounding: |y - ref| <= 2^-8 |ref| + the bar."""
    Bt, T, H, P = inp.x.shape
    npairs = Bt * H
    by, bf = Bar(io, "%s y" % name), Bar(io, "%s final" % name)
    yv = y.view(Bt, T, H, P)
    fv = fin.view(Bt * H, *fin.shape[2:])
    yref_abs_excess = 0.0
    for p0 in range(0, npairs, pairs_per_batch):
        pairs = list(range(p0, min(npairs, p0 + pairs_per_batch)))
        yr, fr, _ = oracle.token_fwd(inp.x, inp.dt if dt is None else dt, inp.A, inp.B, inp.C,
                                     inp.D, inp.init_state, pairs=pairs, **opts)
        bi = torch.tensor([p // H for p in pairs], device=y.device)
        hi = torch.tensor([p % H for p in pairs], device=y.device)
        yg = host(yv[bi, :, hi, :])                     # [npairs, T, P]
        by.add(yg, yr)
        if y_io:
            yref_abs_excess = max(yref_abs_excess,
                                  float(np.max(np.abs(yg - yr) - 2.0 ** -8 * np.abs(yr))))
        bf.add(host(fv[pairs[0]:pairs[-1] + 1]), fr)
    log("  %s: compared all %d of %d (b, h) pairs" % (name, len(range(npairs)), npairs))
    if y_io:
        rms = (by.ss / max(by.n, 1)) ** 0.5
        r = yref_abs_excess / (TOL_BF16 * max(rms, 1e-30))
        log("  %-28s err/tol = %.4f (bar plus the bf16 rounding of y)" % (name + " y (io dtype)",
                                                                        max(r, 0.0)))
        assert r <= 1.0, "%s y: error beyond its bf16 rounding is %.3fx the bar" % (name, r)
    else:
        by.check()
    bf.check()
    return by, bf
