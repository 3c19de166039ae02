"""GPU parity of the chunked forward (through the C ABI) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_amd import inputs as gen
from selective_state_space_amd import ssd

from _gpu import assert_close, host, log, upload_fwd

pytestmark = pytest.mark.gpu


def run_fwd(inp, io, L, init_override=None):
    t = upload_fwd(inp, io)
    init = t["init_state"] if init_override is None else init_override
    y, fin = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], L, init)
    torch.cuda.synchronize()
    return y, fin


def oracle_full(inp):
    y, fin, _ = oracle.token_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state)
    Bt, T, H, P = inp.x.shape
    return y.reshape(Bt, H, T, P).transpose(0, 2, 1, 3), fin.reshape(Bt, H, P, -1)


def test_tiny_fp32_workload():
    w = gen.WORKLOADS[0]
    log("workload", w.name)
    inp = gen.make_fwd(w, 0)
    y, fin = run_fwd(inp, w.io_dtype, w.chunk_size)
    yr, fr = oracle_full(inp)
    assert y.dtype == torch.float32  # y is fp32 for every input dtype
    assert_close(host(y), yr, gen.F32, "tiny fp32 y")
    assert_close(host(fin), fr, gen.F32, "tiny fp32 final")


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
@pytest.mark.parametrize("L", [64, 128, 256])
@pytest.mark.parametrize("N", [64, 128])
def test_small_shapes(io, L, N):
    T = 2 * L + 37                     # ragged last chunk
    log("small", io, "L", L, "N", N, "T", T)
    inp = gen.make_small(2, T, 4, 64, N, 2, io, init_state=True, seed=L + N)
    y, fin = run_fwd(inp, io, L)
    yr, fr = oracle_full(inp)
    assert_close(host(y), yr, io, "y")
    assert_close(host(fin), fr, io, "final")


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_single_chunk_and_short_sequences(io):
    for T in (1, 5, 63, 64, 65):
        inp = gen.make_small(1, T, 2, 64, 128, 1, io, init_state=True, seed=T)
        y, fin = run_fwd(inp, io, 64)
        yr, fr = oracle_full(inp)
        assert_close(host(y), yr, io, "y T=%d" % T)
        assert_close(host(fin), fr, io, "final T=%d" % T)


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_intermediates_against_chunked_reference(io):
    L, N, T = 64, 128, 200
    log("intermediates", io)
    inp = gen.make_small(2, T, 4, 64, N, 2, io, init_state=True, seed=31)
    t = upload_fwd(inp, io)
    a = ssd.FwdArgs(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], L, t["init_state"])
    ssd.ssd_chunk_cumsum(a)
    ssd.ssd_chunk_state(a)
    ssd.ssd_state_passing(a)
    ssd.ssd_chunk_scan(a)
    torch.cuda.synchronize()
    ws = ssd.workspace_views(a)
    ref = oracle.chunked_reference(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, L, inp.init_state)
    G = host(ws["G"])
    Gref = ref["G"] * np.log2(np.e)
    assert np.max(np.abs(G - Gref)) <= 2e-6 * max(1.0, np.max(np.abs(Gref)))
    nc = -(-T // L)
    dtp = np.zeros((2, nc * L, 4))
    dtp[:, :T] = inp.dt
    np.testing.assert_array_equal(host(ws["DT"]), dtp.reshape(2, nc, L, 4).transpose(0, 3, 1, 2))
    assert_close(host(ws["S"]), ref["S"], io, "S (chunk states)")
    assert_close(host(ws["h_prev"]), ref["h_prev"], io, "h_prev")
    assert_close(host(a.y), ref["y"], io, "y")
    assert_close(host(a.final), ref["final"], io, "final")


@pytest.mark.parametrize("io,path", [(gen.F32, "auto"), (gen.BF16, "0"), (gen.BF16, "4")])
def test_fused_call_equals_stage_calls_bitwise(io, path, monkeypatch):
    # ssd_chunked_fwd is cumsum, state + passing or the one-pass state stage, scan
    if path != "auto":
        monkeypatch.setenv("SSD_STATE_FWD_ROWS", path)
    inp = gen.make_small(2, 300, 8, 64, 128, 2, io, init_state=True, seed=37)
    t = upload_fwd(inp, io)
    y1, f1 = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 128,
                                 t["init_state"])
    a = ssd.FwdArgs(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 128, t["init_state"])
    mid = (ssd.ssd_state_fwd,) if path == "4" else (ssd.ssd_chunk_state, ssd.ssd_state_passing)
    for stage in (ssd.ssd_chunk_cumsum,) + mid + (ssd.ssd_chunk_scan,):
        stage(a)
    torch.cuda.synchronize()
    assert torch.equal(y1, a.y) and torch.equal(f1, a.final)


@pytest.mark.parametrize("rows", ["0", "4", "2", "1"])
def test_both_state_paths_against_oracle(rows, monkeypatch):
    # the same forward through the two stages and through each one-pass split
    monkeypatch.setenv("SSD_STATE_FWD_ROWS", rows)
    inp = gen.make_small(2, 3 * 128 + 21, 4, 64, 128, 2, gen.BF16, init_state=True, seed=83)
    y, fin = run_fwd(inp, gen.BF16, 128)
    yr, fr = oracle_full(inp)
    assert_close(host(y), yr, gen.BF16, "y rows=%s" % rows)
    assert_close(host(fin), fr, gen.BF16, "final rows=%s" % rows)


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_reruns_are_bitwise_identical(io):
    inp = gen.make_small(2, 520, 8, 64, 128, 4, io, init_state=True, seed=41)
    t = upload_fwd(inp, io)
    outs = [ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 256,
                                t["init_state"]) for _ in range(3)]
    torch.cuda.synchronize()
    for y, f in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(f, outs[0][1])


@pytest.mark.parametrize("rows", ["0", "4"])
def test_init_state_may_alias_final_state(rows, monkeypatch):
    monkeypatch.setenv("SSD_STATE_FWD_ROWS", rows)
    io = gen.BF16
    inp = gen.make_small(2, 256, 4, 64, 128, 1, io, init_state=True, seed=43)
    t = upload_fwd(inp, io)
    y1, f1 = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 64,
                                 t["init_state"])
    st = t["init_state"].clone()
    y2, f2 = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 64, st,
                                 final_state=st)
    torch.cuda.synchronize()
    assert f2.data_ptr() == st.data_ptr()
    assert torch.equal(y1, y2) and torch.equal(f1, st)


@pytest.mark.parametrize("io,rows", [(gen.F32, ""), (gen.BF16, "0"), (gen.BF16, "4")])
def test_chunk_aligned_split_equals_one_call(io, rows, monkeypatch):
    monkeypatch.setenv("SSD_STATE_FWD_ROWS", rows)
    L = 64
    inp = gen.make_small(2, 5 * L, 4, 64, 64, 2, io, init_state=True, seed=47)
    t = upload_fwd(inp, io)
    y, f = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], L,
                               t["init_state"])
    T1 = 2 * L
    sl = lambda k, a, b: t[k][:, a:b].contiguous()
    ya, fa = ssd.ssd_chunked_fwd(sl("x", 0, T1), sl("dt", 0, T1), t["A"], sl("B", 0, T1),
                                 sl("C", 0, T1), t["D"], L, t["init_state"])
    yb, fb = ssd.ssd_chunked_fwd(sl("x", T1, 5 * L), sl("dt", T1, 5 * L), t["A"],
                                 sl("B", T1, 5 * L), sl("C", T1, 5 * L), t["D"], L, fa)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([ya, yb], dim=1), y)
    assert torch.equal(fb, f)


@pytest.mark.parametrize("io,rows", [(gen.F32, ""), (gen.BF16, "0"), (gen.BF16, "4")])
def test_empty_sequence_passes_state_through(io, rows, monkeypatch):
    monkeypatch.setenv("SSD_STATE_FWD_ROWS", rows)
    dt = torch.bfloat16 if io == gen.BF16 else torch.float32
    x = torch.empty((2, 0, 4, 64), dtype=dt, device="cuda")
    B = torch.empty((2, 0, 1, 64), dtype=dt, device="cuda")
    dtt = torch.empty((2, 0, 4), device="cuda")
    A = -torch.ones(4, device="cuda")
    D = torch.ones(4, device="cuda")
    init = torch.randn(2, 4, 64, 64, device="cuda")
    y, f = ssd.ssd_chunked_fwd(x, dtt, A, B, B, D, 64, init)
    _, f0 = ssd.ssd_chunked_fwd(x, dtt, A, B, B, D, 64, None)
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(f, init)
    assert torch.count_nonzero(f0) == 0


def test_zero_dt_keeps_state():
    io = gen.BF16
    inp = gen.make_small(1, 200, 4, 64, 128, 2, io, init_state=True, seed=53)
    inp.dt[:] = 0
    y, fin = run_fwd(inp, io, 64)
    assert torch.equal(fin, torch.from_numpy(inp.init_state).cuda())


def test_no_decay_is_causal_linear_attention():
    # A = 0: y = ((C B^T) . M) diag(dt) X + D X, checked against the oracle
    io = gen.BF16
    inp = gen.make_small(1, 256, 4, 64, 64, 1, io, seed=59)
    inp.A[:] = 0
    y, fin = run_fwd(inp, io, 128)
    yr, fr = oracle_full(inp)
    assert_close(host(y), yr, io, "A=0 y")
    assert_close(host(fin), fr, io, "A=0 final")


def test_strong_decay_does_not_overflow():
    # exp2 of the masked (positive) exponents is huge; they must be discarded
    io = gen.BF16
    inp = gen.make_small(1, 256, 2, 64, 128, 1, io, seed=61)
    inp.A[:] = -2000.0
    inp.dt[:] = 0.5
    y, fin = run_fwd(inp, io, 256)
    yr, fr = oracle_full(inp)
    assert torch.isfinite(y.float()).all()
    assert_close(host(y), yr, io, "strong decay y")


# --- the full-size workloads, on sampled (b, h) pairs -------------------------------

def _sample_pairs(Bt, H, k, seed=0):
    rng = np.random.default_rng(seed)
    pr = {0, Bt * H - 1}
    while len(pr) < min(k, Bt * H):
        pr.add(int(rng.integers(Bt * H)))
    return sorted(pr)


def _check_sampled(w, inp, y, fin, npairs=12):
    Bt, T, H, P = inp.x.shape
    pairs = _sample_pairs(Bt, H, npairs)
    log("  oracle on %d sampled (b, h) pairs of %d" % (len(pairs), Bt * H))
    yr, fr, nth = oracle.token_fwd(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state,
                                   pairs=pairs)
    yg = np.stack([host(y[b, :, h]) for b, h in (divmod(p, H) for p in pairs)])
    fg = np.stack([host(fin[b, h]) for b, h in (divmod(p, H) for p in pairs)])
    assert_close(yg, yr, w.io_dtype, "%s y" % w.name)
    assert_close(fg, fr, w.io_dtype, "%s final" % w.name)


@pytest.mark.parametrize("idx,rows", [(1, ""), (1, "0"), (2, ""), (2, "0"), (3, "")])
def test_full_size_workload(idx, rows, monkeypatch):
    # rows "" = the path the shape selects (the one-pass state stage, with
    # two row sets per workgroup for 1 and 3 and all four for 2); "0" = the
    # two-stage state path
    monkeypatch.setenv("SSD_STATE_FWD_ROWS", rows)
    w = gen.WORKLOADS[idx]
    log("workload", w.name, w.description, "rows", rows or "auto")
    inp = gen.make_fwd(w, 0)
    t = upload_fwd(inp, w.io_dtype)
    y, fin = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], w.chunk_size,
                                 t["init_state"])
    torch.cuda.synchronize()
    _check_sampled(w, inp, y, fin)
    if idx == 3:
        # two halves of 32768 tokens in sequence give the same final state
        T1 = w.seqlen // 2
        sl = lambda k, a, b: t[k][:, a:b].contiguous()
        _, f1 = ssd.ssd_chunked_fwd(sl("x", 0, T1), sl("dt", 0, T1), t["A"], sl("B", 0, T1),
                                    sl("C", 0, T1), t["D"], w.chunk_size, None)
        y2, f2 = ssd.ssd_chunked_fwd(sl("x", T1, w.seqlen), sl("dt", T1, w.seqlen), t["A"],
                                     sl("B", T1, w.seqlen), sl("C", T1, w.seqlen), t["D"],
                                     w.chunk_size, f1)
        torch.cuda.synchronize()
        assert torch.equal(f2, fin), "split-halves final state differs from one call"
        assert torch.equal(y2, y[:, T1:]), "split-halves second-half y differs from one call"
        log("  two 32768-token halves reproduce the single call bitwise")
