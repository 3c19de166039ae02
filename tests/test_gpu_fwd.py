"""GPU parity of the chunked forward (through the C ABI) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_amd import inputs as gen
from selective_state_space_amd import ssd

from _gpu import assert_close, compare_all_pairs, host, log, upload_fwd

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


@pytest.mark.parametrize("L", [64, 128, 256])
@pytest.mark.parametrize("N", [64, 128])
def test_small_shapes_fused_path(L, N, force_path):
    # every (L, N) instantiation of the fused pass, ragged last chunk, init state
    force_path("fused")
    T = 2 * L + 37
    log("small fused", "L", L, "N", N, "T", T)
    inp = gen.make_small(2, T, 4, 64, N, 2, gen.BF16, init_state=True, seed=L + N + 1)
    y, fin = run_fwd(inp, gen.BF16, L)
    yr, fr = oracle_full(inp)
    assert_close(host(y), yr, gen.BF16, "fused y")
    assert_close(host(fin), fr, gen.BF16, "fused final")


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
def test_whole_call_equals_stage_calls_bitwise(io, path, force_path):
    # ssd_chunked_fwd is cumsum, state + passing or the one-pass state stage, scan
    if path != "auto":
        force_path(path)
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


@pytest.mark.parametrize("rows", ["0", "4", "2", "1", "fused"])
def test_every_path_against_oracle(rows, force_path):
    # the same forward through the four stages, each one-pass split and the fused pass
    force_path(rows)
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


@pytest.mark.parametrize("rows", ["0", "4", "fused"])
def test_init_state_may_alias_final_state(rows, force_path):
    force_path(rows)
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


@pytest.mark.parametrize("io,rows", [(gen.F32, ""), (gen.BF16, "0"), (gen.BF16, "4"),
                                     (gen.BF16, "fused")])
def test_chunk_aligned_split_equals_one_call(io, rows, force_path):
    force_path(rows)
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


@pytest.mark.parametrize("io,rows", [(gen.F32, ""), (gen.BF16, "0"), (gen.BF16, "4"),
                                     (gen.BF16, "fused")])
def test_empty_sequence_passes_state_through(io, rows, force_path):
    force_path(rows)
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


PATHS = ["0", "4", "fused"]   # four stages, one-pass state stage, fused pass


@pytest.mark.parametrize("rows", PATHS)
@pytest.mark.parametrize("L", [64, 256])
def test_no_decay_is_causal_linear_attention(rows, L, force_path):
    # A = 0: y = ((C B^T) . M) diag(dt) X + D X, checked against the oracle
    force_path(rows)
    io = gen.BF16
    log("A = 0, path", rows, "L", L)
    inp = gen.make_small(1, 2 * L + 13, 4, 64, 64, 1, io, init_state=True, seed=59)
    inp.A[:] = 0
    y, fin = run_fwd(inp, io, L)
    yr, fr = oracle_full(inp)
    assert_close(host(y), yr, io, "A=0 y")
    assert_close(host(fin), fr, io, "A=0 final")


@pytest.mark.parametrize("rows", PATHS)
@pytest.mark.parametrize("L", [64, 256])
def test_strong_decay_does_not_overflow(rows, L, force_path):
    # exp2 of the masked (positive) exponents is huge; they must be discarded,
    # and heads from no decay to exp(-1000) per token share each launch
    force_path(rows)
    io = gen.BF16
    log("strong decay, path", rows, "L", L)
    inp = gen.make_small(1, 2 * L + 13, 4, 64, 128, 1, io, init_state=True, seed=61)
    inp.A[:] = np.array([-2000.0, -30.0, -1.0, -1e-3], np.float32)
    inp.dt[:] = 0.5
    y, fin = run_fwd(inp, io, L)
    yr, fr = oracle_full(inp)
    assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
    assert_close(host(y), yr, io, "strong decay y")
    assert_close(host(fin), fr, io, "strong decay final")


# --- the full-size workloads, every (b, h) pair ----------------------------------

@pytest.mark.parametrize("idx,rows", [(1, ""), (1, "0"), (1, "fused"), (2, ""), (2, "0"),
                                      (2, "fused"), (3, ""), (3, "fused")])
def test_full_size_workload(idx, rows, force_path):
    # rows "" = the path the shape selects (the one-pass state stage for
    # bf16); "0" = the four stages; "fused" = the fused pass
    force_path(rows)
    w = gen.WORKLOADS[idx]
    log("workload", w.name, w.description, "rows", rows or "auto")
    inp = gen.make_fwd(w, 0)
    t = upload_fwd(inp, w.io_dtype)
    y, fin = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], w.chunk_size,
                                 t["init_state"])
    torch.cuda.synchronize()
    compare_all_pairs(oracle, inp, y, fin, w.io_dtype, w.name,
                      pairs_per_batch=16 if idx == 3 else 64)
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


def test_full_size_y_in_io_dtype():
    # the 2.7B layer with y stored in bf16: the same call as the fp32 output
    # rounded to nearest even, and within the bar plus that rounding of the oracle
    w = gen.WORKLOADS[2]
    log("workload", w.name, "y in bf16")
    inp = gen.make_fwd(w, 0)
    t = upload_fwd(inp, w.io_dtype)
    y32, f32 = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                   w.chunk_size, t["init_state"])
    y16, f16 = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                   w.chunk_size, t["init_state"], y_io_dtype=True)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    assert torch.equal(y16, y32.to(torch.bfloat16)), "bf16 y is not the fp32 y rounded"
    assert torch.equal(f16, f32)
    compare_all_pairs(oracle, inp, y16, f16, w.io_dtype, w.name, y_io=True)


def test_stage_call_refuses_io_dtype_y():
    # the stage calls write y in float32: a y allocated in bf16 for the
    # y_io_dtype option is refused on the host, before anything is launched
    inp = gen.make_small(1, 64, 2, 64, 64, 1, gen.BF16, seed=3)
    t = upload_fwd(inp, gen.BF16)
    a = ssd.FwdArgs(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], 64, y_io_dtype=True)
    assert a.y.dtype == torch.bfloat16
    with pytest.raises(ValueError):
        ssd.ssd_chunk_scan(a)


@pytest.mark.parametrize("io,rows", [(gen.F32, ""), (gen.BF16, ""), (gen.BF16, "fused")])
def test_one_head_per_group(io, rows, force_path):
    # G = H: every head has its own B and C (no sharing across heads)
    force_path(rows)
    L = 128
    inp = gen.make_small(2, 3 * L + 11, 8, 64, 128, 8, io, init_state=True, seed=89)
    log("one head per group", io)
    y, fin = run_fwd(inp, io, L)
    yr, fr = oracle_full(inp)
    assert_close(host(y), yr, io, "G=H y")
    assert_close(host(fin), fr, io, "G=H final")


@pytest.mark.parametrize("rows", ["", "0", "fused"])
def test_partial_last_head_block(rows, force_path):
    # chunk_scan sizes its head blocks for about 256 workgroups: 3 sequences of
    # 3 chunks (one group) give blocks of 3 heads, so the last block of the 80
    # heads holds 2 (the ragged block); the other paths see the same inputs
    force_path(rows)
    Bt, T, H = 3, 2 * 256 + 19, 80
    inp = gen.make_small(Bt, T, H, 64, 128, 1, gen.BF16, init_state=True, seed=97)
    nc = -(-T // 256)
    groups = Bt * nc
    nh = max(1, min(H, -(-groups * H // 256)))
    assert H % nh != 0
    log("partial head block: heads per block", nh, "last block", H % nh)
    y, fin = run_fwd(inp, gen.BF16, 256)
    yr, fr = oracle_full(inp)
    assert_close(host(y), yr, gen.BF16, "partial head block y")
    assert_close(host(fin), fr, gen.BF16, "partial head block final")


@pytest.mark.parametrize("rows", ["", "0", "fused"])
@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("L,N", [(64, 64), (256, 128)])
def test_y_in_io_dtype_every_path(rows, gate, L, N, force_path):
    """y stored in bf16 (ssd_layer_opts.y_io_dtype) on every forward path,
    with and without the output gate: the same call's fp32 y rounded to
    nearest even, bit for bit (the output type is a template parameter of
    the kernels that store y, so each instantiation is exercised), and the
    final state unchanged."""
    force_path(rows)
    Bt, T, H, G = 2, 2 * L + 37, 8, 2
    inp = gen.make_small(Bt, T, H, 64, N, G, gen.BF16, init_state=True, seed=131 + L)
    t = upload_fwd(inp, gen.BF16)
    z = None
    if gate:
        rng = np.random.default_rng(7)
        z = torch.from_numpy(gen.bf16_round(rng.normal(0, 1.5, inp.x.shape).astype(np.float32)))
        z = z.to(torch.bfloat16).cuda()
    log("y in bf16: path", rows or "auto", "gate", gate, "L", L, "N", N)
    y32, f32 = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], L,
                                   t["init_state"], z=z)
    y16, f16 = ssd.ssd_chunked_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], L,
                                   t["init_state"], z=z, y_io_dtype=True)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    assert torch.equal(y16, y32.to(torch.bfloat16)), "bf16 y is not the fp32 y rounded"
    assert torch.equal(f16, f32)
