"""GPU parity of the backward (ssd_chunked_bwd) through the C ABI against the
fp64 oracle's exact adjoint (the "mamba3" kernel card, section "Backward", for
the chunked order the GPU takes)."""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_amd import inputs as gen
from selective_state_space_amd import ssd

from _gpu import assert_close, dev_tensor, host, log, upload_fwd

pytestmark = pytest.mark.gpu

NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit")


def run_both(inp, io, L, dy, dfin, want_dinit=True):
    t = upload_fwd(inp, io)
    g = ssd.ssd_chunked_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], L, dev_tensor(dy),
                            t["init_state"], None if dfin is None else dev_tensor(dfin),
                            want_dinit=want_dinit)
    torch.cuda.synchronize()
    ref = oracle.token_bwd(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, dy, inp.init_state, dfin)
    return g, ref


def compare(g, ref, io, names=NAMES):
    for k in names:
        if g.get(k) is not None:
            assert_close(host(g[k]), ref[k], io, k)


def grads_inputs(inp, seed, dfinal=True):
    rng = np.random.default_rng(seed)
    dy = rng.normal(0, 1, inp.x.shape).astype(np.float32)
    Bt, T, H, P = inp.x.shape
    N = inp.B.shape[3]
    dfin = rng.normal(0, 1, (Bt, H, P, N)).astype(np.float32) if dfinal else None
    return dy, dfin


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
@pytest.mark.parametrize("L", [64, 128, 256])
@pytest.mark.parametrize("N", [64, 128])
def test_backward_against_oracle(io, L, N):
    log("bwd", io, "L", L, "N", N)
    inp = gen.make_small(2, 2 * L + 29, 4, 64, N, 2, io, init_state=True, seed=L + N)
    dy, dfin = grads_inputs(inp, 1)
    g, ref = run_both(inp, io, L, dy, dfin)
    compare(g, ref, io)


# --- the method's degenerate cases: decay so strong that exp underflows
# within a token, no decay at all (causal linear attention), and dt = 0 ----

@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
@pytest.mark.parametrize("L", [64, 256])
def test_backward_strong_decay(io, L):
    # heads from no decay to exp(-1000) per token: every factored decay and
    # the per-element diagonal ones must stay finite where exp2 underflows
    log("bwd strong decay", io, "L", L)
    inp = gen.make_small(1, 2 * L + 11, 4, 64, 128, 1, io, init_state=True, seed=71 + L)
    inp.A[:] = np.array([-2000.0, -30.0, -1.0, -1e-3], np.float32)
    inp.dt[:] = 0.5
    dy, dfin = grads_inputs(inp, 7)
    g, ref = run_both(inp, io, L, dy, dfin)
    for k in NAMES:
        assert torch.isfinite(g[k]).all(), k
    compare(g, ref, io)


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
@pytest.mark.parametrize("L", [64, 256])
def test_backward_no_decay(io, L):
    # A = 0: the forward is causal linear attention, every decay factor is 1
    log("bwd A = 0", io, "L", L)
    inp = gen.make_small(2, L + 37, 4, 64, 64, 2, io, init_state=True, seed=73 + L)
    inp.A[:] = 0
    dy, dfin = grads_inputs(inp, 9)
    g, ref = run_both(inp, io, L, dy, dfin)
    compare(g, ref, io)


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_backward_zero_dt(io):
    # dt = 0: the state stays init_state at every token, so y_t = C_t init +
    # D x_t, and in closed form dinit = dfinal + sum_t dy_t (outer) C_t and
    # dx = D dy; ddt, dA, dB and dC are still defined (against the oracle)
    log("bwd dt = 0", io)
    inp = gen.make_small(1, 300, 4, 64, 128, 2, io, init_state=True, seed=79)
    inp.dt[:] = 0
    dy, dfin = grads_inputs(inp, 11)
    g, ref = run_both(inp, io, 128, dy, dfin)
    compare(g, ref, io)
    H = inp.x.shape[2]
    Cg = np.repeat(inp.C.astype(np.float64), H // inp.C.shape[2], axis=2)   # [Bt, T, H, N]
    closed = dfin + np.einsum("bthp,bthn->bhpn", dy.astype(np.float64), Cg)
    assert_close(host(g["dinit"]), closed, io, "dinit closed form")
    assert_close(host(g["dx"]), dy * inp.D.reshape(1, 1, -1, 1), io, "dx = D dy")


@pytest.mark.parametrize("fwd_rows,adj_rows", [("0", ""), ("4", "1"), ("2", "2"), ("1", "4")])
@pytest.mark.parametrize("L", [64, 256])
def test_state_stage_paths(force_path, fwd_rows, adj_rows, L):
    """Every form of the recomputed forward states and of the state adjoint:
    chunk_state + state_passing with per-chunk adjoint sums and a separate
    reverse scan (rows 0), and the one-pass scans in both directions at each
    row split; the ragged last chunk and dfinal enter each."""
    force_path(fwd_rows, adj_rows)
    log("bwd state paths", fwd_rows, adj_rows, "L", L)
    inp = gen.make_small(2, 3 * L + 17, 8, 64, 128, 2, gen.BF16, init_state=True, seed=L + 3)
    dy, dfin = grads_inputs(inp, 5)
    g, ref = run_both(inp, gen.BF16, L, dy, dfin)
    compare(g, ref, gen.BF16)


def test_long_context_layout():
    """The long-context layer's head layout (128 heads in 8 groups of 16, N 128,
    chunk 256, bf16, one sequence) over its first 4096 tokens: every gradient,
    dB and dC summed over 16 heads per group."""
    log("bwd long-context layout, 4096 tokens")
    inp = gen.make_small(1, 4096, 128, 64, 128, 8, gen.BF16, init_state=False, seed=12)
    dy, dfin = grads_inputs(inp, 7)
    g, ref = run_both(inp, gen.BF16, 256, dy, dfin)
    compare(g, ref, gen.BF16)


@pytest.mark.parametrize("G", [1, 2, 8])
def test_group_counts(G):
    """dB and dC sum over the heads of a group: 8, 4 and 1 heads per group."""
    log("bwd groups", G)
    inp = gen.make_small(2, 300, 8, 64, 128, G, gen.BF16, init_state=True, seed=4)
    dy, dfin = grads_inputs(inp, 2)
    g, ref = run_both(inp, gen.BF16, 128, dy, dfin)
    compare(g, ref, gen.BF16)


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_without_init_and_dfinal(io):
    log("bwd no init, no dfinal", io)
    inp = gen.make_small(1, 200, 4, 64, 64, 1, io, init_state=False, seed=6)
    dy, _ = grads_inputs(inp, 3, dfinal=False)
    g, ref = run_both(inp, io, 64, dy, None)
    compare(g, ref, io)
    g2, _ = run_both(inp, io, 64, dy, None, want_dinit=False)
    assert g2["dinit"] is None
    for k in NAMES[:-1]:
        assert torch.equal(g[k], g2[k]), k


@pytest.mark.parametrize("H,G,T", [(8, 1, 700), (8, 8, 513), (6, 3, 1024), (12, 2, 300)])
def test_chunk256_heads_and_groups(H, G, T):
    """256-token chunks (the persistent dx kernel) over head and group
    counts, one head per group included, and ragged and whole last chunks."""
    log("bwd L256", "H", H, "G", G, "T", T)
    inp = gen.make_small(2, T, H, 64, 128, G, gen.BF16, init_state=True, seed=H + G + T)
    dy, dfin = grads_inputs(inp, 7)
    g, ref = run_both(inp, gen.BF16, 256, dy, dfin)
    compare(g, ref, gen.BF16)


@pytest.mark.parametrize("L", [128, 256])
def test_reruns_are_bitwise_identical(L):
    inp = gen.make_small(2, 333, 8, 64, 128, 2, gen.BF16, init_state=True, seed=8)
    dy, dfin = grads_inputs(inp, 4)
    t = upload_fwd(inp, gen.BF16)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], L, dev_tensor(dy), t["init_state"],
            dev_tensor(dfin))
    a = ssd.ssd_chunked_bwd(*args)
    b = ssd.ssd_chunked_bwd(*args)
    torch.cuda.synchronize()
    for k in NAMES:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_no_tokens(dtype):
    Bt, H, P, N = 2, 4, 64, 64
    x = torch.empty((Bt, 0, H, P), device="cuda", dtype=dtype)
    Bm = torch.empty((Bt, 0, 1, N), device="cuda", dtype=dtype)
    dt = torch.empty((Bt, 0, H), device="cuda")
    A = -torch.ones(H, device="cuda")
    D = torch.ones(H, device="cuda")
    dfin = torch.randn(Bt, H, P, N, device="cuda")
    g = ssd.ssd_chunked_bwd(x, dt, A, Bm, Bm, D, 64, torch.empty((Bt, 0, H, P), device="cuda"),
                            torch.randn(Bt, H, P, N, device="cuda"), dfin)
    torch.cuda.synchronize()
    assert torch.equal(g["dinit"], dfin)
    assert torch.count_nonzero(g["dA"]) == 0 and torch.count_nonzero(g["dD"]) == 0


@pytest.mark.parametrize("wi", [0, 1, 2])
def test_backward_full_size(wi):
    """The tiny fp32, 370M-shaped and 2.7B-shaped layers at their full sizes:
    every gradient against the oracle."""
    w = gen.WORKLOADS[wi]
    log("bwd full size", w.name)
    inp = gen.make_fwd(w, 0)
    dy, dfin = grads_inputs(inp, 5)
    g, ref = run_both(inp, w.io_dtype, w.chunk_size, dy, dfin)
    compare(g, ref, w.io_dtype)
