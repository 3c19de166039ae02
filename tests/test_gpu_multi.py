"""GPU parity of the multi-token decode (per-step snapshots, the no-update
flag, draft-tree parents; "Optimizing Nemotron v3 Super in TensorRT-LLM",
sections 10.3 and 10.4), through the C ABI, against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from selective_state_space_amd import inputs as gen
from selective_state_space_amd import ssd

from _gpu import assert_close, dev_tensor, host, log, row_pairs

pytestmark = pytest.mark.gpu


def small(io, Bt, K, H, N, G, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (Bt, K, H, 64)).astype(np.float32)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (Bt, K, H))).astype(np.float32)
    B = (rng.normal(0, 1, (Bt, K, G, N)) / np.sqrt(N)).astype(np.float32)
    C = (rng.normal(0, 1, (Bt, K, G, N)) / np.sqrt(N)).astype(np.float32)
    A = -np.exp(rng.uniform(0.0, np.log(16.0), H)).astype(np.float32)
    D = rng.normal(0, 1, H).astype(np.float32)
    st = rng.normal(0, 0.1, (Bt, H, 64, N)).astype(np.float32)
    if io == gen.BF16:
        x, B, C = map(gen.bf16_round, (x, B, C))
    return x, dt, B, C, A, D, st


def run(io, x, dt, B, C, A, D, st, parent=None, update=True, snaps=True, **opt):
    dty = torch.bfloat16 if io == gen.BF16 else torch.float32
    s = dev_tensor(st)
    z = opt.pop("z", None)
    y, sn = ssd.ssd_decode_multi(
        s, dev_tensor(x, dty), dev_tensor(dt), dev_tensor(B, dty), dev_tensor(C, dty),
        dev_tensor(A), dev_tensor(D), snapshots=True if snaps else None,
        parent=None if parent is None else dev_tensor(parent, torch.int32),
        update_state=update, z=None if z is None else dev_tensor(z, dty),
        **{k: (dev_tensor(v) if isinstance(v, np.ndarray) else v) for k, v in opt.items()})
    torch.cuda.synchronize()
    return s, y, sn


def reference(x, dt, B, C, A, D, st, parent=None, update=True, **opt):
    Bt, K, H, P = x.shape
    ref = st.astype(np.float64).reshape(Bt * H, P, -1).copy()
    yr, sr = oracle.token_decode_multi(ref, x, dt, B, C, A, D, parent=parent,
                                       update_state=update, **opt)
    return ref, yr, sr


def compare(io, Bt, H, got, ref):
    s, y, sn = got
    rs, yr, sr = ref
    K, P = yr.shape[1], yr.shape[2]
    assert_close(host(y).transpose(0, 2, 1, 3).reshape(Bt * H, K, P), yr, io, "y (all steps)")
    if sn is not None:
        N = sr.shape[-1]
        assert_close(host(sn).transpose(0, 2, 1, 3, 4).reshape(Bt * H, K, P, N), sr, io,
                     "snapshots")
    assert_close(host(s).reshape(Bt * H, P, -1), rs, io, "state")


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
@pytest.mark.parametrize("N", [64, 128])
def test_chain(io, N):
    log("multi chain", io, "N", N)
    inp = small(io, 3, 5, 8, N, 2, seed=N)
    compare(io, 3, 8, run(io, *inp), reference(*inp))


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
def test_degenerate_decay(io):
    # heads from exp(-1000) per token to no decay (A = 0), and a token with
    # dt = 0 (the state is carried unchanged through it), on a chain and on a tree
    log("multi degenerate decay", io)
    Bt, K, H = 2, 5, 8
    x, dt, B, C, A, D, st = small(io, Bt, K, H, 128, 2, seed=23)
    A[:] = np.array([-2000.0, -30.0, -1.0, -1e-3, 0.0, 0.0, -1.0, -2000.0], np.float32)
    dt[:] = 0.5
    dt[:, 2] = 0.0
    inp = (x, dt, B, C, A, D, st)
    got = run(io, *inp)
    assert torch.isfinite(got[1].float()).all() and torch.isfinite(got[2]).all()
    compare(io, Bt, H, got, reference(*inp))
    par = np.array([[-1, 0, 0, 2, 1], [-1, 0, 1, 1, 3]], np.int32)
    compare(io, Bt, H, run(io, *inp, parent=par), reference(*inp, parent=par))


@pytest.mark.parametrize("io", [gen.F32, gen.BF16])
@pytest.mark.parametrize("update", [True, False])
def test_tree(io, update):
    log("multi tree", io, "update", update)
    Bt, K, H = 4, 7, 8
    inp = small(io, Bt, K, H, 128, 2, seed=5)
    rng = np.random.default_rng(17)
    par = np.array([[rng.integers(0, k) if k else -1 for k in range(K)] for _ in range(Bt)])
    par[3] = [-1, 1, 5, -7, 4, 6, 100]   # values that must be ignored
    got = run(io, *inp, parent=par.astype(np.int32), update=update)
    compare(io, Bt, H, got, reference(*inp, parent=par, update=update))
    if not update:   # the state is only read
        assert torch.equal(got[0].cpu(), torch.from_numpy(inp[-1]))


def test_layer_options_on_a_tree():
    log("multi tree with options")
    Bt, K, H = 2, 5, 8
    x, dt, B, C, A, D, st = small(gen.BF16, Bt, K, H, 128, 2, seed=9)
    rng = np.random.default_rng(4)
    raw = rng.uniform(-6.0, -2.0, dt.shape).astype(np.float32)
    bias = np.linspace(-0.3, 0.3, H).astype(np.float32)
    z = gen.bf16_round(rng.normal(0, 1.5, x.shape).astype(np.float32))
    par = np.array([[-1, 0, 0, 2, 1], [-1, 0, 1, 1, 3]])
    got = run(gen.BF16, x, raw, B, C, A, D, st, parent=par.astype(np.int32), dt_bias=bias,
              dt_softplus=True, z=z)
    ref = reference(x, raw, B, C, A, D, st, parent=par, dt_bias=bias, dt_softplus=True, z=z)
    compare(gen.BF16, Bt, H, got, ref)


def test_no_snapshots_same_results():
    inp = small(gen.BF16, 2, 6, 8, 128, 1, seed=2)
    s1, y1, _ = run(gen.BF16, *inp)
    s2, y2, sn = run(gen.BF16, *inp, snaps=False)
    assert sn is None
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


def test_matches_single_steps():
    """K tokens in one call against K calls of the single-token step."""
    Bt, K, H = 2, 4, 8
    x, dt, B, C, A, D, st = small(gen.BF16, Bt, K, H, 128, 2, seed=3)
    s1, y1, _ = run(gen.BF16, x, dt, B, C, A, D, st, snaps=False)
    s = dev_tensor(st)
    bf = torch.bfloat16
    for k in range(K):
        yk = ssd.ssd_decode_step(s, dev_tensor(x[:, k], bf), dev_tensor(dt[:, k]),
                                 dev_tensor(B[:, k], bf), dev_tensor(C[:, k], bf),
                                 dev_tensor(A), dev_tensor(D))
        d = (yk - y1[:, k]).abs().max().item()
        assert d <= 1e-6 * y1[:, k].abs().max().item(), (k, d)
    d = (s - s1).abs().max().item()
    assert d <= 1e-6 * s1.abs().max().item()


def test_zero_tokens_and_empty_batch():
    x, dt, B, C, A, D, st = small(gen.BF16, 2, 1, 8, 128, 2, seed=1)
    s, y, sn = run(gen.BF16, x[:, :0], dt[:, :0], B[:, :0], C[:, :0], A, D, st)
    assert torch.equal(s.cpu(), torch.from_numpy(st)) and y.numel() == 0


def test_verify_workload_full_size():
    """The multi-token decode workload at full size (snapshots, no state
    update), on every head of 8 batch rows (1024 of 32768 (b, h) pairs)."""
    w = gen.BY_NAME["mtp_verify_b256_k4"]
    prm = gen.decode_params(w, 0)
    m = gen.make_decode_multi(w, prm, 0)
    rng = np.random.default_rng(0)
    st = (rng.normal(0, 0.1, (w.batch, w.nheads, 64, w.dstate))).astype(np.float32)
    log("full-size multi-token decode", w.name)
    bf = torch.bfloat16
    s = dev_tensor(st)
    y, sn = ssd.ssd_decode_multi(s, dev_tensor(m.x, bf), dev_tensor(m.dt), dev_tensor(m.B, bf),
                                 dev_tensor(m.C, bf), dev_tensor(prm.A), dev_tensor(prm.D),
                                 snapshots=True, update_state=False)
    torch.cuda.synchronize()
    H = w.nheads
    pairs = row_pairs(w.batch, H, 8)
    log("  %d (b, h) pairs" % len(pairs))
    ref = st.reshape(-1, 64, w.dstate)[pairs].astype(np.float64)
    yr, sr = oracle.token_decode_multi(ref, m.x, m.dt, m.B, m.C, prm.A, prm.D, pairs=pairs,
                                       update_state=False)
    bi = torch.tensor([p // H for p in pairs], device=y.device)
    hi = torch.tensor([p % H for p in pairs], device=y.device)
    yg = host(y[bi, :, hi])
    sg = host(sn[bi, :, hi])
    assert_close(yg, yr, gen.BF16, "y (8 batch rows)")
    assert_close(sg, sr, gen.BF16, "snapshots (8 batch rows)")
    assert torch.equal(s.cpu(), torch.from_numpy(st))
