"""Pins of the oracle's multi-token decode with per-step snapshots, the
no-update flag and draft-tree parents ("Optimizing Nemotron v3 Super in
TensorRT-LLM", sections 10.3 and 10.4).

Every step k of a draft tree continues the sequence along its path to the
root: the state entering k is the one after step p(k) (the parent when it is
an earlier step, else k - 1).  So y_k and the snapshot of step k must equal
the plain forward recurrence run over the tokens of that path, started from
the initial state -- a different code path of the oracle (the sequence
forward in C), checked here for chains, stars, random trees and parents that
must be ignored.  A scalar case with no decay is checked in closed form."""

import numpy as np
import pytest

import oracle

RTOL = 1e-12


def case(Bt=2, K=5, H=4, P=4, N=6, G=2, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (Bt, K, H, P))
    dt = rng.uniform(0.01, 0.3, (Bt, K, H))
    B = rng.normal(0, 0.5, (Bt, K, G, N))
    C = rng.normal(0, 0.5, (Bt, K, G, N))
    A = -rng.uniform(0.5, 4.0, H)
    D = rng.normal(0, 1, H)
    st = rng.normal(0, 0.3, (Bt * H, P, N))
    return x, dt, B, C, A, D, st


def root_path(par, b, k):
    """Steps from the root to k: p(k) = par[b, k] if 0 <= par[b, k] < k, else k - 1."""
    path = [k]
    while k > 0:
        p = int(par[b, k]) if par is not None else k - 1
        k = p if 0 <= p < k else k - 1
        path.append(k)
    return path[::-1]


def check_against_paths(x, dt, B, C, A, D, st, par, y, snaps, **opt):
    Bt, K, H, P = x.shape
    z = opt.pop("z", None)
    for b in range(Bt):
        for k in range(K):
            path = root_path(par, b, k)
            sl = (slice(b, b + 1), path)
            init = st[b * H:(b + 1) * H].reshape(1, H, P, -1)
            yr, fr, _ = oracle.token_fwd(x[sl], dt[sl], A, B[sl], C[sl], D, init,
                                         z=None if z is None else z[sl], **opt)
            yr = yr.reshape(1, H, len(path), P)[0, :, -1]        # [H, P] at step k
            np.testing.assert_allclose(y[b * H:(b + 1) * H, k], yr, rtol=RTOL, atol=1e-12)
            np.testing.assert_allclose(snaps[b * H:(b + 1) * H, k], fr.reshape(H, P, -1),
                                       rtol=RTOL, atol=1e-12)


def test_chain_equals_forward():
    x, dt, B, C, A, D, st = case()
    s = st.copy()
    y, snaps = oracle.token_decode_multi(s, x, dt, B, C, A, D)
    check_against_paths(x, dt, B, C, A, D, st, None, y, snaps)
    np.testing.assert_array_equal(s, snaps[:, -1])


@pytest.mark.parametrize("kind", ["chain", "star", "random", "ignored"])
def test_tree_equals_forward_along_root_path(kind):
    Bt, K = 3, 7
    x, dt, B, C, A, D, st = case(Bt=Bt, K=K, seed=3)
    rng = np.random.default_rng(9)
    if kind == "chain":
        par = np.tile(np.arange(-1, K - 1), (Bt, 1))
    elif kind == "star":
        par = np.zeros((Bt, K), np.int64)
    elif kind == "random":
        par = np.array([[rng.integers(0, k) if k else -1 for k in range(K)] for _ in range(Bt)])
    else:   # negative, self and later parents: each step continues from k - 1
        par = np.array([[-1, 1, 5, -7, 4, 6, 100] for _ in range(Bt)])
    s = st.copy()
    y, snaps = oracle.token_decode_multi(s, x, dt, B, C, A, D, parent=par)
    check_against_paths(x, dt, B, C, A, D, st, par, y, snaps)
    np.testing.assert_array_equal(s, snaps[:, -1])
    if kind in ("chain", "ignored"):
        y0, s0 = oracle.token_decode_multi(st.copy(), x, dt, B, C, A, D)
        np.testing.assert_array_equal(y, y0)
        np.testing.assert_array_equal(snaps, s0)


def test_no_update_leaves_state_and_changes_nothing_else():
    x, dt, B, C, A, D, st = case(seed=5)
    par = np.array([[-1, 0, 1, 1, 0], [-1, 0, 0, 2, 3]])
    s1, s2 = st.copy(), st.copy()
    y1, n1 = oracle.token_decode_multi(s1, x, dt, B, C, A, D, parent=par)
    y2, n2 = oracle.token_decode_multi(s2, x, dt, B, C, A, D, parent=par, update_state=False)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(n1, n2)
    np.testing.assert_array_equal(s2, st)
    np.testing.assert_array_equal(s1, n1[:, -1])


def test_options_follow_the_path():
    x, dt, B, C, A, D, st = case(seed=7)
    rng = np.random.default_rng(1)
    raw = rng.uniform(-5, 1, dt.shape)
    raw[0, 2, 1] = 30.0                       # above the softplus threshold
    bias = rng.uniform(-0.5, 0.5, x.shape[2])
    z = rng.normal(0, 1.5, x.shape)
    par = np.array([[-1, 0, 0, 1, 3], [-1, 0, 1, 0, 2]])
    y, snaps = oracle.token_decode_multi(st.copy(), x, raw, B, C, A, D, parent=par,
                                         dt_bias=bias, dt_softplus=True, z=z)
    check_against_paths(x, raw, B, C, A, D, st, par, y, snaps, dt_bias=bias, dt_softplus=True,
                        z=z)


def test_pair_subset():
    x, dt, B, C, A, D, st = case(seed=11)
    par = np.array([[-1, 0, 1, 0, 3], [-1, 0, 0, 0, 0]])
    y, n = oracle.token_decode_multi(st.copy(), x, dt, B, C, A, D, parent=par)
    pr = [6, 1, 3]
    ys, ns = oracle.token_decode_multi(st[pr].copy(), x, dt, B, C, A, D, parent=par, pairs=pr)
    np.testing.assert_array_equal(ys, y[pr])
    np.testing.assert_array_equal(ns, n[pr])


def test_scalar_closed_form_without_decay():
    """P = N = H = 1, A = 0, dt = 1: the state after a path is s0 + sum x_j B_j
    over the path and y_k = state_k C_k + D x_k."""
    K = 6
    rng = np.random.default_rng(2)
    # inputs are float32 on both sides; the closed form uses the same values
    x, B, C = (rng.normal(0, 1, (1, K, 1, 1)).astype(np.float32).astype(np.float64)
               for _ in range(3))
    dt = np.ones((1, K, 1))
    s0, Dv = 0.7, 0.25
    par = np.array([[-1, 0, 0, 2, 1, 4]])
    st = np.full((1, 1, 1), s0)
    y, snaps = oracle.token_decode_multi(st, x, dt, B, C, np.zeros(1), np.array([Dv]),
                                         parent=par)
    paths = {0: [0], 1: [0, 1], 2: [0, 2], 3: [0, 2, 3], 4: [0, 1, 4], 5: [0, 1, 4, 5]}
    for k, path in paths.items():
        sk = s0 + sum(x[0, j, 0, 0] * B[0, j, 0, 0] for j in path)
        assert abs(snaps[0, k, 0, 0] - sk) < 1e-13
        assert abs(y[0, k, 0] - (sk * C[0, k, 0, 0] + Dv * x[0, k, 0, 0])) < 1e-13
    assert st[0, 0, 0] == snaps[0, K - 1, 0, 0]
