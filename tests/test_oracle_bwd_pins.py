"""Pins of the oracle's backward: the exact adjoint of the recurrence
(the "mamba3" kernel card, section "Backward", for the chunked order; the values
are those of the chain rule on the token recurrence).

Each gradient is checked against central differences of the forward oracle
(a separate code path) along random directions: for a loss
L = sum(dy * y) + sum(dfinal * final), <grad, v> must equal
(L(theta + v) - L(theta - v)) / 2 up to the third-order term.  The
perturbed float32 inputs are formed first and their exact difference is the
direction used, so input rounding does not enter."""

import numpy as np
import pytest

import oracle


def problem(Bt=2, T=7, H=4, P=3, N=5, G=2, seed=0, init=True):
    rng = np.random.default_rng(seed)
    f = lambda *s, scale=1.0: (rng.normal(0, scale, s)).astype(np.float32)
    th = dict(x=f(Bt, T, H, P), dt=rng.uniform(0.05, 0.6, (Bt, T, H)).astype(np.float32),
              A=(-rng.uniform(0.3, 2.0, H)).astype(np.float32), B=f(Bt, T, G, N, scale=0.5),
              C=f(Bt, T, G, N, scale=0.5), D=f(H),
              init=rng.normal(0, 0.5, (Bt, H, P, N)) if init else None)
    dy = f(Bt, T, H, P)
    dfin = f(Bt, H, P, N)
    return th, dy, dfin


def loss(th, dy, dfin):
    Bt, T, H, P = th["x"].shape
    N = th["B"].shape[3]
    y, fin, _ = oracle.token_fwd(th["x"], th["dt"], th["A"], th["B"], th["C"], th["D"],
                                 th["init"])
    y = y.reshape(Bt, H, T, P).transpose(0, 2, 1, 3)
    L = float(np.sum(dy.astype(np.float64) * y))
    if dfin is not None:
        L += float(np.sum(dfin.astype(np.float64) * fin.reshape(Bt, H, P, N)))
    return L


GRAD = dict(x="dx", dt="ddt", A="dA", B="dB", C="dC", D="dD", init="dinit")


@pytest.mark.parametrize("name", list(GRAD))
@pytest.mark.parametrize("with_dfinal", [True, False])
def test_directional_derivatives(name, with_dfinal):
    th, dy, dfin = problem(seed=3)
    dfin = dfin if with_dfinal else None
    grads = oracle.token_bwd(th["x"], th["dt"], th["A"], th["B"], th["C"], th["D"], dy,
                             th["init"], dfin)
    rng = np.random.default_rng(11)
    base = th[name]
    eps = 1e-3 if name != "init" else 1e-4
    v = rng.normal(0, 1, base.shape) * eps * (np.abs(base).mean() + 0.1)
    plus, minus = dict(th), dict(th)
    dtype = np.float64 if name == "init" else np.float32
    plus[name] = (base + v).astype(dtype)
    minus[name] = (base - v).astype(dtype)
    step = plus[name].astype(np.float64) - minus[name].astype(np.float64)
    fd = loss(plus, dy, dfin) - loss(minus, dy, dfin)
    an = float(np.sum(grads[GRAD[name]] * step))
    scale = float(np.sum(np.abs(grads[GRAD[name]] * step)))
    assert abs(fd - an) <= 2e-6 * scale + 1e-12, (name, fd, an, scale)


def test_elementwise_derivatives():
    """A few single elements of every gradient by central differences."""
    th, dy, dfin = problem(Bt=1, T=5, H=2, P=2, N=3, G=1, seed=5)
    grads = oracle.token_bwd(th["x"], th["dt"], th["A"], th["B"], th["C"], th["D"], dy,
                             th["init"], dfin)
    rng = np.random.default_rng(2)
    for name in GRAD:
        base = th[name]
        for _ in range(3):
            idx = tuple(rng.integers(0, s) for s in base.shape)
            plus, minus = dict(th), dict(th)
            dtype = np.float64 if name == "init" else np.float32
            p, m = base.copy(), base.copy()
            h = 1e-3 * (abs(float(base[idx])) + 0.1)
            p[idx] += h
            m[idx] -= h
            plus[name], minus[name] = p.astype(dtype), m.astype(dtype)
            step = float(plus[name][idx]) - float(minus[name][idx])
            fd = (loss(plus, dy, dfin) - loss(minus, dy, dfin)) / step
            g = float(grads[GRAD[name]][idx])
            assert abs(fd - g) <= 1e-5 * (abs(g) + 1e-3), (name, idx, fd, g)


def test_no_tokens_and_no_init():
    th, dy, dfin = problem(T=0, seed=1)
    g = oracle.token_bwd(th["x"], th["dt"], th["A"], th["B"], th["C"], th["D"], dy, th["init"],
                         dfin)
    np.testing.assert_array_equal(g["dinit"], dfin.astype(np.float64))
    assert np.all(g["dA"] == 0) and np.all(g["dD"] == 0)
    th, dy, dfin = problem(seed=4, init=False)
    g = oracle.token_bwd(th["x"], th["dt"], th["A"], th["B"], th["C"], th["D"], dy, None, dfin)
    # the gradient with respect to a zero initial state is still defined
    th0 = dict(th, init=np.zeros(g["dinit"].shape))
    g0 = oracle.token_bwd(th["x"], th["dt"], th["A"], th["B"], th["C"], th["D"], dy,
                          th0["init"], dfin)
    for k in GRAD.values():
        np.testing.assert_array_equal(g[k], g0[k])


def test_scalar_closed_form():
    """One token, P = N = 1: y = a h0 C + dt x B C + D x, a = exp(A dt)."""
    x, dt, A, B, C, D, h0, dy = 0.7, 0.3, -1.2, 0.9, -0.4, 0.25, 0.5, 1.3
    a = np.exp(A * dt)
    g = oracle.token_bwd(np.full((1, 1, 1, 1), x), np.full((1, 1, 1), dt), np.array([A]),
                         np.full((1, 1, 1, 1), B), np.full((1, 1, 1, 1), C), np.array([D]),
                         np.full((1, 1, 1, 1), dy), np.full((1, 1, 1, 1), h0))
    x, dt, A, B, C, D, dy = (float(np.float32(v)) for v in (x, dt, A, B, C, D, dy))
    a = np.exp(A * dt)
    h1 = a * h0 + dt * x * B
    exp = dict(dx=dy * (D + dt * C * B), ddt=dy * C * (A * a * h0 + x * B),
               dA=dy * C * dt * a * h0, dB=dy * C * dt * x, dC=dy * h1, dD=dy * x,
               dinit=dy * C * a)
    for k, v in exp.items():
        assert abs(float(g[k].reshape(-1)[0]) - v) <= 1e-12 * max(1.0, abs(v)), (k, g[k], v)


def test_zero_dt_closed_form():
    """dt = 0 at every token: the state is init_state throughout, so
    y_t = C_t . init + D x_t.  Then dinit = dfinal + sum_t dy_t (outer) C_t,
    dx = D dy, dD = sum dy . x, dB = 0 (B enters only through dt), and
    dC_t = sum over the group's heads of dy_t . init."""
    th, dy, dfin = problem(Bt=2, T=9, H=4, P=3, N=5, G=2, seed=3)
    th["dt"][:] = 0
    g = oracle.token_bwd(th["x"], th["dt"], th["A"], th["B"], th["C"], th["D"], dy,
                         th["init"], dfin)
    Bt, T, H, P = th["x"].shape
    G, N = th["C"].shape[2], th["C"].shape[3]
    hpg = H // G
    dy64, x64, C64 = (a.astype(np.float64) for a in (dy, th["x"], th["C"]))
    Cg = np.repeat(C64, hpg, axis=2)                             # [Bt, T, H, N]
    dinit = dfin + np.einsum("bthp,bthn->bhpn", dy64, Cg)
    dC = np.einsum("bthp,bhpn->bthn", dy64, th["init"]).reshape(Bt, T, G, hpg, N).sum(axis=3)
    exp = dict(dinit=dinit, dx=dy64 * th["D"].astype(np.float64).reshape(1, 1, H, 1),
               dD=np.einsum("bthp,bthp->h", dy64, x64), dB=np.zeros((Bt, T, G, N)), dC=dC)
    for k, v in exp.items():
        np.testing.assert_allclose(np.asarray(g[k], np.float64).reshape(v.shape), v,
                                   rtol=1e-12, atol=1e-12, err_msg=k)
