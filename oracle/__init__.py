"""CPU oracle for the Mamba-2 SSD layer scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path.

Three independent CPU computations of the same layer, all float64:

* :func:`token_fwd` / :func:`token_decode` -- the plain token-by-token
  recurrence, in C (``ssd_oracle.c``, POSIX threads).  This is the oracle the
  GPU path is compared with.
* :func:`chunked_reference` -- the chunked (SSD) form in NumPy, written out
  from its equations: chunk-local cumulative log-decay G, per-chunk states,
  the state pass between chunks, and the chunk output with the decayed,
  causally masked C B^T.  It exposes the intermediates G, S and h_prev.
* :func:`brute_force` -- the fully expanded sum over all earlier tokens, in
  plain Python loops; for tiny inputs only.

Pages followed ("[T]" = "Accelerating Mamba-2 with High-Performance Forward
Pass Kernels in NVIDIA CUDA Tile"; "[N]" = "Optimizing Nemotron v3 Super in
TensorRT-LLM"):

* recurrence and output: [T] section "Mamba-2 architecture" (first pair of
  equations); [N] section 6.1 "The SSU Math";
* the unrolled recurrence and the log-space chunk equations
  h_{t+T} = exp(G_last) h_t + (exp(G_last - G) . B)^T X and
  Y = exp(G) C h + (exp(G - G^T) . C B^T . M) X + D X: [T] section "Mamba-2
  architecture", the equations after the jump formula;
* the three-stage decomposition (cumulative sum per chunk, state carried from
  chunk to chunk, chunk output): [T] sections "Kernel 1" to "Kernel 3".

Readings where the pages are silent or disagree:
the output uses the updated state h_t; the state is stored [P][N]; head h
uses group h // (H/G); positions past the end of a ragged last chunk carry
dt = 0; a missing initial state means zeros.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libssd_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=gnu11", "-Wall", "-Werror", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, dp, fp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        lib.ssd_oracle_fwd.argtypes = [fp, fp, fp, fp, fp, fp, dp, i64, i64, i64, i64, i64, i64,
                                       dp, i64, dp, dp, ip]
        lib.ssd_oracle_fwd.restype = ctypes.c_int
        lib.ssd_oracle_decode.argtypes = [dp, fp, fp, fp, fp, fp, fp, i64, i64, i64, i64, i64,
                                          dp, i64, dp, ip]
        lib.ssd_oracle_decode.restype = ctypes.c_int
        lib.ssd_oracle_fwd_gated.argtypes = [fp, fp, fp, fp, fp, fp, fp, ip, fp, dp, i64, i64,
                                             i64, i64, i64, i64, dp, i64, dp, dp, ip]
        lib.ssd_oracle_fwd_gated.restype = ctypes.c_int
        lib.ssd_oracle_decode_gated.argtypes = [dp, fp, fp, fp, fp, fp, fp, fp, ip, fp, i64, i64,
                                                i64, i64, i64, dp, i64, dp, ip]
        lib.ssd_oracle_decode_gated.restype = ctypes.c_int
        lib.ssd_oracle_bwd.argtypes = [fp, fp, fp, fp, fp, fp, dp, fp, fp, i64, i64, i64, i64,
                                       i64, i64, dp, dp, dp, dp, dp, dp, dp, ip]
        lib.ssd_oracle_bwd.restype = ctypes.c_int
        lib.ssd_oracle_host_threads.argtypes = []
        lib.ssd_oracle_host_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def host_threads() -> int:
    """Threads the oracle uses by default (the process's CPU affinity count)."""
    return _load().ssd_oracle_host_threads()


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def token_fwd(x, dt, A, B, C, D, init_state=None, pairs: Optional[Sequence[int]] = None,
              want_y: bool = True, nthreads: int = 0, dt_bias=None, dt_softplus: bool = False,
              z=None):
    """Token-by-token float64 forward.

    x [Bt,T,H,P], dt [Bt,T,H], A [H], B/C [Bt,T,G,N], D [H], init_state
    [Bt,H,P,N] or None.  ``pairs`` selects (b, h) pairs as flat indices b*H+h
    (None = all, in order).  Returns (y [npairs,T,P] or None, final
    [npairs,P,N], threads_used).  With pairs=None the results reshape to
    [Bt,H,T,P] and [Bt,H,P,N].

    The optional layer interface ("Optimizing Nemotron v3 Super in
    TensorRT-LLM", sections 6.1 and 6.3): ``dt_bias`` [H] is added to dt, then
    ``dt_softplus`` applies log(1 + e^dt) where dt <= 20; ``z`` [Bt,T,H,P]
    gates the output, y * silu(z), after the D term.
    """
    x, dt, A, B, C, D = map(_f32, (x, dt, A, B, C, D))
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (Bt, T, H) and B.shape == C.shape == (Bt, T, G, N)
    assert A.shape == D.shape == (H,)
    pr = None if pairs is None else np.ascontiguousarray(pairs, dtype=np.int64)
    npairs = Bt * H if pr is None else len(pr)
    init = None
    if init_state is not None:
        init = np.asarray(init_state, dtype=np.float64).reshape(Bt * H, P, N)
        init = np.ascontiguousarray(init if pr is None else init[pr])
    y = np.empty((npairs, T, P), np.float64) if want_y else None
    fin = np.empty((npairs, P, N), np.float64)
    bias = None if dt_bias is None else _f32(dt_bias)
    zz = None if z is None else _f32(z)
    assert bias is None or bias.shape == (H,)
    assert zz is None or zz.shape == x.shape
    rc = _load().ssd_oracle_fwd_gated(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(bias), int(bool(dt_softplus)), _ptr(zz), _ptr(init),
                                      Bt, T, H, P, N, G, _ptr(pr), npairs, _ptr(y), _ptr(fin),
                                      nthreads)
    if rc < 0:
        raise ValueError("ssd_oracle_fwd rejected its arguments (%d)" % rc)
    return y, fin, rc


def token_decode(state, x_t, dt_t, B_t, C_t, A, D, pairs: Optional[Sequence[int]] = None,
                 nthreads: int = 0, dt_bias=None, dt_softplus: bool = False, z_t=None):
    """One float64 decode step, updating ``state`` [npairs,P,N] (float64) in place.

    x_t [Bt,H,P], dt_t [Bt,H], B_t/C_t [Bt,G,N].  Returns y_t [npairs,P].
    dt_bias, dt_softplus and the gate z_t [Bt,H,P] as in token_fwd.
    """
    x_t, dt_t, B_t, C_t, A, D = map(_f32, (x_t, dt_t, B_t, C_t, A, D))
    Bt, H, P = x_t.shape
    G, N = B_t.shape[1], B_t.shape[2]
    assert state.dtype == np.float64 and state.flags.c_contiguous
    pr = None if pairs is None else np.ascontiguousarray(pairs, dtype=np.int64)
    npairs = Bt * H if pr is None else len(pr)
    assert state.shape == (npairs, P, N)
    y = np.empty((npairs, P), np.float64)
    bias = None if dt_bias is None else _f32(dt_bias)
    zz = None if z_t is None else _f32(z_t)
    assert zz is None or zz.shape == x_t.shape
    rc = _load().ssd_oracle_decode_gated(_ptr(state), _ptr(x_t), _ptr(dt_t), _ptr(B_t),
                                         _ptr(C_t), _ptr(A), _ptr(D), _ptr(bias),
                                         int(bool(dt_softplus)), _ptr(zz), Bt, H, P, N, G,
                                         _ptr(pr), npairs, _ptr(y), nthreads)
    if rc < 0:
        raise ValueError("ssd_oracle_decode rejected its arguments (%d)" % rc)
    return y


def token_decode_multi(state, x, dt, B, C, A, D, parent=None, update_state: bool = True,
                       pairs: Optional[Sequence[int]] = None, nthreads: int = 0, dt_bias=None,
                       dt_softplus: bool = False, z=None):
    """K decode steps per sequence in float64, with the state after every step.

    Multi-token state update with per-step snapshots ("Optimizing Nemotron v3
    Super in TensorRT-LLM", sections 10.3 and 10.4): for each sequence b the
    K tokens x[b, k] are taken in order; step k starts from the state that
    step p(k) produced, where p(k) = parent[b, k] when parent is given,
    k >= 1 and 0 <= parent[b, k] < k (a draft tree), and p(k) = k - 1
    otherwise; step 0 starts from ``state``.  The snapshot of step k is the
    state after step k.  With ``update_state`` the final running state (that
    of step K - 1) replaces ``state``; without it ``state`` is left as it was
    (the verification pass that must not overwrite the main state).

    state [npairs,P,N] float64, x [Bt,K,H,P], dt [Bt,K,H], B/C [Bt,K,G,N],
    parent [Bt,K] integers or None; z [Bt,K,H,P] as in token_fwd.
    Returns (y [npairs,K,P], snapshots [npairs,K,P,N]).
    """
    x, dt, B, C = map(_f32, (x, dt, B, C))
    Bt, K, H, P = x.shape
    N = B.shape[3]
    assert state.dtype == np.float64 and state.flags.c_contiguous
    pr = np.arange(Bt * H) if pairs is None else np.asarray(pairs, dtype=np.int64)
    npairs = len(pr)
    assert state.shape == (npairs, P, N)
    zz = None if z is None else _f32(z)
    par = None if parent is None else np.asarray(parent, dtype=np.int64).reshape(Bt, K)
    y = np.empty((npairs, K, P), np.float64)
    snaps = np.empty((npairs, K, P, N), np.float64)
    run = state.copy()
    row = pr // H            # the sequence of each pair
    for k in range(K):
        if par is not None and k >= 1:
            pk = par[row, k]
            take = (pk >= 0) & (pk < k)
            for i in np.nonzero(take)[0]:
                run[i] = snaps[i, pk[i]]
        y[:, k] = token_decode(run, x[:, k], dt[:, k], B[:, k], C[:, k], A, D, pairs=pr,
                               nthreads=nthreads, dt_bias=dt_bias, dt_softplus=dt_softplus,
                               z_t=None if zz is None else zz[:, k])
        snaps[:, k] = run
    if update_state:
        state[...] = run
    return y, snaps


def token_bwd(x, dt, A, B, C, D, dy, init_state=None, dfinal=None, nthreads: int = 0):
    """Float64 gradients of L = sum(dy * y) + sum(dfinal * final_state) for the
    plain forward (no layer options): the exact adjoint of the recurrence,
    token by token (the "mamba3" kernel card, section "Backward", for the order a
    chunked backward takes: a reverse scan of the state adjoint).

    Shapes as token_fwd, dy [Bt,T,H,P], dfinal [Bt,H,P,N] or None.  Returns a
    dict with dx [Bt,T,H,P], ddt [Bt,T,H], dB and dC [Bt,T,G,N] (summed over
    the heads of each group), dA and dD [H] (summed over batch and tokens)
    and dinit [Bt,H,P,N].
    """
    x, dt, A, B, C, D, dy = map(_f32, (x, dt, A, B, C, D, dy))
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dy.shape == x.shape and dt.shape == (Bt, T, H) and B.shape == C.shape
    init = None if init_state is None else np.ascontiguousarray(init_state, np.float64)
    dfin = None if dfinal is None else _f32(dfinal)
    out = dict(dx=np.empty((Bt, T, H, P)), ddt=np.empty((Bt, T, H)), dB=np.empty((Bt, T, G, N)),
               dC=np.empty((Bt, T, G, N)), dA=np.empty(H), dD=np.empty(H),
               dinit=np.empty((Bt, H, P, N)))
    rc = _load().ssd_oracle_bwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                _ptr(init), _ptr(dy), _ptr(dfin), Bt, T, H, P, N, G,
                                *(_ptr(out[k]) for k in ("dx", "ddt", "dB", "dC", "dA", "dD",
                                                        "dinit")), nthreads)
    if rc < 0:
        raise ValueError("ssd_oracle_bwd rejected its arguments (%d)" % rc)
    return out


def chunked_reference(x, dt, A, B, C, D, chunk_size: int, init_state=None):
    """The chunked SSD form in float64 NumPy, with its intermediates.

    The sequence is cut into chunks of L = chunk_size tokens; a ragged last
    chunk is padded with dt = 0 (and zero x, B, C), which leaves state and
    outputs unchanged.  Per (b, h, chunk c), natural-log units:

      G[i]      = sum_{r <= i} A dt_r                     (chunk-local, inclusive)
      S_c       = sum_j exp(G_last - G_j) dt_j x_j (outer) B_j        [P x N]
      h_prev[c] = h;   h <- exp(G_last) h + S_c           (h starts at init)
      y_i       = exp(G_i) C_i h_prev[c]^T
                  + sum_{j <= i} exp(G_i - G_j) (C_i . B_j) dt_j x_j + D x_i

    Returns a dict: G [Bt,H,nc,L], S [Bt,H,nc,P,N], h_prev [Bt,H,nc,P,N],
    y [Bt,T,H,P], final [Bt,H,P,N].
    """
    x, dt, B, C = (np.asarray(a, dtype=np.float64) for a in (x, dt, B, C))
    A = np.asarray(A, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    Bt, T, H, P = x.shape
    G_, N = B.shape[2], B.shape[3]
    hpg = H // G_
    L = int(chunk_size)
    nc = -(-T // L)
    pad = nc * L - T

    def padt(a):
        return np.concatenate([a, np.zeros((a.shape[0], pad) + a.shape[2:])], axis=1) if pad else a

    xp, dtp, Bp, Cp = padt(x), padt(dt), padt(B), padt(C)
    # per-head views: [Bt, H, nc, L, ...]
    xh = xp.reshape(Bt, nc, L, H, P).transpose(0, 3, 1, 2, 4)
    dth = dtp.reshape(Bt, nc, L, H).transpose(0, 3, 1, 2)
    grp = np.arange(H) // hpg
    Bh = Bp.reshape(Bt, nc, L, G_, N)[:, :, :, grp, :].transpose(0, 3, 1, 2, 4)
    Ch = Cp.reshape(Bt, nc, L, G_, N)[:, :, :, grp, :].transpose(0, 3, 1, 2, 4)

    a = A[None, :, None, None] * dth                        # [Bt,H,nc,L]
    Gc = np.cumsum(a, axis=3)
    Glast = Gc[..., -1]                                     # [Bt,H,nc]
    w = np.exp(Glast[..., None] - Gc) * dth                 # [Bt,H,nc,L]
    S = np.einsum("bhcl,bhclp,bhcln->bhcpn", w, xh, Bh)

    h = (np.zeros((Bt, H, P, N)) if init_state is None
         else np.asarray(init_state, dtype=np.float64).copy())
    h_prev = np.empty((Bt, H, nc, P, N))
    for c in range(nc):
        h_prev[:, :, c] = h
        h = np.exp(Glast[:, :, c])[..., None, None] * h + S[:, :, c]

    inter = np.exp(Gc)[..., None] * np.einsum("bhcin,bhcpn->bhcip", Ch, h_prev)
    CB = np.einsum("bhcin,bhcjn->bhcij", Ch, Bh)
    diff = Gc[..., :, None] - Gc[..., None, :]
    causal = np.tril(np.ones((L, L), dtype=bool))
    decay = np.exp(np.where(causal, diff, -np.inf))         # masked before exp
    intra = np.einsum("bhcij,bhcj,bhcjp->bhcip", decay * CB, dth, xh)
    yh = inter + intra + D[None, :, None, None, None] * xh
    y = yh.transpose(0, 2, 3, 1, 4).reshape(Bt, nc * L, H, P)[:, :T]
    return {"G": Gc, "S": S, "h_prev": h_prev, "y": y, "final": h}


def brute_force(x, dt, A, B, C, D, init_state=None):
    """Fully expanded recurrence, explicit loops; tiny T only.

    y_t = sum_{s <= t} exp(sum_{r=s+1..t} a_r) dt_s (C_t . B_s) x_s
          + exp(sum_{r <= t} a_r) h0 C_t + D x_t
    final = exp(sum_r a_r) h0 + sum_s exp(sum_{r > s} a_r) dt_s x_s (outer) B_s
    with a_r = A dt_r.  Returns (y [Bt,T,H,P], final [Bt,H,P,N]).
    """
    x, dt, B, C = (np.asarray(a, dtype=np.float64) for a in (x, dt, B, C))
    A = np.asarray(A, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    Bt, T, H, P = x.shape
    G_, N = B.shape[2], B.shape[3]
    hpg = H // G_
    y = np.zeros((Bt, T, H, P))
    fin = np.zeros((Bt, H, P, N))
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            h0 = (np.zeros((P, N)) if init_state is None
                  else np.asarray(init_state, dtype=np.float64)[b, h])
            a = [A[h] * dt[b, r, h] for r in range(T)]
            for t in range(T):
                acc = math.exp(math.fsum(a[: t + 1])) * (h0 @ C[b, t, g])
                for s in range(t + 1):
                    coef = math.exp(math.fsum(a[s + 1: t + 1])) * dt[b, s, h]
                    acc = acc + coef * float(np.dot(C[b, t, g], B[b, s, g])) * x[b, s, h]
                y[b, t, h] = acc + D[h] * x[b, t, h]
            f = math.exp(math.fsum(a)) * h0
            for s in range(T):
                coef = math.exp(math.fsum(a[s + 1:])) * dt[b, s, h]
                f = f + coef * np.outer(x[b, s, h], B[b, s, g])
            fin[b, h] = f
    return y, fin
