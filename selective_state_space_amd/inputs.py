"""Seeded synthetic inputs for the Mamba-2 SSD layer scan.

This module only draws random numbers and rounds them; it holds none of the
scan's arithmetic. Both the GPU path's tests/bench and the CPU oracle take
their inputs from here, so the two sides always see identical values.

Recipe (the shapes and value distributions of the six workloads):

* ``A_h = -exp(U(ln 1, ln 16))`` per head (a negative decay rate, so that
  ``a_t = A dt_t <= 0``; "Accelerating Mamba-2 with High-Performance Forward
  Pass Kernels in NVIDIA CUDA Tile", section "Mamba-2 architecture").
* ``D_h ~ N(0, 1)`` per head.
* ``dt = softplus(z + dt_bias_h)``, ``z ~ N(0, 1)``, with a per-head
  ``dt_bias_h = ln(expm1(dt0_h))`` (the inverse softplus of
  ``dt0_h = exp(U(ln 1e-3, ln 1e-1))``), so dt sits roughly in [1e-3, 1e-1].
  softplus returns its argument above 20 ("Optimizing Nemotron v3 Super in
  TensorRT-LLM", section 6.2).  The library receives dt after softplus.
* ``x ~ N(0, 1)``; ``B, C ~ N(0, 1) / sqrt(N)``; optional initial state
  ``h0 ~ N(0, 0.1^2)``.
* For bf16 workloads, x, B and C are rounded once to bfloat16 on the host
  (round to nearest even); the arrays returned hold those exact values in
  float32, so an exact upcast is all either side needs.
* Seed 0 by default.  Every tensor has its own NumPy PCG64 stream keyed by
  (seed, tensor id, block): the per-head parameters A, D, dt_bias are drawn in
  that order from ``default_rng([seed, 0])``; the per-token tensors x, z, B, C
  and h0 (ids 1..5) are drawn in blocks of 2^22 elements, block k from
  ``default_rng([seed, id, k])``, so blocks can be drawn in parallel threads
  and the values do not depend on the thread count.  Decode step s uses the
  ids 1000 + 8 s + (1, 2, 3, 4) for its x, z, B, C; call c of a multi-token
  decode with K tokens per sequence takes decode steps cK .. cK + K - 1.
"""

from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one SSD call (or of one decode step when ``kind == 'decode'``)."""

    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int
    io_dtype: str
    init_state: bool = False
    kind: str = "fwd"
    steps: int = 1
    description: str = ""

    @property
    def heads_per_group(self) -> int:
        return self.nheads // self.ngroups

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk_size)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Index 0 is the tiny fp32 case, 1-3 forward layers, 4 decode, 5 multi-token decode.
WORKLOADS = [
    Workload("tiny_fp32", 1, 256, 4, 64, 64, 1, 64, F32,
             description="tiny SSD forward, fp32 throughout"),
    Workload("mamba2_370m", 4, 2048, 32, 64, 128, 1, 256, BF16,
             description="Mamba-2 370M-shaped layer (d_inner 2048 = 32 heads x 64)"),
    Workload("mamba2_2p7b", 8, 4096, 80, 64, 128, 1, 256, BF16, init_state=True,
             description="Mamba-2 2.7B-shaped layer (d_inner 5120 = 80 heads x 64), "
                         "random initial state"),
    Workload("long_ctx_hybrid", 1, 65536, 128, 64, 128, 8, 256, BF16,
             description="long-context hybrid-model layer, 128 heads, 8 groups, T=65536"),
    Workload("decode_b256", 256, 1, 128, 64, 128, 8, 256, BF16, kind="decode", steps=512,
             description="recurrent decode, batch 256, 128 heads, 8 groups, 512 steps"),
    Workload("mtp_verify_b256_k4", 256, 4, 128, 64, 128, 8, 256, BF16, kind="decode_multi",
             description="multi-token decode of speculative verification: 256 sequences x 4 "
                         "tokens (seqlen = tokens per sequence), decode_b256's heads, a snapshot "
                         "of the state after every token, main state not updated"),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)
    return r


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _softplus_thresholded(v: np.ndarray) -> np.ndarray:
    # log1p(exp(v)) for v <= 20, v itself above (input recipe, not the scan)
    return np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))


BLOCK = 1 << 22
_ID_X, _ID_Z, _ID_B, _ID_C, _ID_H0 = 1, 2, 3, 4, 5
_pool = None


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def _blocked(key, shape, fill) -> np.ndarray:
    """A float32 array of `shape`; block k is written by fill(rng_k, view, start)."""
    global _pool
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    nb = -(-n // BLOCK)

    def work(k):
        rng = np.random.default_rng(list(key) + [k])
        fill(rng, out[k * BLOCK: min(n, (k + 1) * BLOCK)], k * BLOCK)

    if nb <= 1:
        for k in range(nb):
            work(k)
    else:
        if _pool is None:
            _pool = cf.ThreadPoolExecutor(_threads())
        list(_pool.map(work, range(nb)))
    return out.reshape(shape)


def _normal(key, shape, scale: float = 1.0, bf16: bool = False) -> np.ndarray:
    sc = np.float32(scale)

    def fill(rng, v, start):
        rng.standard_normal(out=v, dtype=np.float32)
        if scale != 1.0:
            np.multiply(v, sc, out=v)
        if bf16:
            v[:] = bf16_round(v)

    return _blocked(key, shape, fill)


def _dt(key, shape, dt_bias: np.ndarray) -> np.ndarray:
    # dt = softplus(z + dt_bias[h]), z ~ N(0, 1); heads are the last axis
    H = dt_bias.shape[0]
    flat_bias = dt_bias.astype(np.float64)

    def fill(rng, v, start):
        z = rng.standard_normal(v.shape[0], dtype=np.float32).astype(np.float64)
        h = (start + np.arange(v.shape[0])) % H     # flat index -> head
        v[:] = _softplus_thresholded(z + flat_bias[h]).astype(np.float32)

    return _blocked(key, shape, fill)


@dataclasses.dataclass
class Params:
    """Per-head parameters shared by every token of a workload."""

    A: np.ndarray        # [H] float32, negative
    D: np.ndarray        # [H] float32
    dt_bias: np.ndarray  # [H] float64 (only used to draw dt)


@dataclasses.dataclass
class FwdInputs:
    x: np.ndarray        # [Bt, T, H, P] float32 (bf16-exact for bf16 workloads)
    dt: np.ndarray       # [Bt, T, H] float32, > 0
    A: np.ndarray        # [H] float32
    B: np.ndarray        # [Bt, T, G, N]
    C: np.ndarray        # [Bt, T, G, N]
    D: np.ndarray        # [H]
    init_state: Optional[np.ndarray]  # [Bt, H, P, N] float32 or None


def _params(seed: int, H: int) -> Params:
    rng = np.random.default_rng([seed, 0])
    A = (-np.exp(rng.uniform(math.log(1.0), math.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    dt0 = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=H))
    dt_bias = np.log(np.expm1(dt0))
    return Params(A, D, dt_bias)


def make_fwd(w: Workload, seed: int = 0) -> FwdInputs:
    """Inputs of one chunked-forward call for workload ``w``."""
    Bt, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    prm = _params(seed, H)
    bf = w.io_dtype == BF16
    x = _normal((seed, _ID_X), (Bt, T, H, P), bf16=bf)
    dt = _dt((seed, _ID_Z), (Bt, T, H), prm.dt_bias)
    s = 1.0 / math.sqrt(N)
    B = _normal((seed, _ID_B), (Bt, T, G, N), s, bf16=bf)
    C = _normal((seed, _ID_C), (Bt, T, G, N), s, bf16=bf)
    h0 = _normal((seed, _ID_H0), (Bt, H, P, N), 0.1) if w.init_state else None
    return FwdInputs(x, dt, prm.A, B, C, prm.D, h0)


@dataclasses.dataclass
class DecodeInputs:
    x_t: np.ndarray   # [Bt, H, P]
    dt_t: np.ndarray  # [Bt, H]
    B_t: np.ndarray   # [Bt, G, N]
    C_t: np.ndarray   # [Bt, G, N]


def decode_params(w: Workload, seed: int = 0) -> Params:
    """A, D and dt_bias of a decode workload (shared by all its steps)."""
    return _params(seed, w.nheads)


def make_decode_step(w: Workload, step: int, prm: Params, seed: int = 0) -> DecodeInputs:
    """Per-token inputs of decode step ``step`` of workload ``w``."""
    Bt, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    base = 1000 + 8 * step
    bf = w.io_dtype == BF16
    x = _normal((seed, base + 1), (Bt, H, P), bf16=bf)
    dt = _dt((seed, base + 2), (Bt, H), prm.dt_bias)
    s = 1.0 / math.sqrt(N)
    B = _normal((seed, base + 3), (Bt, G, N), s, bf16=bf)
    C = _normal((seed, base + 4), (Bt, G, N), s, bf16=bf)
    return DecodeInputs(x, dt, B, C)


@dataclasses.dataclass
class MultiInputs:
    x: np.ndarray    # [Bt, K, H, P]
    dt: np.ndarray   # [Bt, K, H]
    B: np.ndarray    # [Bt, K, G, N]
    C: np.ndarray    # [Bt, K, G, N]


def make_decode_multi(w: Workload, prm: Params, call: int = 0, seed: int = 0) -> MultiInputs:
    """Inputs of one multi-token decode call: K = w.seqlen tokens per sequence,
    token k being decode step call * K + k of the same stream."""
    K = w.seqlen
    steps = [make_decode_step(w, call * K + k, prm, seed) for k in range(K)]
    return MultiInputs(*(np.stack([getattr(s, f) for s in steps], axis=1)
                         for f in ("x_t", "dt_t", "B_t", "C_t")))


def make_small(Bt: int, T: int, H: int, P: int, N: int, G: int, io_dtype: str = F32,
               init_state: bool = False, seed: int = 0) -> FwdInputs:
    """Same recipe at an arbitrary (small) shape, for tests."""
    w = Workload("custom", Bt, T, H, P, N, G, 64, io_dtype, init_state=init_state)
    return make_fwd(w, seed)
