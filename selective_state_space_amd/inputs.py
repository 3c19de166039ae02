"""Seeded synthetic inputs for the Mamba-2 SSD layer scan.

This module only draws random numbers and rounds them; it holds none of the
scan's arithmetic. Both the GPU path's tests/bench and the CPU oracle take
their inputs from here, so the two sides always see identical values.

Recipe (the shapes and value distributions of the five workloads):

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
* Seed 0 by default; one ``numpy.random.default_rng(seed)`` per workload with
  the fixed draw order A, D, dt_bias, x, z, B, C, h0.  Decode steps draw their
  per-token inputs from ``default_rng([seed, step])``.
"""

from __future__ import annotations

import dataclasses
import math
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


# The five workloads.  Index 0 is the tiny fp32 case, 1-3 forward layers, 4 decode.
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
    out = np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))
    return out


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


def _params(rng: np.random.Generator, H: int) -> Params:
    A = (-np.exp(rng.uniform(math.log(1.0), math.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    dt0 = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=H))
    dt_bias = np.log(np.expm1(dt0))
    return Params(A, D, dt_bias)


def _draw_dt(rng: np.random.Generator, shape, dt_bias: np.ndarray) -> np.ndarray:
    z = rng.standard_normal(shape, dtype=np.float32).astype(np.float64)
    return _softplus_thresholded(z + dt_bias).astype(np.float32)


def _maybe_bf16(a: np.ndarray, io_dtype: str) -> np.ndarray:
    return bf16_round(a) if io_dtype == BF16 else np.ascontiguousarray(a, dtype=np.float32)


def make_fwd(w: Workload, seed: int = 0) -> FwdInputs:
    """Inputs of one chunked-forward call for workload ``w``."""
    Bt, T, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    rng = np.random.default_rng(seed)
    prm = _params(rng, H)
    x = _maybe_bf16(rng.standard_normal((Bt, T, H, P), dtype=np.float32), w.io_dtype)
    dt = _draw_dt(rng, (Bt, T, H), prm.dt_bias)
    s = np.float32(1.0 / math.sqrt(N))
    B = _maybe_bf16(rng.standard_normal((Bt, T, G, N), dtype=np.float32) * s, w.io_dtype)
    C = _maybe_bf16(rng.standard_normal((Bt, T, G, N), dtype=np.float32) * s, w.io_dtype)
    h0 = None
    if w.init_state:
        h0 = (rng.standard_normal((Bt, H, P, N), dtype=np.float32) * np.float32(0.1))
    return FwdInputs(x, dt, prm.A, B, C, prm.D, h0)


@dataclasses.dataclass
class DecodeInputs:
    x_t: np.ndarray   # [Bt, H, P]
    dt_t: np.ndarray  # [Bt, H]
    B_t: np.ndarray   # [Bt, G, N]
    C_t: np.ndarray   # [Bt, G, N]


def decode_params(w: Workload, seed: int = 0) -> Params:
    """A, D and dt_bias of a decode workload (shared by all its steps)."""
    return _params(np.random.default_rng(seed), w.nheads)


def make_decode_step(w: Workload, step: int, prm: Params, seed: int = 0) -> DecodeInputs:
    """Per-token inputs of decode step ``step`` of workload ``w``."""
    Bt, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    rng = np.random.default_rng([seed, step])
    x = _maybe_bf16(rng.standard_normal((Bt, H, P), dtype=np.float32), w.io_dtype)
    dt = _draw_dt(rng, (Bt, H), prm.dt_bias)
    s = np.float32(1.0 / math.sqrt(N))
    B = _maybe_bf16(rng.standard_normal((Bt, G, N), dtype=np.float32) * s, w.io_dtype)
    C = _maybe_bf16(rng.standard_normal((Bt, G, N), dtype=np.float32) * s, w.io_dtype)
    return DecodeInputs(x, dt, B, C)


def make_small(Bt: int, T: int, H: int, P: int, N: int, G: int, io_dtype: str = F32,
               init_state: bool = False, seed: int = 0) -> FwdInputs:
    """Same recipe at an arbitrary (small) shape, for tests."""
    w = Workload("custom", Bt, T, H, P, N, G, 64, io_dtype, init_state=init_state)
    return make_fwd(w, seed)
