"""Reduced-precision decode state for the oracle -- TEST INFRASTRUCTURE ONLY.

"Optimizing Nemotron v3 Super in TensorRT-LLM", section 6.5 ("Quantized State
& Stochastic Rounding"): the decode state may be kept in HBM as

* int16 codes with one scale per state row (per head-dim index p): after the
  update, the row's largest magnitude m sets encode = 32767 / m, the codes are
  the scaled values rounded to integers, and decode = 1 / encode is stored
  beside them;
* fp16, rounded to nearest or stochastically, with the random bits taken
  from a Philox-4x32 counter-based generator (13 bits per element: the bits
  fp32 carries below fp16's last place; a 32-bit word serves two elements)
  whose round count is a parameter of the kernels (zero rounds meaning no
  stochastic rounding);
* and, as the same section's dispatch table lists, bf16 (round to nearest).

The update itself is the plain fp64 decode step of the oracle (section 6.1)
applied to the decoded state; the output y uses the updated state before it
is rounded for storage.  Where a float decides an integer or a rounding
direction (the codes, the scales, the stochastic choice), it is decided in
fp32, the precision the GPU stores from, on the fp64 state rounded to fp32.

Philox-4x32 follows its published definition (J. K. Salmon, M. A. Moraes,
R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11,
section 5): per round, two 32x32 -> 64-bit products of counter words with
the multipliers 0xD2511F53 and 0xCD9E8D57, a swap-and-xor with the key, and a
Weyl increment of the key by (0x9E3779B9, 0xBB67AE85); 10 rounds is the
generator's standard count.

Readings where the page is silent: the abs-max is over
the N values of a row; codes round half to even and are clipped to
[-32767, 32767]; an all-zero row stores codes 0 and decode scale 0; one
Philox block serves 8 consecutive elements of a row, its counter being the
flat index (b, h, p, n) of the first of them (low word, high word, 0, 0) and
its key the 64-bit seed (low word, high word); element n takes word
(n mod 8) // 2, its bits 0..12 for even n and 16..28 for odd n; stochastic
rounding of x adds (r / 2^13) of fp16's unit in the last place at |x| to |x|
and rounds toward zero, saturating at 65504.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF
INT16_MAX = 32767
F16_MAX = 65504.0

F32, F16, BF16, INT16 = "f32", "f16", "bf16", "int16"


def philox4x32(counter, key, rounds: int = 10):
    """Philox-4x32 on arrays of counters: counter [..., 4] and key [..., 2]
    (uint32 values, broadcast together).  Returns [..., 4] uint32."""
    c = [np.asarray(counter, dtype=np.uint64)[..., i] & MASK32 for i in range(4)]
    k = [np.asarray(key, dtype=np.uint64)[..., i] & MASK32 for i in range(2)]
    for r in range(rounds):
        p0 = np.uint64(M0) * c[0]
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
        if r + 1 < rounds:
            k = [(k[0] + np.uint64(W0)) & np.uint64(MASK32),
                 (k[1] + np.uint64(W1)) & np.uint64(MASK32)]
    return np.stack(c, axis=-1).astype(np.uint32)


def state_random_bits(nelem: int, seed: int, start: int = 0, rounds: int = 10):
    """13 random bits for the state elements of flat indices start ..
    start + nelem - 1 (start a multiple of 8), from one Philox block per 8
    consecutive elements: element k of a block takes word k // 2, its low
    half's 13 low bits for even k and its high half's for odd k."""
    assert start % 8 == 0
    first = np.arange(start, start + nelem, 8, dtype=np.uint64)
    ctr = np.stack([first & np.uint64(MASK32), first >> np.uint64(32),
                    np.zeros_like(first), np.zeros_like(first)], axis=-1)
    key = np.array([seed & MASK32, (seed >> 32) & MASK32], dtype=np.uint64)
    words = philox4x32(ctr, key, rounds).astype(np.uint32)      # [nblocks, 4]
    halves = np.stack([words & np.uint32(0xFFFF), words >> np.uint32(16)], axis=-1)
    return (halves.reshape(-1)[:nelem] & np.uint32(0x1FFF)).astype(np.int64)


def _ulp16(a):
    """fp16's unit in the last place at magnitude a >= 0 (float64 array)."""
    a = np.asarray(a, dtype=np.float64)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a < 2.0 ** -14, 2.0 ** -24, 2.0 ** (e - 10))


def round_f16_stochastic(x32, r13):
    """fp32 values -> fp16 values (returned as float64) by stochastic rounding
    with 13-bit random integers r13: |x| + (r13 / 2^13) ulp16(|x|), rounded
    toward zero to fp16, saturated at 65504; the sign is kept.

    Written as a comparison so that it is exact at every magnitude: with
    |x| = (n + f) ulp16 (n an integer, 0 <= f < 1) the result is n ulp16, or
    (n + 1) ulp16 when f 2^13 >= 2^13 - r13.  In fp16's normal range f 2^13 is
    an integer (fp32 keeps 13 bits below fp16's last place); below it, in the
    subnormal range, f has more bits than the random integer resolves."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    u = _ulp16(a)
    A = a / u                         # exact: u is a power of two
    n = np.floor(A)
    f8 = (A - n) * 8192.0             # exact
    up = f8 >= 8192.0 - np.asarray(r13, dtype=np.float64)
    q = (n + up) * u
    q = np.minimum(q, F16_MAX)
    return np.copysign(q, x)


def round_f16_nearest(x32):
    return np.asarray(x32, dtype=np.float32).astype(np.float16).astype(np.float64)


def round_bf16_nearest(x32):
    """fp32 -> bf16 (round to nearest, ties to even) by the bit pattern."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return (r & np.uint64(MASK32)).astype(np.uint32).view(np.float32).astype(np.float64)


def quantize_rows_int16(v32):
    """Rows [..., N] of fp32 values -> (int16 codes [..., N], fp32 decode
    scales [...]): encode = 32767 / max|row| and decode = 1 / encode, both
    fp32 divisions; codes = round-half-even(fp32(v * encode))."""
    v = np.asarray(v32, dtype=np.float32)
    m = np.max(np.abs(v), axis=-1)
    zero = m == 0
    with np.errstate(divide="ignore"):
        enc = np.float32(INT16_MAX) / np.where(zero, np.float32(1), m).astype(np.float32)
    prod = (v * enc[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -INT16_MAX, INT16_MAX).astype(np.int16)
    dec = (np.float32(1) / enc).astype(np.float32)
    codes[zero] = 0
    dec = np.where(zero, np.float32(0), dec).astype(np.float32)
    return codes, dec


def dequantize_rows_int16(codes, dec):
    """int16 codes and fp32 decode scales -> fp32 values (one fp32 product)."""
    return (np.asarray(codes, dtype=np.float32) * np.asarray(dec, np.float32)[..., None]
            ).astype(np.float32)


def encode_state(v, fmt: str, seed: int = 0, philox_rounds: int = 0, start: int = 0):
    """fp64 state [..., N] -> (stored values as float64, int16 scales or None).
    For INT16 the stored values are the decoded fp32 values of the codes and
    the second result is (codes, decode scales).  ``start`` is the flat index
    of v's first element in the whole state (the Philox counter); fp16 is
    rounded stochastically when philox_rounds > 0."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    if fmt == F32:
        return v32.astype(np.float64), None
    if fmt == BF16:
        return round_bf16_nearest(v32), None
    if fmt == F16:
        if philox_rounds <= 0:
            return round_f16_nearest(v32), None
        flat = v32.reshape(-1)
        r = state_random_bits(flat.size, seed, start, philox_rounds)
        return round_f16_stochastic(flat, r).reshape(v32.shape), None
    if fmt == INT16:
        codes, dec = quantize_rows_int16(v32)
        return dequantize_rows_int16(codes, dec).astype(np.float64), (codes, dec)
    raise ValueError("unknown state format %r" % fmt)


def decode_step_lowp(state, x_t, dt_t, B_t, C_t, A, D, fmt: str, seed: int = 0,
                     philox_rounds: int = 0, dt_bias=None, dt_softplus: bool = False,
                     z_t=None, pairs: Optional[Sequence[int]] = None):
    """One decode step on a state stored in ``fmt``.

    ``state`` [Bt,H,P,N] (or [npairs,P,N] for the (b, h) pairs b*H+h listed
    in ``pairs``) float64 holds the values the stored state decodes to (for
    INT16: codes times decode scales, one fp32 product).  The step is the
    oracle's fp64 decode step on those values; the new state is then encoded
    as the format stores it (fp16 stochastically when ``philox_rounds`` > 0,
    Philox key = ``seed``, counters
    from each element's flat index in the whole [Bt,H,P,N] state).
    Returns (y [Bt,H,P] or [npairs,P] from the unrounded new state, new
    stored values shaped like ``state``, (codes, scales) for INT16 else None)."""
    from . import token_decode
    P, N = state.shape[-2], state.shape[-1]
    run = np.ascontiguousarray(state, dtype=np.float64).reshape(-1, P, N).copy()
    y = token_decode(run, x_t, dt_t, B_t, C_t, A, D, pairs=pairs, dt_bias=dt_bias,
                     dt_softplus=dt_softplus, z_t=z_t)
    idx = range(run.shape[0]) if pairs is None else pairs
    stored = np.empty_like(run)
    codes = np.empty(run.shape, np.int16) if fmt == INT16 else None
    scales = np.empty(run.shape[:2], np.float32) if fmt == INT16 else None
    for i, pr in enumerate(idx):
        stored[i], extra = encode_state(run[i], fmt, seed, philox_rounds, start=int(pr) * P * N)
        if extra is not None:
            codes[i], scales[i] = extra
    shape = state.shape
    return (y.reshape(shape[:-1]), stored.reshape(shape),
            None if codes is None else (codes.reshape(shape), scales.reshape(shape[:-1])))
