"""Pins of the oracle's reduced-precision decode state ("Optimizing Nemotron
v3 Super in TensorRT-LLM", section 6.5): the Philox-4x32 generator against
its published known-answer vectors, stochastic rounding to fp16 by exhaustive
enumeration of its 2^13 random inputs, round-to-nearest storage against
worked values, and the int16 row quantizer against its error bound."""

import numpy as np
import pytest

import oracle
from oracle import state_formats as sf


def words(v):
    return [int(w) for w in v]


# Known-answer vectors of Philox-4x32 with 10 rounds, published with the
# generator (Salmon et al., SC'11; the Random123 distribution's kat vectors):
# (counter, key) -> output.
KAT = [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    assert words(sf.philox4x32(np.array(ctr, np.uint64), np.array(key, np.uint64))) == out


def halves13(blk):
    """The 8 element fields of one block: word k // 2, low half for even k,
    high half for odd k, 13 bits each (written out element by element)."""
    out = []
    for wd in blk:
        out.append(int(wd) & 0x1FFF)
        out.append((int(wd) >> 16) & 0x1FFF)
    return out


def test_state_bits_take_one_block_per_eight_elements():
    seed = 0x123456789ABCDEF0
    r = sf.state_random_bits(8 * 1000 + 16, seed)
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint64)
    for first in (0, 8, 1240, 8008):
        blk = sf.philox4x32(np.array([first, 0, 0, 0], np.uint64), key)
        assert [int(v) for v in r[first:first + 8]] == halves13(blk)
    # bits 13..15 and 29..31 of each word are never used
    assert int(r.max()) < 8192
    # past 2^32 elements the index's high word is the counter's second word
    r = sf.state_random_bits(16, seed, start=(1 << 32) + 8)
    blk = sf.philox4x32(np.array([16, 1, 0, 0], np.uint64), key)
    assert [int(v) for v in r[8:]] == halves13(blk)


ALL_R = np.arange(8192)


@pytest.mark.parametrize("x", [1.0 + 0.3 * 2 ** -10, -3.7, 1234.567, 2.0 ** -14 * 1.77,
                               3.0e-6, -5.0e-8, 60000.3, 0.099991])
def test_stochastic_rounding_exhaustive(x):
    """Over all 2^13 random inputs the result is one of the two fp16
    neighbours of x (as fp32), rounds away from zero exactly
    frac * 2^13 times, and the results sum to 2^13 x: unbiased."""
    x32 = np.float32(x)
    q = sf.round_f16_stochastic(np.full(8192, x32), ALL_R)
    lo = float(np.float16(0))
    a = abs(float(x32))
    # the fp16 neighbours, from the fp16 grid itself
    grid = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    i = np.searchsorted(grid, a, side="right") - 1
    lo, hi = grid[i], grid[min(i + 1, len(grid) - 1)]
    qa = np.abs(q)
    assert set(np.unique(qa)) <= {lo, hi}
    if lo == a:
        assert np.all(qa == a)
        return
    frac8 = (a - lo) / (hi - lo) * 8192
    k = int(np.floor(frac8))
    assert int(np.sum(qa == hi)) == k
    if a >= 2.0 ** -14:
        assert frac8 == k                             # 13 bits: exactly unbiased
        assert np.sum(qa) == 8192 * a
    else:                                             # fp16 subnormal: bias < one step
        assert 0 <= 8192 * a - np.sum(qa) < hi - lo
    assert np.all(np.signbit(q) == np.signbit(x32))
    assert float(sf.round_f16_stochastic(x32, 0)) == np.copysign(lo, x32)   # r = 0: toward zero


def test_stochastic_rounding_fixed_points_and_saturation():
    exact = np.array([0.0, 1.0, -2.5, 65504.0, 2.0 ** -24, 2.0 ** -14, 1000.0], np.float32)
    for r in (0, 1, 4095, 8191):
        np.testing.assert_array_equal(sf.round_f16_stochastic(exact, r), exact)
    assert float(sf.round_f16_stochastic(np.float32(70000.0), 8191)) == 65504.0
    assert float(sf.round_f16_stochastic(np.float32(-65519.0), 8191)) == -65504.0


def test_nearest_roundings_worked_values():
    # fp16: 1 + 2^-11 is a tie between 1 and 1 + 2^-10 -> even (1)
    assert sf.round_f16_nearest(np.float32(1 + 2 ** -11)) == 1.0
    assert sf.round_f16_nearest(np.float32(1 + 3 * 2 ** -11)) == 1 + 2 ** -9
    # bf16: 8 significant bits; ties to even
    assert sf.round_bf16_nearest(np.float32(1 + 2 ** -8)) == 1.0
    assert sf.round_bf16_nearest(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6
    assert sf.round_bf16_nearest(np.float32(-(1 + 2 ** -8 + 2 ** -20))) == -(1 + 2 ** -7)
    rng = np.random.default_rng(0)
    v = rng.normal(0, 10, 10000).astype(np.float32)
    b = sf.round_bf16_nearest(v)
    e = np.floor(np.log2(np.abs(v).astype(np.float64)))
    step = 2.0 ** (e - 7)
    np.testing.assert_array_equal(b, np.round(v.astype(np.float64) / step) * step)


def test_int16_rows():
    rng = np.random.default_rng(1)
    v = (rng.normal(0, 1, (50, 128)) * rng.uniform(1e-3, 1e3, (50, 1))).astype(np.float32)
    v[7] = 0.0
    v[9, 5] = -1e4                       # one large value
    codes, dec = sf.quantize_rows_int16(v)
    assert codes.dtype == np.int16 and dec.dtype == np.float32
    assert np.all(np.abs(codes.astype(np.int64)) <= 32767)
    assert np.all(codes[7] == 0) and dec[7] == 0
    m = np.max(np.abs(v), axis=1)
    live = m > 0
    # the largest magnitude of each row maps to +-32767
    am = np.argmax(np.abs(v), axis=1)
    assert np.all(np.abs(codes[np.arange(50), am][live]) == 32767)
    assert np.all(dec[live] == np.float32(1) / (np.float32(32767) / m[live]))
    deq = sf.dequantize_rows_int16(codes, dec).astype(np.float64)
    err = np.abs(deq - v)
    assert np.all(err <= (0.5 + 1e-3) * dec[:, None].astype(np.float64) + 1e-7 * np.abs(v))
    assert codes[9, 5] == -32767


def test_encode_formats():
    rng = np.random.default_rng(2)
    v = rng.normal(0, 1, (2, 3, 4, 8))
    s32, _ = sf.encode_state(v, sf.F32)
    np.testing.assert_array_equal(s32, v.astype(np.float32))
    s16, _ = sf.encode_state(v, sf.F16)
    np.testing.assert_array_equal(s16, v.astype(np.float32).astype(np.float16))
    sr, _ = sf.encode_state(v, sf.F16, seed=7, philox_rounds=10)
    assert np.all(np.abs(sr - v) <= sf._ulp16(np.abs(v)) * (1 + 1e-9))
    si, (codes, dec) = sf.encode_state(v, sf.INT16)
    np.testing.assert_array_equal(si, codes.astype(np.float32) * dec[..., None])


def test_lowp_step_f32_is_the_plain_step():
    rng = np.random.default_rng(3)
    Bt, H, P, N, G = 2, 4, 8, 16, 2
    st = rng.normal(0, 0.3, (Bt, H, P, N))
    x = rng.normal(0, 1, (Bt, H, P)); dt = rng.uniform(0.01, 0.2, (Bt, H))
    B = rng.normal(0, 0.3, (Bt, G, N)); C = rng.normal(0, 0.3, (Bt, G, N))
    A = -rng.uniform(0.5, 4, H); D = rng.normal(0, 1, H)
    y, new, _ = sf.decode_step_lowp(st, x, dt, B, C, A, D, sf.F32)
    ref = st.reshape(Bt * H, P, N).copy()
    yr = oracle.token_decode(ref, x, dt, B, C, A, D)
    np.testing.assert_array_equal(y.reshape(-1, P), yr)
    np.testing.assert_array_equal(new.reshape(ref.shape), ref.astype(np.float32))


@pytest.mark.parametrize("fmt,stoch", [(sf.F16, True), (sf.INT16, False), (sf.BF16, False)])
def test_lowp_step_pair_subset_equals_full(fmt, stoch):
    rng = np.random.default_rng(4)
    Bt, H, P, N, G = 3, 4, 8, 16, 2
    st, _ = sf.encode_state(rng.normal(0, 0.3, (Bt, H, P, N)), fmt)
    x = rng.normal(0, 1, (Bt, H, P)); dt = rng.uniform(0.01, 0.2, (Bt, H))
    B = rng.normal(0, 0.3, (Bt, G, N)); C = rng.normal(0, 0.3, (Bt, G, N))
    A = -rng.uniform(0.5, 4, H); D = rng.normal(0, 1, H)
    y, new, ex = sf.decode_step_lowp(st, x, dt, B, C, A, D, fmt, seed=99, philox_rounds=10 * stoch)
    pr = [11, 0, 5]
    ys, news, exs = sf.decode_step_lowp(st.reshape(-1, P, N)[pr], x, dt, B, C, A, D, fmt,
                                        seed=99, philox_rounds=10 * stoch, pairs=pr)
    np.testing.assert_array_equal(ys, y.reshape(-1, P)[pr])
    np.testing.assert_array_equal(news, new.reshape(-1, P, N)[pr])
    if ex is not None:
        np.testing.assert_array_equal(exs[0], ex[0].reshape(-1, P, N)[pr])
