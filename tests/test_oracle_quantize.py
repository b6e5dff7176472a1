"""Pins for the oracle's activation quantizers (per-row absmax int8, q8_0
blocks) and its f32 -> f16 rounding.

Each pin comes from outside the oracle's own code: values worked by hand from
the page's rule ("web-xpu-ops": quantize, absmax to int8 in [-127, 127],
reciprocal 127/absmax in f64, Math.round with ties toward +infinity), exact
round trips of values that are already d * q with d a power of two, a brute
force that rounds with exact rationals instead of floor/frac, and numpy's own
f32 -> f16 conversion.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
import workloads as wl


def test_hand_worked_ties_toward_plus_infinity():
    # absmax 127 makes the reciprocal exactly 1, so each code is Math.round(x)
    x = np.array([127, -127, 63.5, -63.5, 0.5, -0.5, 1.5, -1.5, 2.4999998, 100.49, -0.49, 0.0], dtype=np.float32)
    q, s = oracle.quantize_absmax_int8(x)
    assert q.tolist() == [127, -127, 64, -63, 1, 0, 2, -1, 2, 100, 0, 0]
    assert s.tolist() == [1.0]


def test_hand_worked_scaled_row():
    # absmax 2: reciprocal 63.5; 1.0 -> 63.5 -> 64 (tie up); -1.0 -> -63.5 -> -63
    x = np.array([2.0, -1.0, 1.0, -2.0, 0.25], dtype=np.float32)
    q, s = oracle.quantize_absmax_int8(x)
    assert q.tolist() == [127, -63, 64, -127, 16]        # 0.25 * 63.5 = 15.875 -> 16
    assert s[0] == np.float32(2.0 / 127.0)


@pytest.mark.parametrize("e", [-20, -3, 0, 5, 30])
def test_power_of_two_round_trip(e):
    rng = np.random.default_rng(e + 100)
    d = 2.0 ** e
    q = rng.integers(-127, 128, size=(6, 96))
    q[:, 7] = 127 * np.where(np.arange(6) % 2, 1, -1)     # every row reaches |q| = 127
    x = (q * d).astype(np.float32)
    got, s = oracle.quantize_absmax_int8(x)
    assert np.array_equal(got, q.astype(np.int8))
    assert np.all(s == np.float32(d))


def test_q8_0_power_of_two_round_trip():
    rng = np.random.default_rng(5)
    n, K = 3, 128
    q = rng.integers(-127, 128, size=(n, K))
    q.reshape(n, K // 32, 32)[:, :, 3] = 127
    es = rng.integers(-14, 10, size=(n, K // 32))         # f16 normal range
    d = np.repeat(2.0 ** es, 32, axis=1)
    x = (q * d).astype(np.float32)
    out = oracle.quantize_q8_0(x).reshape(n, K // 32, 34)
    dbits = out[:, :, 0].astype(np.uint16) | (out[:, :, 1].astype(np.uint16) << 8)
    want_d = np.float16(2.0 ** es.astype(np.float64)).view(np.uint16)
    assert np.array_equal(dbits, want_d)
    assert np.array_equal(out[:, :, 2:].view(np.int8).reshape(n, K), q.astype(np.int8))


def test_zero_rows_and_blocks():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 40] = -3.0
    q, s = oracle.quantize_absmax_int8(x)
    assert not q[0].any() and s[0] == 0.0 and q[1, 40] == -127
    out = oracle.quantize_q8_0(x).reshape(2, 2, 34)
    assert not out[0].any() and not out[1, 0].any()
    assert out[1, 1, 2 + 8].view(np.int8) == -127


def _math_round_exact(v: float) -> int:
    """Math.round of the f64 value v with exact rationals: floor(v + 1/2)."""
    return math.floor(Fraction(v) + Fraction(1, 2))


def test_brute_force_exact_rationals():
    rng = np.random.default_rng(9)
    x = rng.standard_normal(size=(12, 64)).astype(np.float32)
    x[3] *= 1e-30
    x[4] *= 1e30
    x[5, ::7] = 0.0
    q, s = oracle.quantize_absmax_int8(x)
    for r in range(x.shape[0]):
        amax = max(abs(float(v)) for v in x[r])
        inv = 127.0 / amax                       # Python floats are IEEE f64
        for j in range(x.shape[1]):
            want = max(-127, min(127, _math_round_exact(float(x[r, j]) * inv)))
            assert q[r, j] == want, (r, j)
        assert s[r] == np.float32(amax / 127.0)
    blocks = oracle.quantize_q8_0(x).reshape(12, 2, 34)
    for r in range(x.shape[0]):
        for i in range(2):
            xb = [float(v) for v in x[r, 32 * i:32 * i + 32]]
            amax = max(abs(v) for v in xb)
            codes = blocks[r, i, 2:].view(np.int8)
            dbits = int(blocks[r, i, 0]) | (int(blocks[r, i, 1]) << 8)
            if amax == 0.0:
                assert not codes.any() and dbits == 0
                continue
            inv = 127.0 / amax
            assert codes.tolist() == [max(-127, min(127, _math_round_exact(v * inv))) for v in xb]
            with np.errstate(over="ignore"):     # amax / 127 past the f16 range is infinity
                assert dbits == int(np.float16(np.float32(amax / 127.0)).view(np.uint16))


def test_invariants_random():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(size=(40, 512)) * rng.uniform(1e-3, 1e3, size=(40, 1))).astype(np.float32)
    q, s = oracle.quantize_absmax_int8(x)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)   # the absmax element maps to +-127
    err = np.abs(x.astype(np.float64) - s[:, None].astype(np.float64) * q)
    assert np.all(err <= s[:, None] * (0.5 + 1e-6))


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(13)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    edges = np.array([0.0, -0.0, 1.0, 65504.0, 65519.996, 65520.0, 1e9, 2.0**-24, 2.0**-25, 3 * 2.0**-26,
                      2.0**-25 * 1.0000001, 2.0**-14, 2.0**-14 * (1 - 2.0**-11), 0.1, 1 / 127, np.inf, -np.inf],
                     dtype=np.float32)
    # keep the random patterns in and around the f16 range (plus a tail beyond it)
    sel = vals[np.isfinite(vals) & (np.abs(vals) < 1e6) & ((np.abs(vals) > 1e-9) | (vals == 0))]
    for v in np.concatenate([edges, sel[:40000]]):
        with np.errstate(over="ignore"):
            want = int(np.array(v, dtype=np.float32).astype(np.float16).view(np.uint16))
        assert oracle.f32_to_f16_bits(v) == want, float(v)
    nan_bits = oracle.f32_to_f16_bits(np.float32("nan"))
    assert (nan_bits & 0x7c00) == 0x7c00 and (nan_bits & 0x3ff) != 0


def test_input_recipe_agrees_with_oracle():
    """The ternary workloads' int8 activation recipe is the same rule."""
    rng = np.random.default_rng(17)
    for K in (32, 2560, 6912):
        x = rng.standard_normal(size=K)
        want_q, want_s = wl.absmax_int8(x)
        q, s = oracle.quantize_absmax_int8(np.asarray(x, dtype=np.float64).astype(np.float32))
        # the recipe quantizes the f64 draw; the oracle takes f32 input, as the device does
        q32, s32 = wl.absmax_int8(np.asarray(x).astype(np.float32))
        assert np.array_equal(q, q32) and s[0] == s32
        assert want_q.shape == q.shape and want_s.dtype == np.float32
