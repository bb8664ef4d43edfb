"""Pins of the oracle's number formats (bf16, E4M3FN, E2M1) against things other than itself.

- bf16 rounding: torch's float32 -> bfloat16 cast (a library routine) plus hand-chosen ties.
- E4M3FN: exhaustive round trip over all finite codes, brute-force nearest search with
  even-code ties over a sweep of every midpoint, torch's float8_e4m3fn cast, and the
  format limits (448 max, 2^-9 smallest subnormal).
- E2M1: the grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} round-trips, brute-force nearest search
  with even-code ties on a dense sweep including every midpoint.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O


# ----------------------------------------------------------------------------- bf16
def test_bf16_rne_matches_torch_cast_random():
    g = np.random.default_rng(1)
    bits = g.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    a = bits.view(np.float32)
    a = a[np.isfinite(a)]
    ours = O.f32_to_bf16_rne(a)
    ref = torch.from_numpy(a.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_rne_ties_and_specials():
    cases = {
        0x3F808000: 0x3F80,   # 1 + 2^-8 exactly between 1 and 1+2^-7: tie -> even (keep)
        0x3F818000: 0x3F82,   # tie with odd kept LSB -> round up
        0x3F808001: 0x3F81,   # just above the tie -> up
        0x3F807FFF: 0x3F80,   # just below -> down
        0x7F7FFFFF: 0x7F80,   # largest finite fp32 rounds to +inf
        0x80000000: 0x8000,   # -0 stays -0
        0x7F800000: 0x7F80,   # +inf
        0xFF800000: 0xFF80,   # -inf
        0x00000001: 0x0000,   # smallest fp32 subnormal rounds to +0
    }
    a = np.array(list(cases.keys()), dtype=np.uint32).view(np.float32)
    out = O.f32_to_bf16_rne(a)
    assert [int(v) for v in out] == list(cases.values())
    nan = O.f32_to_bf16_rne(np.array([np.nan], dtype=np.float32))
    assert np.isnan(O.bf16_to_f32(nan)).all()


def test_bf16_to_f32_is_exact_embedding():
    b = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f32(b)
    fin = np.isfinite(f)
    assert np.array_equal(O.f32_to_bf16_rne(f[fin]), b[fin])


# ----------------------------------------------------------------------------- E4M3
def _e4m3_table():
    """All finite non-negative E4M3FN values from the bit layout, as exact Fractions."""
    vals = []
    for c in range(0x7F):                    # 0x7F is NaN
        e, m = c >> 3, c & 7
        if e == 0:
            v = Fraction(m, 8) * Fraction(1, 2**6)
        else:
            v = (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))
        vals.append(v)
    return vals


E4M3_VALUES = _e4m3_table()


def _brute_e4m3(x: float) -> int:
    """Nearest finite E4M3 value by exhaustive search; ties go to the even code."""
    fx = Fraction(x)
    best, best_d = None, None
    for c, v in enumerate(E4M3_VALUES):
        d = abs(v - fx)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def test_e4m3_format_limits():
    assert float(E4M3_VALUES[0x7E]) == 448.0
    assert float(E4M3_VALUES[1]) == 2.0 ** -9
    assert float(E4M3_VALUES[0x38]) == 1.0
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_e4m3_decode_encode_roundtrip_all_codes():
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    assert [Fraction(float(v)) for v in vals] == E4M3_VALUES
    assert np.array_equal(O.e4m3_encode_rne_satfinite(vals.astype(np.float32)), codes)


def test_e4m3_encoder_equals_brute_force_on_midpoint_sweep():
    xs = []
    for a, b in zip(E4M3_VALUES[:-1], E4M3_VALUES[1:]):
        mid = (a + b) / 2
        m32 = np.float32(float(mid))
        xs += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
               np.float32(float(a)), np.float32(float((3 * a + b) / 4))]
    xs += [np.float32(v) for v in (448.0, 460.0, 464.0, 470.0, 1e6, 2.0 ** -10, 2.0 ** -11, 0.0)]
    xs = np.array(xs, dtype=np.float32)
    ours = O.e4m3_encode_rne_satfinite(xs)
    brute = np.array([_brute_e4m3(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(ours, brute)


def test_e4m3_encoder_matches_torch_cast_in_range():
    g = np.random.default_rng(2)
    x = np.concatenate([
        g.uniform(0, 448, 100_000), np.exp2(g.uniform(-12, 8.8, 100_000)),
    ]).astype(np.float32)
    x = x[x <= 448]
    ours = O.e4m3_encode_rne_satfinite(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates_and_underflows():
    x = np.array([448.0, 449.0, 464.0, 1e30, np.inf, 2.0 ** -10, 1.0000001 * 2.0 ** -10, 0.0],
                 dtype=np.float32)
    assert list(O.e4m3_encode_rne_satfinite(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x00, 0x01, 0x00]
    assert O.e4m3_encode_rne_satfinite(np.array([np.nan], np.float32))[0] == 0x7F


# ----------------------------------------------------------------------------- E2M1
GRID = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _brute_e2m1(a: float) -> int:
    fa = Fraction(a)
    best, best_d = None, None
    for c, v in enumerate(GRID):
        d = abs(v - fa)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def test_e2m1_grid_roundtrip():
    codes = np.arange(16, dtype=np.uint8)
    vals = O.e2m1_decode(codes)
    assert list(np.abs(vals[:8])) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(vals[8:]) == [-v for v in vals[:8]]
    mags = O.e2m1_encode_magnitude(np.abs(vals).astype(np.float32))
    assert np.array_equal(mags, codes & 7)


def test_e2m1_encoder_equals_brute_force_dense_sweep():
    xs = list(np.linspace(0, 8, 20001, dtype=np.float32))
    for a, b in zip(GRID[:-1], GRID[1:]):
        m = np.float32(float((a + b) / 2))
        xs += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(9))]
    xs += [np.float32(v) for v in (6.0, 7.0, 1e30)]
    xs = np.array(xs, dtype=np.float32)
    ours = O.e2m1_encode_magnitude(xs)
    brute = np.array([_brute_e2m1(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(ours, brute)


@pytest.mark.parametrize("mid,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)])
def test_e2m1_midpoints_go_to_even_code(mid, code):
    assert O.e2m1_encode_magnitude(np.array([mid], np.float32))[0] == code
