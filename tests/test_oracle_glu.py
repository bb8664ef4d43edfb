"""Pins of the oracle's gate|up epilogue (h = act(gate) * up rounded to bf16).

What fixes it, independent of the oracle's own formula:
* closed forms: act(0) = 0; GELU-tanh and SiLU tend to g for large positive g and to 0 for large
  negative g; SiLU(g) = g * sigmoid(g) at a few hand values;
* odd-part identities: GELU-tanh(g) - GELU-tanh(-g) = g and SiLU(g) - SiLU(-g) = g for every g;
* a library cross-check: torch's float64 gelu(approximate="tanh") and silu;
* the bf16 rounding of the product: exact products stay exact, a value half-way between two bf16
  neighbours rounds to the even one, and the float32 intermediate does not double-round.
"""
import numpy as np
import pytest
import torch

import oracle as O


G = np.concatenate([np.linspace(-12, 12, 2001), [0.0, 1e-30, -1e-30, 50.0, -50.0]])


@pytest.mark.parametrize("act", [O.ACT_GELU_TANH, O.ACT_SILU])
def test_odd_part_identity(act):
    assert np.allclose(O.activation(G, act) - O.activation(-G, act), G, rtol=0, atol=1e-12)


def test_closed_forms():
    for act in (O.ACT_GELU_TANH, O.ACT_SILU, O.ACT_IDENTITY):
        assert O.activation(np.array([0.0]), act)[0] == 0.0
    for act in (O.ACT_GELU_TANH, O.ACT_SILU):
        assert abs(O.activation(np.array([40.0]), act)[0] - 40.0) < 1e-12
        assert abs(O.activation(np.array([-40.0]), act)[0]) < 1e-12
    # SiLU(g) = g / (1 + e^-g): at g = ln 3, sigmoid = 3/4
    assert abs(O.activation(np.array([np.log(3.0)]), O.ACT_SILU)[0] - 0.75 * np.log(3.0)) < 1e-15
    # GELU-tanh at the point where the tanh argument is atanh(1/2): 0.5 g (1 + 1/2)
    c = np.sqrt(2 / np.pi)
    from scipy.optimize import brentq
    g0 = brentq(lambda g: c * (g + 0.044715 * g ** 3) - np.arctanh(0.5), 0.0, 2.0)
    assert abs(O.activation(np.array([g0]), O.ACT_GELU_TANH)[0] - 0.75 * g0) < 1e-14
    assert np.array_equal(O.activation(G, O.ACT_IDENTITY), G)


def test_matches_torch_float64():
    t = torch.from_numpy(G)
    assert np.allclose(O.activation(G, O.ACT_GELU_TANH),
                       torch.nn.functional.gelu(t, approximate="tanh").numpy(), rtol=1e-14, atol=1e-15)
    assert np.allclose(O.activation(G, O.ACT_SILU), torch.nn.functional.silu(t).numpy(), rtol=1e-14, atol=1e-15)


def test_bf16_rounding_of_the_product():
    # exact products of bf16-representable values stay exact
    g = O.bf16_to_f32(np.array([0x3F80, 0x4000, 0xC040], np.uint16)).astype(np.float64)   # 1, 2, -3
    u = O.bf16_to_f32(np.array([0x3FC0, 0x3F00, 0x4080], np.uint16)).astype(np.float64)   # 1.5, 0.5, 4
    assert np.array_equal(O.glu(g, u, O.ACT_IDENTITY), np.array([0x3FC0, 0x3F80, 0xC140], np.uint16))
    # 1 + 2^-8 lies half-way between bf16 1 (even) and 1 + 2^-7: ties to even
    assert O.glu(np.array([1.0 + 2.0 ** -8]), np.array([1.0]), O.ACT_IDENTITY)[0] == 0x3F80
    # 1 + 3 * 2^-8 is half-way between 1 + 2^-7 (odd) and 1 + 2^-6: rounds up to the even one
    assert O.glu(np.array([1.0 + 3 * 2.0 ** -8]), np.array([1.0]), O.ACT_IDENTITY)[0] == 0x3F82
    # just above a tie by 2^-40: a float32 intermediate rounded to nearest would land on the tie
    # and round to even; the single rounding goes up
    assert O.glu(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]), np.array([1.0]), O.ACT_IDENTITY)[0] == 0x3F81
    assert O.glu(np.array([-(1.0 + 2.0 ** -8 + 2.0 ** -40)]), np.array([1.0]), O.ACT_IDENTITY)[0] == 0xBF81


def test_f64_to_bf16_matches_exact_rounding_on_random_values():
    """Brute force: among the three bf16 patterns around the float32 rounding, the nearest value
    wins, ties to the even pattern."""
    rng = np.random.default_rng(3)
    a = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))
    a = np.concatenate([a, 1.0 + (2 * rng.integers(0, 64, 200) + 1) * 2.0 ** -8])   # exact ties
    got = O.f64_to_bf16_rne(a)
    mid = O.f32_to_bf16_rne(a.astype(np.float32)).astype(np.int64)
    cand = np.stack([mid - 1, mid, mid + 1])
    err = np.abs(O.bf16_to_f32(cand.astype(np.uint16)).astype(np.float64) - a)
    is_min = err == err.min(axis=0)
    pick = np.where((is_min & (cand % 2 == 0)).any(axis=0), np.argmax(is_min & (cand % 2 == 0), axis=0),
                    np.argmax(is_min, axis=0))
    assert np.array_equal(got.astype(np.int64), cand[pick, np.arange(a.size)])


def test_hand_built_gate_up_pairs():
    """A two-segment [gate; up] weight built by hand (K = 32, F = 2 pairs), through the oracle's
    fused GEMV and its SiLU epilogue. Tensor scales: gate 0.5, up 2.0; E4M3 block scale 0x38 = 1.0,
    except block 0 of up row 1, 0x30 = 0.5. Codes (sign<<3 | index into 0 .5 1 1.5 2 3 4 6, the
    even element in the low nibble of a byte):
      gate row 0: element 0 = 4   (code 0x6, byte 0 = 0x06) -> g0 = 4 * 1 * 0.5 = 2
      gate row 1: element 1 = -2  (code 0xC, byte 0 = 0xC0) -> g1 = -2 * 1 * 0.5 = -1
      up row 0:   element 0 = 1.5 (code 0x3, byte 0 = 0x03) -> u0 = 1.5 * 1 * 2 = 3
      up row 1:   element 1 = 0.5 (code 0x1, byte 0 = 0x10) -> u1 = 0.5 * 0.5 * 2 = 0.5
    with x = e0 + e1. SiLU(g) = g / (1 + e^-g):
      h0 = SiLU(2) * 3 = 5.2847824...; bf16 step in [4, 8) is 2^-5: 169.11 steps -> 169 * 2^-5 =
           5.28125 = 0x40A9 (swapping gate and up gives SiLU(3) * 2 = 5.7154 -> 0x40B7);
      h1 = SiLU(-1) * 0.5 = -0.1344707...; step in [1/8, 1/4) is 2^-10: 137.70 steps -> 138 * 2^-10
           = 0.134765625, negative: 0xBE0A (swapped: SiLU(0.5) * -1 = -0.3112 -> 0xBE9F).
    The identity epilogue gives the exact products 6 = 0x40C0 and -0.5 = 0xBF00."""
    codes = np.zeros((4, 16), np.uint8)
    codes[0, 0], codes[1, 0], codes[2, 0], codes[3, 0] = 0x06, 0xC0, 0x03, 0x10
    scales = np.full((4, 2), 0x38, np.uint8)
    scales[3, 0] = 0x30
    ts = np.array([0.5, 2.0], np.float32)
    x = np.zeros(32, np.uint16)
    x[0] = x[1] = 0x3F80
    g, u = O.gemv_nvfp4_glu(codes, scales, ts, x)
    assert list(g) == [2.0, -1.0] and list(u) == [3.0, 0.5]
    assert list(O.glu(g, u, O.ACT_SILU)) == [0x40A9, 0xBE0A]
    assert list(O.glu(g, u, O.ACT_IDENTITY)) == [0x40C0, 0xBF00]
    # the hand values against the rounding of a float64 evaluation (math.exp, a library routine)
    import math
    for gv, uv, want in ((2.0, 3.0, 0x40A9), (-1.0, 0.5, 0xBE0A), (3.0, 2.0, 0x40B7), (0.5, -1.0, 0xBE9F)):
        h = gv / (1.0 + math.exp(-gv)) * uv
        step = 2.0 ** (math.floor(math.log2(abs(h))) - 7)
        assert O.bf16_to_f32(np.array([want], np.uint16))[0] == np.float32(round(h / step) * step)
