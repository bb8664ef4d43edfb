"""Pins of the oracle's runtime low-rank product over a shared NVFP4 block ("Throughput", the
runtime reconstruction path; weightless "Custom-op kernel", "Trained weight sharing"):
y = s * (x . deq(W0)^T) + U (V^T x), the weight never rebuilt.

- exact rational arithmetic: every input is a dyadic rational (bf16, E2M1 x E4M3 x fp32), so
  the exact y is a finite sum of Fractions; the float64 oracle must sit within float64 rounding
  of it. The shapes are non-square (N != K != r) so a transposed factor cannot line up;
- r = 0 without s is the plain GEMV, bit for bit; r = 0 with s is the GEMV scaled row by row;
- one projection's delta is additive: y(U, V) - y(no U, V) is U (V^T x) to float64 rounding,
  and splitting the rank into two halves adds up to the whole.
"""
from fractions import Fraction

import numpy as np

import oracle as O
from nvfp4_weight_only_rtn_amd import inputs
from test_oracle_gemv import _field_dequant


def _bf16_fraction(bits) -> Fraction:
    """Exact value of one bf16 bit pattern from its fields (finite values only)."""
    b = int(bits)
    sign = -1 if b & 0x8000 else 1
    e, m = (b >> 7) & 0xFF, b & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(2) ** -126
    return sign * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def _shared_block(N, K, layer):
    W0, _, _, _ = inputs.theta_bundle(N, K, 0, cfg=9, layer=layer, proj=0, passthrough=True)
    return O.quantize(W0)


def test_lowrank_equals_exact_rational_sum():
    N, K, r = 6, 64, 3
    codes, scales, ts = _shared_block(N, K, 60)
    _, s, U, V = inputs.theta_bundle(N, K, r, cfg=9, layer=60, proj=1, uv_sigma=0.05)
    x = inputs.activation_bf16(1, K, 9, 60, 1)
    D = _field_dequant(codes, scales, ts, [N], N, K)
    xf = [_bf16_fraction(v) for v in x[0]]
    sf = [_bf16_fraction(v) for v in s]
    Uf = [[_bf16_fraction(U[i, j]) for j in range(r)] for i in range(N)]
    Vf = [[_bf16_fraction(V[k, j]) for j in range(r)] for k in range(K)]
    t = [sum(Vf[k][j] * xf[k] for k in range(K)) for j in range(r)]
    tmag = [sum(abs(Vf[k][j] * xf[k]) for k in range(K)) for j in range(r)]
    y = O.gemv_nvfp4_lowrank(codes, scales, ts, s, U, V, x)
    for i in range(N):
        base = sum(a * b for a, b in zip(xf, D[i]))
        delta = sum(Uf[i][j] * t[j] for j in range(r))
        exact = sf[i] * base + delta
        mag = abs(sf[i]) * sum(abs(a * b) for a, b in zip(xf, D[i])) + sum(abs(Uf[i][j]) * tmag[j] for j in range(r))
        assert delta != 0 and abs(delta) > mag * Fraction(1, 2 ** 20)   # the low-rank term is visible
        assert abs(Fraction(float(y[i])) - exact) <= mag * Fraction(1, 2 ** 48)
    # the magnitude helper matches the same sums
    am = O.abs_lowrank(s, U, V, x, O.abs_dot(codes, scales, ts, x)[0])
    for i in range(N):
        mag = abs(sf[i]) * sum(abs(a * b) for a, b in zip(xf, D[i])) + sum(abs(Uf[i][j]) * tmag[j] for j in range(r))
        assert abs(Fraction(float(am[i])) - mag) <= mag * Fraction(1, 2 ** 48)


def test_rank_zero_reduces_to_the_gemv():
    N, K = 40, 160
    codes, scales, ts = _shared_block(N, K, 61)
    _, s, _, _ = inputs.theta_bundle(N, K, 0, cfg=9, layer=61, proj=1)
    x = inputs.activation_bf16(1, K, 9, 61, 1)
    y0 = O.gemv_nvfp4(codes, scales, ts, x)
    assert np.array_equal(O.gemv_nvfp4_lowrank(codes, scales, ts, None, None, None, x), y0)
    ys = O.gemv_nvfp4_lowrank(codes, scales, ts, s, None, None, x)
    assert np.array_equal(ys, y0 * O.bf16_to_f32(s).astype(np.float64))


def test_rank_halves_add_up_and_rows_select():
    N, K, r = 24, 96, 8
    codes, scales, ts = _shared_block(N, K, 62)
    _, s, U, V = inputs.theta_bundle(N, K, r, cfg=9, layer=62, proj=1, uv_sigma=0.05)
    x = inputs.activation_bf16(1, K, 9, 62, 1)
    y = O.gemv_nvfp4_lowrank(codes, scales, ts, s, U, V, x)
    ys = O.gemv_nvfp4_lowrank(codes, scales, ts, s, None, None, x)
    ya = O.gemv_nvfp4_lowrank(codes, scales, ts, s, U[:, :4], V[:, :4], x)
    yb = O.gemv_nvfp4_lowrank(codes, scales, ts, s, U[:, 4:], V[:, 4:], x) - ys
    mag = O.abs_lowrank(s, U, V, x, O.abs_dot(codes, scales, ts, x)[0])
    assert np.all(np.abs((ya + yb) - y) <= mag * 2.0 ** -48)
    rows = np.array([23, 0, 7])
    assert np.array_equal(O.gemv_nvfp4_lowrank(codes, scales, ts, s, U, V, x, rows=rows), y[rows])
