"""Pins of the oracle's runtime low-rank product over a shared NVFP4 block ("Throughput", the
runtime reconstruction path; weightless "Custom-op kernel", "Trained weight sharing"):
y = s * (x . deq(W0)^T) + U (V^T x), the weight never rebuilt.

- exact rational arithmetic: every input is a dyadic rational (bf16, E2M1 x E4M3 x fp32), so
  the exact y is a finite sum of Fractions; the float64 oracle must sit within float64 rounding
  of it. The shapes are non-square (N != K != r) so a transposed factor cannot line up;
- r = 0 without s is the plain GEMV, bit for bit; r = 0 with s is the GEMV scaled row by row;
- the delta is additive over the rank: splitting it into two halves adds up to the whole.
Each segment of a fused weight is one projection with its own factors (V is [n_seg, K, r]); the
rational pin uses two segments so a row paired with the other segment's V fails it.
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


def _shared_block(N, K, layer, seg_end=None):
    W0, _, _, _ = inputs.theta_bundle(N, K, 0, cfg=9, layer=layer, proj=0, passthrough=True)
    return O.quantize(W0, seg_end)


def _segment_factors(seg_end, K, r, layer):
    """Per-segment (s, U, V) as for fused projections: U rows follow the fused rows, V is [n_seg, K, r]."""
    s, U, V, start = [], [], [], 0
    for g, end in enumerate(seg_end):
        _, sg, Ug, Vg = inputs.theta_bundle(end - start, K, r, cfg=9, layer=layer, proj=1 + g, uv_sigma=0.05)
        s.append(sg); U.append(Ug); V.append(Vg)
        start = end
    return np.concatenate(s), np.concatenate(U), np.stack(V)


def test_lowrank_equals_exact_rational_sum():
    N, K, r = 7, 64, 3
    seg_end = [2, 7]
    codes, scales, ts = _shared_block(N, K, 60, seg_end)
    s, U, V = _segment_factors(seg_end, K, r, 60)
    x = inputs.activation_bf16(1, K, 9, 60, 1)
    D = _field_dequant(codes, scales, ts, seg_end, N, K)
    xf = [_bf16_fraction(v) for v in x[0]]
    sf = [_bf16_fraction(v) for v in s]
    Uf = [[_bf16_fraction(U[i, j]) for j in range(r)] for i in range(N)]
    seg_of = [0 if i < seg_end[0] else 1 for i in range(N)]
    t, tmag = [], []
    for g in range(2):
        Vf = [[_bf16_fraction(V[g, k, j]) for j in range(r)] for k in range(K)]
        t.append([sum(Vf[k][j] * xf[k] for k in range(K)) for j in range(r)])
        tmag.append([sum(abs(Vf[k][j] * xf[k]) for k in range(K)) for j in range(r)])
    y = O.gemv_nvfp4_lowrank(codes, scales, ts, s, U, V, x, seg_end)
    am = O.abs_lowrank(s, U, V, x, O.abs_dot(codes, scales, ts, x, seg_end)[0], seg_end)
    for i in range(N):
        g = seg_of[i]
        base = sum(a * b for a, b in zip(xf, D[i]))
        delta = sum(Uf[i][j] * t[g][j] for j in range(r))
        exact = sf[i] * base + delta
        mag = abs(sf[i]) * sum(abs(a * b) for a, b in zip(xf, D[i])) + \
            sum(abs(Uf[i][j]) * tmag[g][j] for j in range(r))
        assert delta != 0 and abs(delta) > mag * Fraction(1, 2 ** 20)   # the low-rank term is visible
        assert abs(Fraction(float(y[i])) - exact) <= mag * Fraction(1, 2 ** 48)
        # the magnitude helper matches the same sums
        assert abs(Fraction(float(am[i])) - mag) <= mag * Fraction(1, 2 ** 48)
    # the rows argument selects from the full result
    rows = np.array([6, 1, 2])
    assert np.array_equal(O.gemv_nvfp4_lowrank(codes, scales, ts, s, U, V, x, seg_end, rows=rows), y[rows])


def test_rank_zero_reduces_to_the_gemv():
    N, K = 40, 160
    codes, scales, ts = _shared_block(N, K, 61)
    _, s, _, _ = inputs.theta_bundle(N, K, 0, cfg=9, layer=61, proj=1)
    x = inputs.activation_bf16(1, K, 9, 61, 1)
    y0 = O.gemv_nvfp4(codes, scales, ts, x)
    assert np.array_equal(O.gemv_nvfp4_lowrank(codes, scales, ts, None, None, None, x), y0)
    ys = O.gemv_nvfp4_lowrank(codes, scales, ts, s, None, None, x)
    assert np.array_equal(ys, y0 * O.bf16_to_f32(s).astype(np.float64))


def test_rank_halves_add_up():
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
    # one segment given as [K, r] or as [1, K, r] is the same product
    assert np.array_equal(O.gemv_nvfp4_lowrank(codes, scales, ts, s, U, V[None], x), y)
