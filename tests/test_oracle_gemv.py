"""Pins of the oracle's decode products ("GPU acceleration", "Where GPU time goes": the
weight-reading GEMVs consume fp4 directly; y = x * W_eff^T).

- exact rational arithmetic on small cases: the float64 GEMV equals the exact sum to within
  float64 rounding, with the dequantized weight taken apart from the bit fields here;
- one-hot x picks out a dequantized column exactly;
- small-M rows equal the GEMV of each row; M = 1 is the GEMV;
- the bf16 GEMV against the same exact sum.
"""
from fractions import Fraction

import numpy as np

import oracle as O
from nvfp4_weight_only_rtn_amd import inputs


def _field_dequant(codes, scales, ts, seg_end, N, K):
    """Exact Fractions from the raw bit fields, written independently of the oracle helpers."""
    rows = []
    seg_of = []
    start = 0
    for k, end in enumerate(seg_end):
        seg_of += [k] * (end - start)
        start = end
    for i in range(N):
        row = []
        for j in range(K):
            byte = int(codes[i, j // 2])
            nib = (byte >> 4) if (j % 2) else (byte & 0xF)
            e, m = (nib >> 1) & 3, nib & 1
            mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
            if nib & 8:
                mag = -mag
            sc = int(scales[i, j // 16])
            se, sm = (sc >> 3) & 0xF, sc & 7
            sv = Fraction(sm, 8) * Fraction(1, 64) if se == 0 else (1 + Fraction(sm, 8)) * Fraction(2) ** (se - 7)
            row.append(mag * sv * Fraction(float(ts[seg_of[i]])))
        rows.append(row)
    return rows


def test_gemv_equals_exact_rational_sum():
    N, K = 7, 64
    W, s, U, V = inputs.theta_bundle(N, K, 4, cfg=9, layer=8, proj=0)
    We = O.reconstruct(W, s, U, V)
    seg_end = [3, 5, 7]
    codes, scales, ts = O.quantize(We, seg_end)
    x = inputs.activation_bf16(1, K, 9, 8, 0)
    xf = [Fraction(float(v)) for v in O.bf16_to_f32(x)[0]]
    D = _field_dequant(codes, scales, ts, seg_end, N, K)
    y = O.gemv_nvfp4(codes, scales, ts, x, seg_end)
    for i in range(N):
        exact = sum(a * b for a, b in zip(xf, D[i]))
        mag = sum(abs(a * b) for a, b in zip(xf, D[i]))
        assert abs(Fraction(float(y[i])) - exact) <= mag * Fraction(1, 2 ** 50)
    # the exact dequantized values match the oracle's float64 dequantization bit for bit
    deq = O.dequantize(codes, scales, ts, seg_end)
    assert all(Fraction(float(deq[i, j])) == D[i][j] for i in range(N) for j in range(K))


def test_one_hot_selects_a_column():
    N, K = 16, 96
    W, _, _, _ = inputs.theta_bundle(N, K, 0, cfg=9, layer=9, proj=0, passthrough=True)
    codes, scales, ts = O.quantize(W)
    deq32 = O.dequantize_f32(codes, scales, ts)
    for k in (0, 17, 95):
        x = np.zeros((1, K), dtype=np.uint16)
        x[0, k] = 0x3F80
        y = O.gemv_nvfp4(codes, scales, ts, x)
        assert np.array_equal(y.astype(np.float32), deq32[:, k])


def test_small_m_rows_are_gemvs():
    N, K, M = 40, 128, 5
    W, _, _, _ = inputs.theta_bundle(N, K, 0, cfg=9, layer=10, proj=0, passthrough=True)
    codes, scales, ts = O.quantize(W, [24, 40])
    X = inputs.activation_bf16(M, K, 9, 10, 0)
    Y = O.gemm_nvfp4_small_m(codes, scales, ts, X, [24, 40])
    for m in range(M):
        assert np.allclose(Y[m], O.gemv_nvfp4(codes, scales, ts, X[m], [24, 40]), rtol=0, atol=1e-12)
    Y1 = O.gemm_nvfp4_small_m(codes, scales, ts, X[:1], [24, 40])
    assert np.allclose(Y1[0], O.gemv_nvfp4(codes, scales, ts, X[0], [24, 40]), rtol=0, atol=1e-12)


def test_row_subset_matches_full():
    N, K = 300, 64
    W, _, _, _ = inputs.theta_bundle(N, K, 0, cfg=9, layer=11, proj=0, passthrough=True)
    codes, scales, ts = O.quantize(W, [100, 300])
    x = inputs.activation_bf16(1, K, 9, 11, 0)
    full = O.gemv_nvfp4(codes, scales, ts, x, [100, 300], chunk_rows=64)
    rows = np.array([0, 99, 100, 257, 299])
    assert np.array_equal(O.gemv_nvfp4(codes, scales, ts, x, [100, 300], rows=rows), full[rows])


def test_bf16_gemv_exact():
    N, K = 6, 40
    W = inputs.normal_bf16((N, K), 0.02, 9, 12, 0, 0)
    x = inputs.activation_bf16(1, K, 9, 12, 0)
    y = O.gemv_bf16(W, x)
    wf, xf = O.bf16_to_f32(W), O.bf16_to_f32(x)[0]
    for i in range(N):
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(wf[i], xf))
        mag = sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(wf[i], xf))
        assert abs(Fraction(float(y[i])) - exact) <= mag * Fraction(1, 2 ** 50)
