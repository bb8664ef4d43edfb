"""Edge cases across the entry points, against the float64 oracle:

* the segment table at its limit: four segments, some of them one row long, in every launch
  class of the GEMV, in the small-M product and in the runtime low-rank product (one factor
  set per segment);
* activations at extreme magnitudes (2^100, -2^100 and 2^-100 next to ordinary values) and with
  exact zeros and a negative zero, where fp32 accumulation must neither overflow nor lose the large terms;
* the smallest gate|up (F = 1) and a one-row weight in the small-M product;
* non-finite activations (+inf, NaN) in the GEMV and both small-M kernels: the NaN / +-inf
  pattern of every output equals the float64 oracle's, and other tokens are unaffected.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import assert_close_products, dev, gpu_quantize, host, oracle_quantize, say
from nvfp4_weight_only_rtn_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def _bundles(segs, K, layer):
    return [inputs.theta_bundle(n, K, 0, cfg=9, layer=layer, proj=i, passthrough=True) for i, n in enumerate(segs)]


FOUR_SEGMENTS = [((1, 1, 1, 5), 96), ((1, 300, 1, 2000), 1152), ((1, 4095, 1, 2048), 5376), ((513, 1, 1, 1), 21504),
                 ((1, 64, 1, 63), 8192 + 32)]


@pytest.mark.parametrize("segs,K", FOUR_SEGMENTS)
def test_gemv_four_segments(A, segs, K):
    what = f"gemv segments {segs} K {K}"
    say(what)
    b = _bundles(segs, K, 90)
    W, seg_end = gpu_quantize(A, b, K)
    c, s, t, _ = oracle_quantize(b)
    x = inputs.activation_bf16(1, K, 9, 90, len(segs))
    y = torch.full((W.N,), float("nan"), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, dev(x.reshape(-1)), y)
    torch.cuda.synchronize()
    assert_close_products(host(y), O.gemv_nvfp4(c, s, t, x, seg_end), O.abs_dot(c, s, t, x, seg_end)[0], what)


@pytest.mark.parametrize("M", [1, 4, 7])
def test_small_m_four_segments(A, M):
    segs, K = (1, 37, 1, 90), 1184
    what = f"small-M segments {segs} M {M}"
    say(what)
    b = _bundles(segs, K, 91)
    W, seg_end = gpu_quantize(A, b, K)
    c, s, t, _ = oracle_quantize(b)
    X = inputs.activation_bf16(M, K, 9, 91, M)
    Y = torch.full((M, W.N), float("nan"), dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m(W, dev(X), Y)
    torch.cuda.synchronize()
    Yr = O.gemm_nvfp4_small_m(c, s, t, X, seg_end)
    ad = O.abs_dot(c, s, t, X, seg_end)
    for m in range(M):
        assert_close_products(host(Y)[m], Yr[m], ad[m], f"{what} token {m}")


def test_lowrank_four_segments(A):
    segs, K, r = (1, 200, 1, 55), 2080, 8
    say(f"lowrank segments {segs}")
    b = _bundles(segs, K, 92)
    W, seg_end = gpu_quantize(A, b, K)
    c, sc, t, _ = oracle_quantize(b)
    N = sum(segs)
    s = inputs.uniform_bf16((N,), 0.9, 1.1, 9, 92, 9, inputs.T_S)
    U = inputs.normal_bf16((N, r), 0.02, 9, 92, 9, inputs.T_U)
    V = np.stack([inputs.normal_bf16((K, r), 0.02, 9, 92, 10 + g, inputs.T_V) for g in range(4)])
    x = inputs.activation_bf16(1, K, 9, 92, 0)
    y = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros((A.attnq_gemv_nvfp4_lowrank_workspace(K, 4, r),), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4_lowrank(W, dev(s), dev(U), dev(V), dev(x.reshape(-1)), ws, y)
    torch.cuda.synchronize()
    yref = O.gemv_nvfp4_lowrank(c, sc, t, s, U, V, x, seg_end)
    mag = O.abs_lowrank(s, U, V, x, O.abs_dot(c, sc, t, x, seg_end)[0], seg_end)
    err = np.abs(host(y).astype(np.float64) - yref)
    assert np.all(err <= 2.0 ** -14 * mag), f"max err/mag {np.max(err / mag)}"


def _extreme_x(K, seed):
    x = inputs.activation_bf16(1, K, 9, 93, seed).reshape(-1).copy()
    big, nbig, tiny = inputs.bits_from_floats([2.0 ** 100, -(2.0 ** 100), 2.0 ** -100])
    x[3] = big
    x[K // 2] = nbig
    x[5] = tiny
    x[7:39] = 0                                # a whole zero chunk
    x[K - 1] = 0x8000                          # -0
    return x


def test_gemv_extreme_activations(A):
    K = 5376
    segs = (300, 41)
    say("gemv extreme activations")
    b = _bundles(segs, K, 93)
    W, seg_end = gpu_quantize(A, b, K)
    c, s, t, _ = oracle_quantize(b)
    x = _extreme_x(K, 0)
    y = torch.full((W.N,), float("nan"), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, dev(x), y)
    torch.cuda.synchronize()
    yh = host(y)
    assert np.all(np.isfinite(yh))
    assert_close_products(yh, O.gemv_nvfp4(c, s, t, x, seg_end), O.abs_dot(c, s, t, x, seg_end)[0], "extreme x")


def test_glu_single_pair(A):
    K = 1152
    say("glu F = 1")
    b = _bundles((1, 1), K, 94)
    W, _ = gpu_quantize(A, b, K)
    c, s, t, _ = oracle_quantize(b)
    x = inputs.activation_bf16(1, K, 9, 94, 0)
    g, u = O.gemv_nvfp4_glu(c, s, t, x)
    ad_g = O.abs_dot(c, s, t, x, [1, 2], rows=np.array([0]))[0]
    ad_u = O.abs_dot(c, s, t, x, [1, 2], rows=np.array([1]))[0]
    for act in (A.ACT_GELU_TANH, A.ACT_SILU, A.ACT_IDENTITY):
        h = torch.full((1,), 0x7FFF, dtype=torch.int16, device="cuda")
        A.attnq_gemv_nvfp4_glu(W, dev(x.reshape(-1)), act, h)
        torch.cuda.synchronize()
        href = O.bf16_to_f32(O.glu(g, u, act)).astype(np.float64)
        hg = O.bf16_to_f32(host(h).view(np.uint16)).astype(np.float64)
        a = O.activation(g, act)
        bound = 2.0 ** -8 * np.abs(href) + 2.0 ** -14 * (ad_g * np.abs(u) + ad_u * np.abs(a)) + 1e-30
        assert np.all(np.abs(hg - href) <= bound), (act, hg, href, bound)


def _check_nonfinite(got, want, what):
    """Non-finite outputs must sit where the oracle's are, with the same kind and sign."""
    got = got.astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{what}: NaN pattern differs"
    inf_w = np.isinf(want)
    assert np.array_equal(np.isinf(got), inf_w), f"{what}: inf pattern differs"
    assert np.array_equal(np.sign(got[inf_w]), np.sign(want[inf_w])), f"{what}: inf sign differs"


@pytest.mark.filterwarnings("ignore:invalid value encountered")   # the oracle's inf * 0, by design
@pytest.mark.parametrize("M", [1, 4, 8])
def test_nonfinite_activations_propagate(A, M):
    """x holding +inf at one position gives, row by row, NaN where the dequantized weight at that
    position is zero (inf * 0) and +-inf elsewhere, exactly as the float64 oracle; a NaN anywhere
    in x makes every output of that token NaN. Other tokens of a small-M product are unaffected."""
    K = 1152
    segs = (300, 41)
    what = f"non-finite x, M {M}"
    say(what)
    b = _bundles(segs, K, 95)
    W, seg_end = gpu_quantize(A, b, K)
    c, s, t, _ = oracle_quantize(b)
    X = inputs.activation_bf16(M, K, 9, 95, M).copy()
    pinf, nan = inputs.bits_from_floats([float("inf")])[0], 0x7FC0
    X[0, 5] = pinf
    if M > 1:
        X[1, K - 1] = nan
    if M == 1:
        y = torch.full((W.N,), 0.0, dtype=torch.float32, device="cuda")
        A.attnq_gemv_nvfp4(W, dev(X.reshape(-1)), y)
        torch.cuda.synchronize()
        got = host(y)[None]
        want = O.gemv_nvfp4(c, s, t, X, seg_end)[None]
    else:
        Y = torch.full((M, W.N), 0.0, dtype=torch.float32, device="cuda")
        A.attnq_gemm_nvfp4_small_m(W, dev(X), Y)
        torch.cuda.synchronize()
        got = host(Y)
        want = O.gemm_nvfp4_small_m(c, s, t, X, seg_end)
    assert np.isnan(want[0]).any() and np.isinf(want[0]).any(), "the case must hold both kinds"
    for m in range(M):
        _check_nonfinite(got[m], want[m], f"{what} token {m}")
    if M > 1:
        assert np.all(np.isnan(got[1]))
    # tokens without a non-finite input stay finite and within the GEMV bound
    if M > 2:
        ad = O.abs_dot(c, s, t, X, seg_end)
        for m in range(2, M):
            assert_close_products(got[m], want[m], ad[m], f"{what} finite token {m}")
