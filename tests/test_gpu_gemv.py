"""GPU parity of the decode products through the C ABI: attnq_gemv_nvfp4, attnq_gemv_bf16 and
attnq_gemm_nvfp4_small_m against the float64 oracle (relative L2 <= 1e-3 contract, plus the
per-element fp32 bound in gpu_helpers), and bit-exact one-hot columns."""
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


def _gemv_case(A, bundles, K, x_bits, what):
    say(what)
    W, seg_end = gpu_quantize(A, bundles, K)
    c, s, t, _ = oracle_quantize(bundles)
    assert np.array_equal(host(W.codes), c) and np.array_equal(host(W.scales), s)
    y = torch.full((W.N,), np.nan, dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, dev(x_bits.reshape(-1)), y)
    torch.cuda.synchronize()
    y_ref = O.gemv_nvfp4(c, s, t, x_bits, seg_end)
    absdot = O.abs_dot(c, s, t, x_bits, seg_end)[0]
    assert_close_products(host(y), y_ref, absdot, what)
    return W, c, s, t, seg_end


def test_gemv_single_projection(A):
    b = inputs.theta_bundle(1024, 1152, 0, cfg=0, layer=0, proj=0, passthrough=True)
    x = inputs.activation_bf16(1, 1152, 0, 0, 0)
    _gemv_case(A, [b], 1152, x, "gemv 1024x1152")


def test_gemv_small_decoder_layer(A):
    L = 3
    x = lambda K, p: inputs.activation_bf16(1, K, 1, L, p)
    qkv = [inputs.theta_bundle(n, 1152, 4, cfg=1, layer=L, proj=p) for p, n in enumerate((1024, 256, 256))]
    _gemv_case(A, qkv, 1152, x(1152, 0), "1B-like fused qkv gemv")
    _gemv_case(A, [inputs.theta_bundle(1152, 1024, 4, cfg=1, layer=L, proj=3)], 1024, x(1024, 3), "1B-like o gemv")
    gu = [inputs.theta_bundle(6912, 1152, 4, cfg=1, layer=L, proj=p) for p in (4, 5)]
    _gemv_case(A, gu, 1152, x(1152, 4), "1B-like gate|up gemv")
    _gemv_case(A, [inputs.theta_bundle(1152, 6912, 4, cfg=1, layer=L, proj=6)], 6912, x(6912, 6), "1B-like down gemv")


# shapes chosen to hit every launch configuration, ragged rows and ragged K slices
@pytest.mark.parametrize("N,K", [(1, 32), (3, 64), (17, 96), (1000, 1152), (8193, 2048), (4097, 2080), (8193, 4096),
                                 (100, 6144 + 32), (4099, 8192), (513, 8192 + 32), (77, 16384 + 32), (300, 21504)])
def test_gemv_ragged_shapes(A, N, K):
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=30, proj=N, passthrough=True)
    x = inputs.activation_bf16(1, K, 9, 30, N)
    _gemv_case(A, [b], K, x, f"gemv ragged {N}x{K}")


# long rows (K = 21504, the down projection's K split over a workgroup): one row, an odd row count
# (rows past N clamped) and a two-segment weight whose boundary falls inside a workgroup's rows
@pytest.mark.parametrize("segs", [(1,), (301,), (1501, 2596)])
def test_gemv_long_rows_segments(A, segs):
    K = 21504
    bs = [inputs.theta_bundle(n, K, 0, cfg=9, layer=34, proj=i, passthrough=True) for i, n in enumerate(segs)]
    x = inputs.activation_bf16(1, K, 9, 34, len(segs))
    _gemv_case(A, bs, K, x, f"gemv long rows {segs}x{K}")


# more long-row shapes for the K-split loop kernel: row counts near 1800 (a ragged last workgroup),
# K = 16384, 16416 (a ragged last step in each K half) and 24576, three- and two-segment weights
# whose boundaries fall inside a workgroup's rows
@pytest.mark.parametrize("segs,K", [((1792,), 16384), ((700, 3, 1097), 16416), ((1000, 799), 24576)])
def test_gemv_long_rows_more_shapes(A, segs, K):
    bs = [inputs.theta_bundle(n, K, 0, cfg=9, layer=35, proj=i, passthrough=True) for i, n in enumerate(segs)]
    x = inputs.activation_bf16(1, K, 9, 35, len(segs))
    _gemv_case(A, bs, K, x, f"gemv long rows {segs}x{K}")


def test_gemv_one_hot_columns_are_exact_long_rows(A):
    """One-hot x through the K-split loop kernel: the other K half's partial sum is zero, so the
    fp32 dequantized column comes back bit for bit."""
    N, K = 1800, 16416
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=36, proj=0, passthrough=True)
    say("one-hot gemv, long rows")
    W, _ = gpu_quantize(A, [b], K)
    c, s, t, _ = oracle_quantize([b])
    deq32 = O.dequantize_f32(c, s, t)
    y = torch.empty((N,), dtype=torch.float32, device="cuda")
    for k in (0, 31, 2048, 8209, K - 1):
        xb = np.zeros(K, np.uint16)
        xb[k] = 0x3F80
        A.attnq_gemv_nvfp4(W, dev(xb), y)
        torch.cuda.synchronize()
        assert np.array_equal(host(y), deq32[:, k]), k


def test_gemv_one_hot_columns_are_exact(A):
    N, K = 96, 2048
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=31, proj=0, passthrough=True)
    say("one-hot gemv")
    W, _ = gpu_quantize(A, [b], K)
    c, s, t, _ = oracle_quantize([b])
    deq32 = O.dequantize_f32(c, s, t)
    y = torch.empty((N,), dtype=torch.float32, device="cuda")
    for k in (0, 15, 16, 1023, 2047):
        xb = np.zeros(K, np.uint16)
        xb[k] = 0x3F80
        A.attnq_gemv_nvfp4(W, dev(xb), y)
        torch.cuda.synchronize()
        assert np.array_equal(host(y), deq32[:, k]), k


def test_gemv_zero_and_nan_segments(A):
    z = np.zeros((64, 256), np.uint16)
    bad = inputs.normal_bf16((64, 256), 0.02, 9, 32, 1, 0).copy()
    bad[10, 10] = 0x7FC0
    ok = inputs.normal_bf16((64, 256), 0.02, 9, 32, 2, 0)
    say("gemv zero/NaN/ok segments")
    W, _ = gpu_quantize(A, [(z, None, None, None), (bad, None, None, None), (ok, None, None, None)], 256)
    x = inputs.activation_bf16(1, 256, 9, 32, 0)
    y = torch.empty((192,), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, dev(x.reshape(-1)), y)
    torch.cuda.synchronize()
    yh = host(y)
    assert (yh[:64] == 0).all() and np.isnan(yh[64:128]).all() and np.isfinite(yh[128:]).all()


def test_gemv_empty_is_noop(A):
    say("empty gemv")
    W = A.NVFP4Weight.empty(0, 64, [0])
    A.attnq_gemv_nvfp4(W, dev(np.zeros(64, np.uint16)), torch.empty((0,), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()


# launch classes of the bf16 GEMV: one-shot with 8 steps (K <= 4096), 11 steps (K <= 5632), the loop
# kernel beyond; each boundary from both sides
@pytest.mark.parametrize("N,K", [(1, 32), (7, 64), (1000, 1152), (4096, 5376), (333, 21504),
                                 (301, 4096), (301, 4096 + 32), (301, 5632), (301, 5632 + 32)])
def test_gemv_bf16(A, N, K):
    W = inputs.normal_bf16((N, K), 0.02, 9, 33, N, 0)
    x = inputs.activation_bf16(1, K, 9, 33, N)
    say(f"bf16 gemv {N}x{K}")
    y = torch.full((N,), np.nan, dtype=torch.float32, device="cuda")
    A.attnq_gemv_bf16(dev(W), dev(x.reshape(-1)), y)
    torch.cuda.synchronize()
    assert_close_products(host(y), O.gemv_bf16(W, x), O.abs_dot_bf16(W, x), f"bf16 {N}x{K}")


@pytest.mark.parametrize("M", [0, 1, 2, 4, 5, 8, 16])
def test_small_m(A, M):
    K = 1152
    qkv = [inputs.theta_bundle(n, K, 4, cfg=4, layer=0, proj=p) for p, n in enumerate((1024, 256, 256))]
    say(f"small-M {M} fused 1536x1152")
    W, seg_end = gpu_quantize(A, qkv, K)
    c, s, t, _ = oracle_quantize(qkv)
    X = inputs.activation_bf16(max(M, 1), K, 4, 0, 9)[:M]
    ldx, ldy = K + 64, W.N + 40                   # padded leading dimensions
    Xd = torch.zeros((max(M, 1), ldx), dtype=torch.int16, device="cuda")
    if M:
        Xd[:M, :K] = dev(X)
    Yd = torch.full((max(M, 1), ldy), -7.0, dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m(W, Xd[:M] if M else Xd[:0], Yd[:M] if M else Yd[:0])
    torch.cuda.synchronize()
    Y = host(Yd)
    if M == 0:
        assert (Y == -7.0).all()
        return
    assert (Y[:, W.N:] == -7.0).all()                 # padding untouched
    Y_ref = O.gemm_nvfp4_small_m(c, s, t, X, seg_end)
    absdot = O.abs_dot(c, s, t, X, seg_end)
    assert_close_products(Y[:M, :W.N], Y_ref, absdot, f"small-M {M}")


# ragged K (K % 128 in {32, 64, 96} exercises the 32-element tail), ragged 16-row tiles, both
# launch configurations (N >= 16384 uses two row tiles per wave), every token-row count class, and
# M <= 4 on either side of the batch-1 walk's row limit (6144 elements)
@pytest.mark.parametrize("N,K,M", [(1, 32, 1), (17, 96, 3), (333, 1184, 16), (1000, 1248, 5), (4097, 2080, 8),
                                   (16385, 224, 4), (16400, 1152 + 64, 13), (600, 21504 + 32, 2),
                                   (301, 6144, 3), (301, 6144 + 32, 4)])
def test_small_m_ragged(A, N, K, M):
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=31, proj=N % 97, passthrough=True)
    say(f"small-M ragged {M}x{N}x{K}")
    W, seg_end = gpu_quantize(A, [b], K)
    c, s, t, _ = oracle_quantize([b])
    X = inputs.activation_bf16(M, K, 9, 31, N % 89)
    Y = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m(W, dev(X), Y)
    torch.cuda.synchronize()
    assert_close_products(host(Y), O.gemm_nvfp4_small_m(c, s, t, X, seg_end), O.abs_dot(c, s, t, X, seg_end),
                          f"small-M ragged {M}x{N}x{K}")


# rows of at most 192 chunks: M <= 4 runs on the batch-1 walk, and each token's row is the batch-1
# GEMV of that token bit for bit (same launch shape, same per-block arithmetic and wave sums); the
# shapes straddle its class boundaries (two steps up to K = 4096, three up to 6144, one row per wave
# below N = 16384 and two from there)
@pytest.mark.parametrize("N,K", [(4097, 2080), (5376, 4096), (6144, 5376), (16400, 5376), (300, 96),
                                 (301, 4096 + 32), (16383, 6144), (16384, 4096 + 32)])
def test_small_m_tokens_equal_the_gemv_bitwise(A, N, K):
    say(f"small-M vs GEMV bitwise {N}x{K}")
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=37, proj=0, passthrough=True)
    W, _ = gpu_quantize(A, [b], K)
    X = inputs.activation_bf16(4, K, 9, 37, 1)
    y = torch.empty((N,), dtype=torch.float32, device="cuda")
    for M in (1, 2, 3, 4):
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        A.attnq_gemm_nvfp4_small_m(W, dev(X[:M]), Y)
        torch.cuda.synchronize()
        for m in range(M):
            A.attnq_gemv_nvfp4(W, dev(X[m]), y)
            torch.cuda.synchronize()
            assert np.array_equal(host(Y)[m].view(np.uint32), host(y).view(np.uint32)), (M, m)


@pytest.mark.parametrize("M_small,M_big", [(1, 4), (2, 3), (5, 16), (8, 13)])
def test_small_m_rows_are_independent_of_padding(A, M_small, M_big):
    """Token rows m < M must not depend on how many rows follow or what they hold: within one
    launch class (M <= 4, and 4 < M <= 16, which share a kernel and its summation order), the
    first M_small rows of the M_big product equal the M_small product bit for bit, also after
    the rows past M_small are overwritten."""
    N, K = 2048, 1152
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=32, proj=0, passthrough=True)
    W, _ = gpu_quantize(A, [b], K)
    X = dev(inputs.activation_bf16(16, K, 9, 32, 1))
    Xb = X.clone()
    Xb[M_small:] = dev(inputs.activation_bf16(16, K, 9, 32, 2))[M_small:]
    Yb = torch.empty((M_big, N), dtype=torch.float32, device="cuda")
    Yb2 = torch.empty((M_big, N), dtype=torch.float32, device="cuda")
    Ys = torch.empty((M_small, N), dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m(W, X[:M_big], Yb)
    A.attnq_gemm_nvfp4_small_m(W, Xb[:M_big], Yb2)
    A.attnq_gemm_nvfp4_small_m(W, X[:M_small], Ys)
    torch.cuda.synchronize()
    s_bits = host(Ys).view(np.uint32)
    assert np.array_equal(s_bits, host(Yb)[:M_small].view(np.uint32))
    assert np.array_equal(s_bits, host(Yb2)[:M_small].view(np.uint32))
