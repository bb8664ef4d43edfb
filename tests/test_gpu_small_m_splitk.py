"""GPU parity of attnq_gemm_nvfp4_small_m_splitk, the small-M product with K cut into one-shot slices
on separate workgroups ("Throughput", "Speculative decoding": verification at gamma + 1 = 4 tokens and
batches of 8), against the float64 oracle with the fp32 bounds of gpu_helpers: every token class
(M <= 4 on long rows, 4 < M <= 8 with one- and two-step slices, M <= 16), ragged K (partial steps
and chunks), ragged row groups, multi-segment weights, bit-identical repeats (the workspace holding
another call's partials in between), a workspace shared by several shapes, exact one-hot columns,
and shapes on the batch-1 walk equal to attnq_gemm_nvfp4_small_m. Weights of at least 16384 rows
whose rows split into whole strips take the walking strips, with X staged in fp16 when every
token's window lies within fp16's normal range after a power-of-two scale, and in bf16 otherwise:
both operand paths are checked, the fallback forced by X values far apart, subnormal or huge."""
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


def _case(A, segs, K, M, layer, what):
    bs = [inputs.theta_bundle(n, K, 0, cfg=9, layer=layer, proj=i, passthrough=True) for i, n in enumerate(segs)]
    X = inputs.activation_bf16(M, K, 9, layer, 7)
    say(what)
    W, seg_end = gpu_quantize(A, bs, K)
    c, s, t, _ = oracle_quantize(bs)
    ws = A.small_m_workspace(W.N, K, M)
    Y = torch.full((M, W.N), np.nan, dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m_splitk(W, dev(X), Y, ws)
    torch.cuda.synchronize()
    Yh = host(Y)
    Yr = O.gemm_nvfp4_small_m(c, s, t, X, seg_end)
    ad = O.abs_dot(c, s, t, X, seg_end)
    for m in range(M):
        assert_close_products(Yh[m], Yr[m], ad[m], f"{what}: token {m}")
    return W, X, ws, Yh


# (segments, K, M): long rows at M <= 4 (21 one-step slices, ragged last step), M = 5..8 with one-step
# slices and with two-step slices (>= 16384 rows), M = 9..16, K with a partial last step, K a
# multiple of 1024, row counts of one row, a ragged row group and several groups, segment
# boundaries inside a group; narrower weights with long rows at 4 < M <= 8 that split into whole
# strips (the walk: 21 strips of 32 chunks, 8 of 32, 17 of 24)
@pytest.mark.parametrize("segs,K,M", [((300,), 21504, 1), ((129,), 21504 + 32, 4), ((1, 2), 16384, 3),
                                      ((1,), 6144 + 32, 8), ((77,), 8192 + 96, 5), ((1000, 24), 16384 + 32, 8),
                                      ((16384, 16), 1152 + 96, 6), ((8200, 8200), 2048, 8),
                                      ((16400,), 4096 + 32, 7), ((333,), 21504, 16), ((700, 3, 1097), 7168, 13),
                                      ((64,), 21504, 9), ((5, 6, 7, 8), 12288, 11), ((16383, 2), 3072, 16),
                                      ((300, 77), 21504, 6), ((5,), 8192, 5), ((64,), 12288 + 256 * 3, 7)])
def test_small_m_splitk_against_oracle(A, segs, K, M):
    _case(A, segs, K, M, 70, f"small-M split-K {segs}x{K} M {M}")


def test_small_m_splitk_repeats_are_bit_identical(A):
    W, X, ws, first = _case(A, (900,), 21504, 8, 71, "small-M split-K repeat 900x21504 M 8")
    Xd = dev(X)
    Y = torch.empty((8, 900), dtype=torch.float32, device="cuda")
    for r in range(5):
        Y.fill_(float("nan"))
        ws.fill_(0xFF)                       # whatever the workspace holds on entry
        A.attnq_gemm_nvfp4_small_m_splitk(W, Xd, Y, ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(Y).view(np.uint32), first.view(np.uint32)), r


def test_small_m_splitk_one_workspace_for_several_shapes(A):
    shapes = [((2000,), 21504, 8), ((16400,), 5376, 8), ((100,), 4096, 16), ((64,), 16384, 2)]
    need = max(A.attnq_gemm_nvfp4_small_m_splitk_workspace(sum(sg), K, M) for sg, K, M in shapes)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    cases = []
    for j, (segs, K, M) in enumerate(shapes):
        bs = [inputs.theta_bundle(n, K, 0, cfg=9, layer=72, proj=10 * j + i, passthrough=True) for i, n in enumerate(segs)]
        say(f"small-M split-K shared workspace {segs}x{K} M {M}")
        W, seg_end = gpu_quantize(A, bs, K)
        X = inputs.activation_bf16(M, K, 9, 72, j)
        cases.append((W, seg_end, bs, X, torch.empty((M, W.N), dtype=torch.float32, device="cuda")))
    for _ in range(2):
        for W, _, _, X, Y in cases:
            Y.fill_(float("nan"))
            A.attnq_gemm_nvfp4_small_m_splitk(W, dev(X), Y, ws)
    torch.cuda.synchronize()
    for W, seg_end, bs, X, Y in cases:
        c, s, t, _ = oracle_quantize(bs)
        Yh, Yr, ad = host(Y), O.gemm_nvfp4_small_m(c, s, t, X, seg_end), O.abs_dot(c, s, t, X, seg_end)
        for m in range(X.shape[0]):
            assert_close_products(Yh[m], Yr[m], ad[m], f"shared workspace N {W.N} token {m}")


def test_small_m_splitk_one_hot_columns_are_exact(A):
    """X rows one-hot at different columns: each token's row of Y is a dequantized column, bit for bit."""
    N, K, M = 300, 21504, 8
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=73, proj=0, passthrough=True)
    say("small-M split-K one-hot")
    W, _ = gpu_quantize(A, [b], K)
    c, s, t, _ = oracle_quantize([b])
    deq32 = O.dequantize_f32(c, s, t)
    cols = [0, 31, 1023, 1024, 5000, 12345, 20480, K - 1]
    X = np.zeros((M, K), np.uint16)
    for m, k in enumerate(cols):
        X[m, k] = 0x3F80
    ws = A.small_m_workspace(N, K, M)
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m_splitk(W, dev(X), Y, ws)
    torch.cuda.synchronize()
    for m, k in enumerate(cols):
        assert np.array_equal(host(Y)[m], deq32[:, k]), k


def test_small_m_splitk_zero_and_nan_segments(A):
    K, M = 4096, 8
    z = np.zeros((70, K), np.uint16)
    bad = inputs.normal_bf16((70, K), 0.02, 9, 74, 1, 0).copy()
    bad[3, 3000] = 0x7FC0
    ok = inputs.normal_bf16((70, K), 0.02, 9, 74, 2, 0)
    say("small-M split-K zero/NaN/ok segments")
    W, _ = gpu_quantize(A, [(z, None, None, None), (bad, None, None, None), (ok, None, None, None)], K)
    X = inputs.activation_bf16(M, K, 9, 74, 0)
    ws = A.small_m_workspace(W.N, K, M)
    Y = torch.empty((M, 210), dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m_splitk(W, dev(X), Y, ws)
    torch.cuda.synchronize()
    Yh = host(Y)
    assert (Yh[:, :70] == 0).all() and np.isnan(Yh[:, 70:140]).all() and np.isfinite(Yh[:, 140:]).all()


def test_small_m_splitk_single_slice_needs_no_workspace(A):
    """K of one step: a single slice stores Y directly, with no workspace."""
    assert A.attnq_gemm_nvfp4_small_m_splitk_workspace(16390, 1024, 8) == 0
    _case(A, (16390,), 1024, 8, 76, "small-M split-K single slice 16390x1024 M 8")


@pytest.mark.parametrize("N,K,M", [(6144, 5376, 4), (301, 4096 + 32, 2), (16400, 5376, 1), (6144, 5376, 8),
                                   (5376, 4096, 16)])
def test_small_m_splitk_walk_shapes_equal_the_plain_call(A, N, K, M):
    """Shapes without slices (rows of up to 6144 elements at M <= 4, or fewer than 16384 rows) run the
    plain call's kernels: bitwise the same Y."""
    assert A.attnq_gemm_nvfp4_small_m_splitk_workspace(N, K, M) == 0
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=75, proj=0, passthrough=True)
    X = dev(inputs.activation_bf16(M, K, 9, 75, 0))
    say(f"small-M split-K unsliced {N}x{K} M {M}")
    W, _ = gpu_quantize(A, [b], K)
    Y1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Y2 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m(W, X, Y1)
    A.attnq_gemm_nvfp4_small_m_splitk(W, X, Y2, None)
    torch.cuda.synchronize()
    assert np.array_equal(host(Y1).view(np.uint32), host(Y2).view(np.uint32))


def _walk_case(A, X, K, what, layer, n=16400):
    b = inputs.theta_bundle(n, K, 0, cfg=9, layer=layer, proj=0, passthrough=True)
    M = X.shape[0]
    say(what)
    W, seg_end = gpu_quantize(A, [b], K)
    c, s, t, _ = oracle_quantize([b])
    ws = A.small_m_workspace(W.N, K, M)
    assert ws is not None and ws.numel() > 0                 # the walking strips with partial sums
    Y = torch.full((M, W.N), np.nan, dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m_splitk(W, dev(X), Y, ws)
    torch.cuda.synchronize()
    Yh, Yr, ad = host(Y), O.gemm_nvfp4_small_m(c, s, t, X, seg_end), O.abs_dot(c, s, t, X, seg_end)
    for m in range(M):
        assert_close_products(Yh[m], Yr[m], ad[m], f"{what}: token {m}")
    return W, c, s, t


def _x_with(M, K, layer, edits):
    X = inputs.activation_bf16(M, K, 9, layer, 3).copy()
    for (m, k, v) in edits:
        X[m, k] = v
    return X


# X windows for the two operand paths of the walk (16400 x 5376: 7 strips of 24 chunks):
# - plain activations (fp16 operands);
# - a token with one value 2^40 below its largest (the window falls back to bf16 operands);
# - one value of 2^100 in a token (fallback; that token's sums are huge, the others' are not);
# - a bf16 subnormal (fallback);
# - an all-zero token next to ordinary ones (fp16, that token's factor is 1).
@pytest.mark.parametrize("M", [3, 4, 8, 13])
def test_small_m_walk_operand_paths(A, M):
    K = 5376
    cases = [("plain", []), ("2^-40 value", [(M - 1, 700, 0x2B80)]), ("2^100 value", [(0, 4000, 0x71C0)]),
             ("bf16 subnormal", [(M // 2, 10, 0x0003)])]
    for j, (name, edits) in enumerate(cases):
        _walk_case(A, _x_with(M, K, 77 + j, edits), K, f"small-M walk {name} M {M}", 77)
    Z = inputs.activation_bf16(M, K, 9, 81, 3).copy()
    Z[M - 1, :] = 0
    _walk_case(A, Z, K, f"small-M walk zero token M {M}", 77)


def test_small_m_walk_narrow_long_rows_operand_paths(A):
    """A narrower weight with long rows (377 x 21504 at M = 6: 21 strips of 32 chunks, 6 row groups, the
    last one ragged) on both operand paths."""
    M, K = 6, 21504
    for j, (name, edits) in enumerate([("plain", []), ("2^-40 value", [(2, 20000, 0x2B80)])]):
        _walk_case(A, _x_with(M, K, 83 + j, edits), K, f"small-M walk narrow {name} M {M}", 83, n=377)


def test_small_m_walk_one_hot_columns_are_exact(A):
    """On the walking strips (fp16 operands with per-token power-of-two factors) one-hot X rows still
    return the dequantized columns bit for bit."""
    N, K, M = 16400, 5376, 8
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=82, proj=0, passthrough=True)
    say("small-M walk one-hot")
    W, _ = gpu_quantize(A, [b], K)
    c, s, t, _ = oracle_quantize([b])
    cols = [0, 31, 767, 768, 2000, 4095, 5000, K - 1]
    X = np.zeros((M, K), np.uint16)
    for m, k in enumerate(cols):
        X[m, k] = 0x3F80 if m % 2 == 0 else 0x4C00          # 1.0, and 2^25 (a factor of 2^-10)
    ws = A.small_m_workspace(N, K, M)
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m_splitk(W, dev(X), Y, ws)
    torch.cuda.synchronize()
    deq32 = O.dequantize_f32(c, s, t)
    for m, k in enumerate(cols):
        scale = np.float32(1.0 if m % 2 == 0 else 2.0 ** 25)
        assert np.array_equal(host(Y)[m], deq32[:, k] * scale), k
