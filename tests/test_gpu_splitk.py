"""GPU parity of attnq_gemv_nvfp4_splitk, the NVFP4 GEMV with K split across workgroups for long
rows ("Throughput", "The NVFP4 MLP kernels are the least bandwidth-efficient on the step": the down
projection's launch was short of parallelism). Against the float64 oracle with the fp32 bounds of
gpu_helpers; repeated calls bit-identical; the ticket area of the workspace zero again after every
call; one-hot columns bit-exact; shorter rows identical to attnq_gemv_nvfp4."""
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


RECORD = 832          # bytes per 16-row tile: a 64-byte ticket slot and twelve 64-byte partial slots


def _tickets_zero(A, ws, N):
    tiles = (N + 15) // 16
    t = ws[:RECORD * tiles].view(tiles, RECORD)[:, :4]
    return int(torch.count_nonzero(t).item()) == 0


def _splitk_case(A, segs, K, what, layer=40):
    bs = [inputs.theta_bundle(n, K, 0, cfg=9, layer=layer, proj=i, passthrough=True) for i, n in enumerate(segs)]
    x = inputs.activation_bf16(1, K, 9, layer, len(segs))
    say(what)
    W, seg_end = gpu_quantize(A, bs, K)
    c, s, t, _ = oracle_quantize(bs)
    assert np.array_equal(host(W.codes), c) and np.array_equal(host(W.scales), s)
    ws = A.splitk_workspace(W.N, K)
    y = torch.full((W.N,), np.nan, dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4_splitk(W, dev(x.reshape(-1)), y, ws)
    torch.cuda.synchronize()
    assert_close_products(host(y), O.gemv_nvfp4(c, s, t, x, seg_end), O.abs_dot(c, s, t, x, seg_end)[0], what)
    if ws is not None:
        assert _tickets_zero(A, ws, W.N), "tickets left non-zero"
    return W, x, ws, y


# K = 16384 (4 slices of 128 chunks), 16416 (5 slices, ragged last slice), 21504 (6 x 112, the down
# projection), 24576 (6 x 128), 49152 (12 x 128), 21600 (6 slices, ragged); row counts of one row,
# a ragged last tile, several tiles; segment boundaries inside a tile
@pytest.mark.parametrize("segs,K", [((1,), 16384), ((17,), 16384 + 32), ((300,), 21504), ((1792,), 16384),
                                    ((700, 3, 1097), 16416), ((1000, 799), 24576), ((333,), 49152),
                                    ((1501, 2596), 21504), ((5, 6, 7, 8), 21504 + 96)])
def test_splitk_against_oracle(A, segs, K):
    _splitk_case(A, segs, K, f"splitk {segs}x{K}")


def test_splitk_repeated_calls_are_bit_identical(A):
    W, x, ws, y = _splitk_case(A, (1201,), 21504, "splitk repeat 1201x21504")
    first = host(y).view(np.uint32).copy()
    xd = dev(x.reshape(-1))
    for i in range(6):
        y.fill_(float("nan"))
        A.attnq_gemv_nvfp4_splitk(W, xd, y, ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(y).view(np.uint32), first), i
    assert _tickets_zero(A, ws, W.N)


def test_splitk_one_workspace_for_several_weights(A):
    """Weights of different shapes take turns on one workspace sized for the largest, in stream order."""
    K = 21504
    big = [inputs.theta_bundle(2000, K, 0, cfg=9, layer=41, proj=0, passthrough=True)]
    small = [inputs.theta_bundle(37, 16384, 0, cfg=9, layer=41, proj=1, passthrough=True)]
    say("splitk shared workspace")
    Wb, _ = gpu_quantize(A, big, K)
    Ws, _ = gpu_quantize(A, small, 16384)
    ws = A.splitk_workspace(2000, K)
    assert ws.numel() >= A.attnq_gemv_nvfp4_splitk_workspace(37, 16384)
    xb = inputs.activation_bf16(1, K, 9, 41, 0)
    xs = inputs.activation_bf16(1, 16384, 9, 41, 1)
    yb = torch.empty(2000, dtype=torch.float32, device="cuda")
    ys = torch.empty(37, dtype=torch.float32, device="cuda")
    for _ in range(3):                   # y is refilled with NaN, so every call must store every row
        yb.fill_(float("nan"))
        ys.fill_(float("nan"))
        A.attnq_gemv_nvfp4_splitk(Wb, dev(xb.reshape(-1)), yb, ws)
        A.attnq_gemv_nvfp4_splitk(Ws, dev(xs.reshape(-1)), ys, ws)
    torch.cuda.synchronize()
    for W, b, x, y in ((Wb, big, xb, yb), (Ws, small, xs, ys)):
        c, s, t, seg_end = oracle_quantize(b)
        assert_close_products(host(y), O.gemv_nvfp4(c, s, t, x, seg_end), O.abs_dot(c, s, t, x, seg_end)[0],
                              "shared workspace")
    assert _tickets_zero(A, ws, 2000)


def test_splitk_one_hot_columns_are_exact(A):
    """One-hot x: every slice but one contributes +0, so y is the fp32 dequantized column."""
    N, K = 700, 21504
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=42, proj=0, passthrough=True)
    say("splitk one-hot")
    W, _ = gpu_quantize(A, [b], K)
    c, s, t, _ = oracle_quantize([b])
    deq32 = O.dequantize_f32(c, s, t)
    ws = A.splitk_workspace(N, K)
    y = torch.empty((N,), dtype=torch.float32, device="cuda")
    for k in (0, 31, 3583, 3584, 10751, 17920, K - 1):      # slices start at multiples of 3584
        xb = np.zeros(K, np.uint16)
        xb[k] = 0x3F80
        A.attnq_gemv_nvfp4_splitk(W, dev(xb), y, ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(y), deq32[:, k]), k


def test_splitk_zero_and_nan_segments(A):
    K = 16384
    z = np.zeros((40, K), np.uint16)
    bad = inputs.normal_bf16((40, K), 0.02, 9, 43, 1, 0).copy()
    bad[3, 5000] = 0x7FC0
    ok = inputs.normal_bf16((40, K), 0.02, 9, 43, 2, 0)
    say("splitk zero/NaN/ok segments")
    W, _ = gpu_quantize(A, [(z, None, None, None), (bad, None, None, None), (ok, None, None, None)], K)
    x = inputs.activation_bf16(1, K, 9, 43, 0)
    ws = A.splitk_workspace(W.N, K)
    y = torch.empty((120,), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4_splitk(W, dev(x.reshape(-1)), y, ws)
    torch.cuda.synchronize()
    yh = host(y)
    assert (yh[:40] == 0).all() and np.isnan(yh[40:80]).all() and np.isfinite(yh[80:]).all()
    assert _tickets_zero(A, ws, W.N)


@pytest.mark.parametrize("N,K", [(5376, 4096), (6144, 5376), (300, 16384 - 32), (64, 49152 + 32)])
def test_splitk_unsplit_shapes_equal_the_gemv(A, N, K):
    """Shapes that are not split run attnq_gemv_nvfp4's kernels: bitwise the same y, no workspace."""
    assert A.attnq_gemv_nvfp4_splitk_workspace(N, K) == 0
    b = inputs.theta_bundle(N, K, 0, cfg=9, layer=44, proj=0, passthrough=True)
    x = dev(inputs.activation_bf16(1, K, 9, 44, 0).reshape(-1))
    say(f"splitk unsplit {N}x{K}")
    W, _ = gpu_quantize(A, [b], K)
    y1 = torch.empty((N,), dtype=torch.float32, device="cuda")
    y2 = torch.empty((N,), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, x, y1)
    A.attnq_gemv_nvfp4_splitk(W, x, y2, None)
    torch.cuda.synchronize()
    assert np.array_equal(host(y1).view(np.uint32), host(y2).view(np.uint32))


def test_splitk_empty_is_noop(A):
    say("splitk empty")
    W = A.NVFP4Weight.empty(0, 21504, [0])
    A.attnq_gemv_nvfp4_splitk(W, dev(np.zeros(21504, np.uint16)), torch.empty((0,), dtype=torch.float32, device="cuda"),
                              None)
    torch.cuda.synchronize()
