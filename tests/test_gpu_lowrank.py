"""GPU parity of the runtime low-rank product over a shared NVFP4 block
(attnq_gemv_nvfp4_lowrank): y = s * (x . deq(W0)^T) + U (V^T x), the weight never rebuilt.

* r = 0 without s equals attnq_gemv_nvfp4 element for element, and r = 0 with s equals
  fl32(y_gemv * s), in every launch class of the GEMV table (wiring of the epilogue);
* r = 1 .. 64 against the float64 oracle: every element within the GEMV's fp32 bound on the
  s-scaled W0 term plus a worst-case fp32 bound on the low-rank term (the longest chain of
  roundings through the chunk partials, their reduction and the wave sum), and relative L2
  <= 1e-3 (the contract) and <= 1e-5 (internal gate). U and V are drawn with sigma 0.02 so the
  low-rank term is a few percent of y and a dropped or mis-scaled term cannot hide in the bound;
* one quantized W0 serves several projections in turn (shared-block reading), a two-segment W0,
  N = 0, ragged K and N, and 31B-like shapes on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import dev, gpu_quantize, host, oracle_quantize, say
from nvfp4_weight_only_rtn_amd import inputs

pytestmark = pytest.mark.gpu

UV_SIGMA = 0.02
GEMV_BOUND = 2.0 ** -16


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def _shared(A, N, K, layer, seg_end=None):
    """One shared W0, quantized on the GPU (possibly as several segments of one weight)."""
    W0, _, _, _ = inputs.theta_bundle(N, K, 0, cfg=9, layer=layer, proj=0, passthrough=True)
    seg_end = [N] if seg_end is None else seg_end
    parts, start = [], 0
    for end in seg_end:
        parts.append((W0[start:end], None, None, None))
        start = end
    W, _ = gpu_quantize(A, parts, K)
    return W, parts


def _factors(N, K, r, layer, proj):
    """s ~ U(0.9, 1.1), U, V ~ N(0, 0.02^2) for one projection over the shared block."""
    s = inputs.uniform_bf16((N,), 0.9, 1.1, 9, layer, proj, inputs.T_S)
    if r == 0:
        return s, None, None
    U = inputs.normal_bf16((N, r), UV_SIGMA, 9, layer, proj, inputs.T_U)
    V = inputs.normal_bf16((K, r), UV_SIGMA, 9, layer, proj, inputs.T_V)
    return s, U, V


def _segment_factors(seg_end, K, r, layer):
    """Per-segment factors of a fused weight: s and U follow the fused rows, V is [n_seg, K, r]."""
    s, U, V, start = [], [], [], 0
    for g, end in enumerate(seg_end):
        sg, Ug, Vg = _factors(end - start, K, r, layer, 1 + g)
        s.append(sg); U.append(Ug); V.append(Vg)
        start = end
    return np.concatenate(s), np.concatenate(U), np.stack(V)


def _parts(K, r):
    """Partial sums per segment in the workspace: one per floor(16384 / r) rows of V."""
    kc = 16384 // r
    return -(-K // kc)


def _depth(K, r):
    """fp32 roundings along the longest path of the low-rank term: the chunk sums (8 fused
    multiply-adds, or up to floor(16384 / r) / (256 // r) + 1 of them), the 8 + 256 // r slot adds,
    a lane's ceil(P r / 64) <= P fused multiply-adds in the GEMV, the wave sum and the final
    products."""
    return 96 + 2 * (256 // r) + _parts(K, r) + 9


def _run(A, W, s, U, V, x):
    r = 0 if U is None else U.shape[1]
    y = torch.full((W.N,), float("nan"), dtype=torch.float32, device="cuda")
    ws = None
    if r:
        n = A.attnq_gemv_nvfp4_lowrank_workspace(W.K, len(W.seg_end), r)
        assert n == len(W.seg_end) * _parts(W.K, r) * r
        ws = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4_lowrank(W, dev(s), dev(U), dev(V), dev(x.reshape(-1)), ws, y)
    torch.cuda.synchronize()
    if not r:
        return host(y), None
    t = host(ws).reshape(len(W.seg_end), _parts(W.K, r), r).astype(np.float64).sum(axis=1)   # [n_seg, r]
    return host(y), t


def _plain(A, W, x):
    y = torch.empty((W.N,), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, dev(x.reshape(-1)), y)
    torch.cuda.synchronize()
    return host(y)


def _check(y, parts, s, U, V, x, K, rows, what):
    c, sc, ts, _ = oracle_quantize(parts, rows=rows)
    local = _local_segments(parts, rows)
    r = 0 if U is None else U.shape[1]
    sr = None if s is None else s[rows]
    Ur = None if U is None else U[rows]
    yref = O.gemv_nvfp4_lowrank(c, sc, ts, sr, Ur, V, x, seg_end=local)
    ad = O.abs_dot(c, sc, ts, x, local)[0]
    w0 = O.abs_lowrank(sr, None, None, x, ad)
    lrm = O.abs_lowrank(None, Ur, V, x, np.zeros_like(ad), local) if r else np.zeros_like(ad)
    depth = _depth(K, r) if r else 0
    bound = GEMV_BOUND * w0 + depth * 2.0 ** -24 * lrm + 1e-30
    yg = y[rows].astype(np.float64)
    err = np.abs(yg - yref)
    bad = np.argwhere(~(err <= bound))
    assert len(bad) == 0, f"{what}: {len(bad)} elements out of bound, first {bad[:5].ravel().tolist()} " \
                          f"err {err[bad[:1].ravel()]} bound {bound[bad[:1].ravel()]}"
    rel = np.linalg.norm(yg - yref) / np.linalg.norm(yref)
    assert rel <= 1e-3, f"{what}: rel-L2 {rel} over the contract"
    assert rel <= 1e-5, f"{what}: rel-L2 {rel} over the internal gate"
    if r:
        delta = yref - O.gemv_nvfp4_lowrank(c, sc, ts, sr, None, None, x, seg_end=local)
        assert np.linalg.norm(delta) > 4 * np.linalg.norm(bound), f"{what}: low-rank term not visible"


def _local_segments(parts, rows):
    """oracle_quantize returns only the selected rows; their segment table in that order."""
    bounds, n = [], 0
    for p in parts:
        n += p[0].shape[0]
        bounds.append(n)
    rows = np.asarray(rows)
    assert np.all(np.diff(rows) > 0), "sampled rows must be increasing"
    return [int(np.sum(rows < b)) for b in bounds if np.sum(rows < b) > 0]


# one shape per class of the GEMV launch table (K <= 4096; q|k|v-like; gate|up-like; long rows)
CLASSES = [(17, 96), (1000, 2080), (6144, 5376), (16400, 5376), (500, 8192), (77, 16416)]


@pytest.mark.parametrize("N,K", CLASSES)
def test_rank_zero_matches_the_gemv(A, N, K):
    say(f"lowrank r=0 {N}x{K}")
    W, _ = _shared(A, N, K, 70)
    x = inputs.activation_bf16(1, K, 9, 70, N)
    y0 = _plain(A, W, x)
    y, _ = _run(A, W, None, None, None, x)
    assert np.array_equal(y, y0)
    s, _, _ = _factors(N, K, 0, 70, 1)
    ys, _ = _run(A, W, s, None, None, x)
    want = (y0 * O.bf16_to_f32(s)).astype(np.float32)
    assert np.array_equal(ys, want)


@pytest.mark.parametrize("N,K,r", [(17, 96, 4), (1000, 2080, 16), (6144, 5376, 64), (16400, 5376, 8),
                                   (500, 8192, 1), (77, 16416, 3), (300, 21504, 32), (1, 32, 64),
                                   (129, 4128, 63)])
def test_lowrank_vs_oracle(A, N, K, r):
    what = f"lowrank {N}x{K} rank {r}"
    say(what)
    W, parts = _shared(A, N, K, 71)
    s, U, V = _factors(N, K, r, 71, 1)
    x = inputs.activation_bf16(1, K, 9, 71, r)
    y, t = _run(A, W, s, U, V, x)
    rows = None if N * K <= (1 << 24) else np.unique(np.concatenate([
        np.arange(4), np.arange(N - 4, N), np.random.default_rng(N + K).choice(N, 500, replace=False)]))
    _check(y, parts, s, U, V, x, K, np.arange(N) if rows is None else rows, what)
    # the workspace's partial sums add up to V^T x within their own fp32 bound
    xv = O.bf16_to_f32(x).astype(np.float64).reshape(-1)
    Vf = O.bf16_to_f32(V).astype(np.float64)
    tb = _depth(K, r) * 2.0 ** -24 * (np.abs(Vf).T @ np.abs(xv))
    assert np.all(np.abs(t[0] - Vf.T @ xv) <= tb), what


def test_shared_block_serves_several_projections(A):
    N, K = 2048, 3072
    say(f"lowrank shared block {N}x{K}")
    W, parts = _shared(A, N, K, 72)
    codes0, scales0 = W.codes.clone(), W.scales.clone()
    x = inputs.activation_bf16(1, K, 9, 72, 0)
    for proj, r in [(1, 8), (2, 0), (3, 32), (4, 64)]:
        s, U, V = _factors(N, K, r, 72, proj)
        y, _ = _run(A, W, s, U, V, x)
        _check(y, parts, s, U, V, x, K, np.arange(N), f"shared block proj {proj} rank {r}")
    assert torch.equal(W.codes, codes0) and torch.equal(W.scales, scales0)


def test_repeated_calls_are_bitwise_identical(A):
    N, K, r = 4096, 5376, 64
    say(f"lowrank determinism {N}x{K} rank {r}")
    W, _ = _shared(A, N, K, 73)
    s, U, V = _factors(N, K, r, 73, 1)
    x = inputs.activation_bf16(1, K, 9, 73, 1)
    y1, t1 = _run(A, W, s, U, V, x)
    y2, t2 = _run(A, W, s, U, V, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(t1, t2)


@pytest.mark.parametrize("N,K,r", [(1000, 2080, 16), (6144, 5376, 16), (16400, 5376, 8), (500, 8192, 32),
                                   (300, 21504, 16), (77, 16416, 3)])
def test_one_workspace_across_calls_with_new_inputs(A, N, K, r):
    """Calls that reuse one workspace with a different x each time must each equal a call on a
    fresh workspace, bit for bit: no partial sum of an earlier call may be read from any cache."""
    what = f"lowrank reused workspace {N}x{K} rank {r}"
    say(what)
    W, _ = _shared(A, N, K, 78)
    s, U, V = _factors(N, K, r, 78, 1)
    ws = torch.zeros((A.attnq_gemv_nvfp4_lowrank_workspace(K, 1, r),), dtype=torch.float32, device="cuda")
    for i in (0, 1, 2, 0):
        x = inputs.activation_bf16(1, K, 9, 78, i)
        y = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        A.attnq_gemv_nvfp4_lowrank(W, dev(s), dev(U), dev(V), dev(x.reshape(-1)), ws, y)
        torch.cuda.synchronize()
        y_fresh, _ = _run(A, W, s, U, V, x)
        assert np.array_equal(host(y).view(np.uint32), y_fresh.view(np.uint32)), f"{what}, input {i}"


def test_two_segment_block_with_per_segment_factors(A):
    N, K, r = 4000, 5376, 16
    say(f"lowrank two segments {N}x{K} rank {r}")
    W, parts = _shared(A, N, K, 74, seg_end=[1500, N])
    s, U, V = _segment_factors([1500, N], K, r, 74)
    x = inputs.activation_bf16(1, K, 9, 74, 1)
    y, t = _run(A, W, s, U, V, x)
    _check(y, parts, s, U, V, x, K, np.arange(N), "two-segment block")
    xv = O.bf16_to_f32(x).astype(np.float64).reshape(-1)
    for g in range(2):
        Vf = O.bf16_to_f32(V[g]).astype(np.float64)
        tb = _depth(K, r) * 2.0 ** -24 * (np.abs(Vf).T @ np.abs(xv))
        assert np.all(np.abs(t[g] - Vf.T @ xv) <= tb)


def test_fused_qkv_31b_like_per_segment_factors(A):
    seg_end = [4096, 5120, 6144]
    N, K, r = 6144, 5376, 16
    say(f"lowrank fused q|k|v {N}x{K} rank {r}")
    W, parts = _shared(A, N, K, 76, seg_end=seg_end)
    s, U, V = _segment_factors(seg_end, K, r, 76)
    x = inputs.activation_bf16(1, K, 9, 76, 1)
    y, _ = _run(A, W, s, U, V, x)
    rows = np.unique(np.concatenate([np.arange(4090, 4100), np.arange(5115, 5125), np.arange(N - 4, N),
                                     np.random.default_rng(76).choice(N, 300, replace=False)]))
    _check(y, parts, s, U, V, x, K, rows, "fused q|k|v per-segment")


def test_empty_weight_is_a_no_op(A):
    say("lowrank N=0")
    W = A.NVFP4Weight.empty(0, 64)
    x = torch.zeros((64,), dtype=torch.int16, device="cuda")
    t = torch.full((A.attnq_gemv_nvfp4_lowrank_workspace(64, 1, 4),), 7.0, dtype=torch.float32, device="cuda")
    U = torch.zeros((0, 4), dtype=torch.int16, device="cuda")
    V = torch.zeros((64, 4), dtype=torch.int16, device="cuda")
    A.attnq_gemv_nvfp4_lowrank(W, None, U, V, x, t, torch.empty((0,), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(t == 7.0)      # nothing was launched


@pytest.mark.parametrize("N,K,r", [(21504, 5376, 64), (5376, 21504, 64)])
def test_31b_like_shapes_on_sampled_rows(A, N, K, r):
    what = f"lowrank 31B-like {N}x{K} rank {r}"
    say(what)
    W, parts = _shared(A, N, K, 75)
    s, U, V = _factors(N, K, r, 75, 1)
    x = inputs.activation_bf16(1, K, 9, 75, 1)
    y, _ = _run(A, W, s, U, V, x)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(N - 8, N),
                                     np.random.default_rng(75).choice(N, 400, replace=False)]))
    _check(y, parts, s, U, V, x, K, rows, what)


def _run_splitk(A, W, s, U, V, x, split_ws):
    """attnq_gemv_nvfp4_lowrank_splitk with a fresh NaN-filled t workspace and the given records."""
    r = 0 if U is None else U.shape[1]
    y = torch.full((W.N,), float("nan"), dtype=torch.float32, device="cuda")
    ws = None
    if r:
        ws = torch.full((A.attnq_gemv_nvfp4_lowrank_workspace(W.K, len(W.seg_end), r),), float("nan"),
                        dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4_lowrank_splitk(W, dev(s), dev(U), dev(V), dev(x.reshape(-1)), ws, split_ws, y)
    torch.cuda.synchronize()
    return host(y)


# the split-K form (attnq_gemv_nvfp4_lowrank_splitk): 6 slices (K = 21504 and 24576, rank 16 and 64),
# 5 slices with a ragged last one (K = 16416), rank 0 with s, a two-segment block whose boundary falls
# inside a row tile, and an unsplit row length (K = 8192, the plain low-rank call), every element
# against the oracle's bound; a second call on the same records gives the same bits
@pytest.mark.parametrize("segs,K,r", [((300,), 21504, 16), ((129,), 24576, 64), ((77,), 16416, 3),
                                      ((300,), 21504, 0), ((150, 301), 21504, 16), ((64,), 8192, 8)])
def test_lowrank_splitk_vs_oracle(A, segs, K, r):
    seg_end = list(np.cumsum(segs))
    N = seg_end[-1]
    what = f"lowrank split-K {segs}x{K} rank {r}"
    say(what)
    W, parts = _shared(A, N, K, 77, seg_end=seg_end)
    if len(segs) > 1:
        s, U, V = _segment_factors(seg_end, K, r, 77)
    else:
        s, U, V = _factors(N, K, r, 77, 1)
    x = inputs.activation_bf16(1, K, 9, 77, r)
    split_ws = A.splitk_workspace(N, K)
    y = _run_splitk(A, W, s, U, V, x, split_ws)
    _check(y, parts, s, U, V, x, K, np.arange(N), what)
    y2 = _run_splitk(A, W, s, U, V, x, split_ws)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), what
    if r == 0:
        # with no row terms the epilogue is the split-K GEMV's y times s
        yp = torch.empty((N,), dtype=torch.float32, device="cuda")
        A.attnq_gemv_nvfp4_splitk(W, dev(x.reshape(-1)), yp, split_ws)
        torch.cuda.synchronize()
        assert np.array_equal(y, (host(yp) * O.bf16_to_f32(s)).astype(np.float32)), what
