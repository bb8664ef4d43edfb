"""Full-size parity at the 31B-like shapes, in the same launch configurations the benchmark
times: the fused q|k|v 6144x5376, o 5376x4096, gate|up 2x21504x5376 and down 5376x21504
projections, the tied bf16 lm_head 262144x5376, the small-M verify product at M = 4 and 8,
and the rank-16 load path. The GPU computes every row; the oracle is evaluated on sampled
rows (every segment's first and last row plus random ones), bit-exact for the packed weight
and within the fp32 bounds for the products."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import assert_close_products, assert_same_bits, dev, gpu_quantize, host, oracle_quantize, say
from nvfp4_weight_only_rtn_amd import inputs

pytestmark = pytest.mark.gpu

H = 5376
SHAPES = {  # name -> (segment rows, K)
    "qkv": ((4096, 1024, 1024), H),
    "o": ((H,), 4096),
    "gate_up": ((21504, 21504), H),
    "down": ((H,), 21504),
}


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def _sample_rows(seg_rows, n_random=96, seed=0):
    g = np.random.default_rng(seed)
    N = sum(seg_rows)
    rows = set(g.choice(N, size=min(n_random, N), replace=False).tolist())
    start = 0
    for n in seg_rows:
        rows |= {start, start + n - 1}
        start += n
    return np.array(sorted(rows))


def _sampled_seg_end(rows, seg_rows):
    ends, start = [], 0
    for n in seg_rows:
        start += n
        ends.append(int(np.sum(rows < start)))
    return ends


def _check_projection(A, name, bundles, seg_rows, K, x, X=None):
    rows = _sample_rows(seg_rows, seed=len(name))
    say(f"full-size {name} quantize")
    W, seg_end = gpu_quantize(A, bundles, K)
    c, s, t, _ = oracle_quantize(bundles, rows=rows)
    assert_same_bits(host(W.codes)[rows], c, f"{name} codes")
    assert_same_bits(host(W.scales)[rows], s, f"{name} scales")
    assert_same_bits(host(W.tensor_scale).view(np.uint32), t.view(np.uint32), f"{name} tensor scales")
    sseg = _sampled_seg_end(rows, seg_rows)
    say(f"full-size {name} gemv")
    y = torch.full((W.N,), np.nan, dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, dev(x.reshape(-1)), y)
    torch.cuda.synchronize()
    yh = host(y)
    assert np.isfinite(yh).all()
    assert_close_products(yh[rows], O.gemv_nvfp4(c, s, t, x, sseg), O.abs_dot(c, s, t, x, sseg)[0], f"{name} gemv")
    if X is not None:
        M = X.shape[0]
        say(f"full-size {name} small-M {M}")
        Y = torch.full((M, W.N), np.nan, dtype=torch.float32, device="cuda")
        A.attnq_gemm_nvfp4_small_m(W, dev(X), Y)
        torch.cuda.synchronize()
        Yh = host(Y)
        assert np.isfinite(Yh).all()
        assert_close_products(Yh[:, rows], O.gemm_nvfp4_small_m(c, s, t, X, sseg), O.abs_dot(c, s, t, X, sseg),
                              f"{name} small-M {M}")
        say(f"full-size {name} small-M {M}, K slices")
        Y.fill_(float("nan"))
        A.attnq_gemm_nvfp4_small_m_splitk(W, dev(X), Y, A.small_m_workspace(W.N, K, M))
        torch.cuda.synchronize()
        Yh = host(Y)
        assert np.isfinite(Yh).all()
        assert_close_products(Yh[:, rows], O.gemm_nvfp4_small_m(c, s, t, X, sseg), O.abs_dot(c, s, t, X, sseg),
                              f"{name} small-M {M}, K slices")


@pytest.mark.parametrize("name", list(SHAPES))
def test_31b_layer_projection(A, name):
    seg_rows, K = SHAPES[name]
    bundles = [inputs.theta_bundle(n, K, 0, cfg=2, layer=0, proj=10 * list(SHAPES).index(name) + i, passthrough=True)
               for i, n in enumerate(seg_rows)]
    x = inputs.activation_bf16(1, K, 2, 0, list(SHAPES).index(name))
    X = inputs.activation_bf16(8, K, 4, 0, list(SHAPES).index(name)) if name in ("gate_up", "down") else None
    _check_projection(A, name, bundles, seg_rows, K, x, X)
    if X is not None:
        # M = 4 (three drafted tokens plus one) through the same weights
        W, _ = gpu_quantize(A, bundles, K)
        say(f"full-size {name} small-M 4")
        rows = _sample_rows(seg_rows, seed=3)
        c, s, t, _ = oracle_quantize(bundles, rows=rows)
        sseg = _sampled_seg_end(rows, seg_rows)
        Y = torch.full((4, W.N), np.nan, dtype=torch.float32, device="cuda")
        A.attnq_gemm_nvfp4_small_m(W, dev(X[:4]), Y)
        torch.cuda.synchronize()
        assert_close_products(host(Y)[:, rows], O.gemm_nvfp4_small_m(c, s, t, X[:4], sseg),
                              O.abs_dot(c, s, t, X[:4], sseg), f"{name} small-M 4")
        Y.fill_(float("nan"))
        A.attnq_gemm_nvfp4_small_m_splitk(W, dev(X[:4]), Y, A.small_m_workspace(W.N, K, 4))
        torch.cuda.synchronize()
        assert_close_products(host(Y)[:, rows], O.gemm_nvfp4_small_m(c, s, t, X[:4], sseg),
                              O.abs_dot(c, s, t, X[:4], sseg), f"{name} small-M 4, K slices")


def test_lm_head_bf16_full_size(A):
    N, K = 262144, H
    say("lm_head generate")
    W = inputs.normal_bf16((N, K), 0.02, 3, 60, 0, 0)
    x = inputs.activation_bf16(1, K, 3, 60, 0)
    rows = _sample_rows((N,), n_random=256, seed=7)
    say("lm_head gemv 262144x5376")
    Wd = dev(W)
    y = torch.full((N,), np.nan, dtype=torch.float32, device="cuda")
    A.attnq_gemv_bf16(Wd, dev(x.reshape(-1)), y)
    torch.cuda.synchronize()
    yh = host(y)
    assert np.isfinite(yh).all()
    assert_close_products(yh[rows], O.gemv_bf16(W, x, rows=rows), O.abs_dot_bf16(W, x, rows=rows), "lm_head")


@pytest.mark.parametrize("name", ["qkv", "o"])
def test_rank16_load_path_full_size(A, name):
    # load path at the 31B-like shapes: s ~ U(0.9, 1.1), rank-16 U, V ~ N(0, 1e-3^2)
    seg_rows, K = SHAPES[name]
    bundles = [inputs.theta_bundle(n, K, 16, cfg=4, layer=1, proj=10 * list(SHAPES).index(name) + i)
               for i, n in enumerate(seg_rows)]
    x = inputs.activation_bf16(1, K, 4, 1, list(SHAPES).index(name))
    _check_projection(A, f"rank16 {name}", bundles, seg_rows, K, x)


def _abs_dot_chunked(c, s, t, x, seg_end, chunk=4096):
    """abs_dot over every row, a row chunk at a time (bounded host memory)."""
    out = np.empty(c.shape[0], dtype=np.float64)
    for a in range(0, c.shape[0], chunk):
        rows = np.arange(a, min(a + chunk, c.shape[0]))
        out[rows] = O.abs_dot(c, s, t, x, seg_end, rows=rows)[0]
    return out


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_every_row_at_full_size(A, name):
    """The dominant launch class (the fused gate|up, 43008 x 5376) and the down projection, each
    quantized by the oracle in full: packed bytes bit-exact on every row, and y on every row within
    the fp32 bounds -- gate|up through attnq_gemv_nvfp4, down through both attnq_gemv_nvfp4 and the
    split-K call."""
    seg_rows, K = SHAPES[name]
    bundles = [inputs.theta_bundle(n, K, 0, cfg=2, layer=5, proj=10 * list(SHAPES).index(name) + i, passthrough=True)
               for i, n in enumerate(seg_rows)]
    x = inputs.activation_bf16(1, K, 2, 5, list(SHAPES).index(name))
    say(f"every row {name}: quantize")
    W, seg_end = gpu_quantize(A, bundles, K)
    c, s, t, _ = oracle_quantize(bundles)
    assert_same_bits(host(W.codes), c, f"{name} codes")
    assert_same_bits(host(W.scales), s, f"{name} scales")
    assert_same_bits(host(W.tensor_scale).view(np.uint32), t.view(np.uint32), f"{name} tensor scales")
    y_ref = O.gemv_nvfp4(c, s, t, x, seg_end, chunk_rows=2048)
    absdot = _abs_dot_chunked(c, s, t, x, seg_end)
    xd = dev(x.reshape(-1))
    say(f"every row {name}: gemv")
    y = torch.full((W.N,), np.nan, dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, xd, y)
    torch.cuda.synchronize()
    assert_close_products(host(y), y_ref, absdot, f"{name} gemv, every row")
    if name == "down":
        say("every row down: split-K gemv")
        ws = A.splitk_workspace(W.N, K)
        y.fill_(float("nan"))
        A.attnq_gemv_nvfp4_splitk(W, xd, y, ws)
        torch.cuda.synchronize()
        assert_close_products(host(y), y_ref, absdot, "down split-K gemv, every row")
