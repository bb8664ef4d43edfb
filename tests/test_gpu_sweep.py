"""Seeded random sweep over the entry points, against the float64 oracle.

Each case draws, from numpy's PCG64 seeded with the case number (so a failure names a
reproducible case):
* a launch class of the GEMV table by the row length in 32-element chunks (at most 128, 129-192,
  193-511, at least 512) and a K inside it;
* N (log-uniform up to about 3 M elements), a table of 1-4 segments cut at random rows, and the
  theta's rank (passthrough, s only, rank 4 or 16);
* M for the small-M product and r for the runtime low-rank product.

It checks the packed weight bit for bit against the oracle's RTN quantization, then the batch-1
GEMV, the small-M product and the runtime low-rank product to the bounds of their targeted tests,
and on two-segment draws of equal halves the gate|up activation epilogue. The gate|up launch
class (N >= 16384) is left to the targeted tests (16400 x 5376 in the GEMV and low-rank tests,
43008 x 5376 on sampled rows in the full-size tests): the oracle's quantization of a segment
that size takes minutes.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import assert_close_products, assert_same_bits, dev, gpu_quantize, host, oracle_quantize, say
from nvfp4_weight_only_rtn_amd import inputs
from test_gpu_glu import _check_vs_oracle as glu_check
from test_gpu_lowrank import _check as lowrank_check
from test_gpu_lowrank import _run as lowrank_run
from test_gpu_lowrank import _segment_factors

CASES = 64
CLASSES = [(1, 128), (129, 192), (193, 511), (512, 768)]   # chunks of 32 elements per row
MAX_ELEMS = 3_000_000


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def _draw(i):
    rng = np.random.default_rng(20_000 + i)
    lo, hi = CLASSES[i % len(CLASSES)]
    K = 32 * int(rng.integers(lo, hi + 1))
    nmax = max(2, min(16383, MAX_ELEMS // K))
    N = max(1, int(np.exp(rng.uniform(0.0, np.log(nmax)))))
    n_seg = int(rng.integers(1, min(4, N) + 1))
    cuts = np.sort(rng.choice(np.arange(1, N), n_seg - 1, replace=False)) if n_seg > 1 else np.array([], int)
    segs = [int(v) for v in np.diff(np.concatenate([[0], cuts, [N]]))]
    kind = int(rng.integers(0, 4))                    # 0 passthrough, 1 s only, 2 rank 4, 3 rank 16
    M = int(rng.integers(1, 17))
    lr_r = int(rng.choice([1, 3, 8, 16, 64]))
    return K, N, segs, kind, M, lr_r


def _bundles(segs, K, kind, i):
    r = {0: 0, 1: 0, 2: 4, 3: 16}[kind]
    return [inputs.theta_bundle(n, K, r, cfg=11, layer=i, proj=p, passthrough=kind == 0) for p, n in enumerate(segs)]


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(CASES))
def test_sweep_case(A, i):
    K, N, segs, kind, M, lr_r = _draw(i)
    what = f"sweep case {i}: N {N} K {K} segments {segs} theta kind {kind} M {M} r {lr_r}"
    say(what)
    bundles = _bundles(segs, K, kind, i)
    W, seg_end = gpu_quantize(A, bundles, K)
    c, s, t, _ = oracle_quantize(bundles)
    assert_same_bits(host(W.codes), c, f"{what}: codes")
    assert_same_bits(host(W.scales), s, f"{what}: scales")
    assert_same_bits(host(W.tensor_scale), t, f"{what}: tensor scales")

    # batch-1 GEMV
    x = inputs.activation_bf16(1, K, 11, i, 50)
    y = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, dev(x.reshape(-1)), y)
    torch.cuda.synchronize()
    assert_close_products(host(y), O.gemv_nvfp4(c, s, t, x, seg_end), O.abs_dot(c, s, t, x, seg_end)[0],
                          f"{what}: gemv")

    # small-M product
    X = inputs.activation_bf16(M, K, 11, i, 51)
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    A.attnq_gemm_nvfp4_small_m(W, dev(X), Y)
    torch.cuda.synchronize()
    Yr = O.gemm_nvfp4_small_m(c, s, t, X, seg_end)
    ad = O.abs_dot(c, s, t, X, seg_end)
    Yh = host(Y)
    for m in range(M):
        assert_close_products(Yh[m], Yr[m], ad[m], f"{what}: small-M token {m}")

    # runtime low-rank product over the same packed weight, one factor set per segment
    sf, Uf, Vf = _segment_factors(seg_end, K, lr_r, 200 + i)
    xl = inputs.activation_bf16(1, K, 11, i, 52)
    yl, _ = lowrank_run(A, W, sf, Uf, Vf, xl)
    lowrank_check(yl, bundles, sf, Uf, Vf, xl, K, np.arange(N), f"{what}: low-rank")

    # gate|up epilogue when the draw is a pair of equal halves
    if len(segs) == 2 and segs[0] == segs[1]:
        h = torch.full((N // 2,), 0x7FFF, dtype=torch.int16, device="cuda")
        A.attnq_gemv_nvfp4_glu(W, dev(x.reshape(-1)), A.ACT_SILU, h)
        torch.cuda.synchronize()
        glu_check(host(h).view(np.uint16), c, s, t, x, np.arange(N // 2), A.ACT_SILU, f"{what}: glu")


def test_sweep_covers_every_launch_class():
    """The draw reaches every GEMV launch class below the gate|up rows, multi-segment tables and
    every theta kind (a CPU check of the sweep itself)."""
    draws = [_draw(i) for i in range(CASES)]
    cls = {min(j for j, (lo, hi) in enumerate(CLASSES) if K // 32 <= hi) for K, *_ in draws}
    assert cls == set(range(len(CLASSES)))
    assert any(len(segs) >= 3 for _, _, segs, *_ in draws)
    assert {kind for _, _, _, kind, *_ in draws} == {0, 1, 2, 3}
    assert all(sum(segs) == N and min(segs) >= 1 for _, N, segs, *_ in draws)
