"""GPU parity of the fused gate|up projection with its activation (attnq_gemv_nvfp4_glu):
h[j] = bf16(act(gate_j) * up_j) for a two-segment [gate; up] NVFP4 weight.

* identity activation: h equals bf16(fl32(y[j] * y[F + j])) computed from attnq_gemv_nvfp4's own
  outputs bit for bit wherever the plain GEMV takes the same per-row summation (rows of up to
  6144 elements), which pins the row pairing and the epilogue wiring;
* GELU-tanh and SiLU against the float64 oracle: every element within one bf16 step of the
  oracle's single rounding plus the fp32 GEMV bound propagated through act and the product, and
  relative L2 <= 1e-3 (the contract) -- at ragged shapes, the 1B-like gate|up, long rows (loop
  kernel) and the 31B-like 2 x 21504 x 5376 shape on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import dev, gpu_quantize, host, oracle_quantize, say
from nvfp4_weight_only_rtn_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def _bundles(F, K, r, layer):
    return [inputs.theta_bundle(F, K, r, cfg=9, layer=layer, proj=p, passthrough=(r == 0)) for p in (0, 1)]


def _run(A, W, x, act):
    h = torch.full((W.N // 2,), 0x7FFF, dtype=torch.int16, device="cuda")
    A.attnq_gemv_nvfp4_glu(W, dev(x.reshape(-1)), act, h)
    torch.cuda.synchronize()
    return host(h).view(np.uint16)


@pytest.mark.parametrize("F,K", [(17, 96), (1000, 2080), (6912, 1152), (2000, 5376), (8200, 5376)])
def test_glu_identity_matches_the_gemv_bitwise(A, F, K):
    say(f"glu identity {F}x{K}")
    W, _ = gpu_quantize(A, _bundles(F, K, 0, 40), K)
    x = inputs.activation_bf16(1, K, 9, 40, F)
    h = _run(A, W, x, A.ACT_IDENTITY)
    y = torch.empty((W.N,), dtype=torch.float32, device="cuda")
    A.attnq_gemv_nvfp4(W, dev(x.reshape(-1)), y)
    torch.cuda.synchronize()
    yh = host(y)
    want = O.f32_to_bf16_rne((yh[:F] * yh[F:]).astype(np.float32))
    assert np.array_equal(h, want)


def _check_vs_oracle(h, c, s, t, x, rows, act, what):
    g, u = O.gemv_nvfp4_glu(c, s, t, x, rows=None)
    href = O.bf16_to_f32(O.glu(g, u, act)).astype(np.float64)
    hg = O.bf16_to_f32(h[rows]).astype(np.float64)
    F = c.shape[0] // 2
    sseg = [F, 2 * F]
    ad_g = O.abs_dot(c, s, t, x, sseg, rows=np.arange(F))[0]
    ad_u = O.abs_dot(c, s, t, x, sseg, rows=np.arange(F, 2 * F))[0]
    a = O.activation(g, act)
    bound = 2.0 ** -8 * np.abs(href) + 2.0 ** -14 * (ad_g * np.abs(u) + ad_u * np.abs(a)) + 1e-30
    err = np.abs(hg - href)
    bad = np.argwhere(~(err <= bound))
    assert len(bad) == 0, f"{what}: {len(bad)} elements out of bound, first {bad[:5].ravel().tolist()}"
    rel = np.linalg.norm(hg - href) / np.linalg.norm(href)
    assert rel <= 1e-3, f"{what}: rel-L2 {rel}"


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("F,K,r", [(17, 96, 0), (1000, 2080, 0), (6912, 1152, 4), (300, 21504, 0), (77, 16384 + 32, 0)])
def test_glu_activation_vs_oracle(A, act, F, K, r):
    what = f"glu act {act} {F}x{K} rank {r}"
    say(what)
    b = _bundles(F, K, r, 41)
    W, _ = gpu_quantize(A, b, K)
    c, s, t, _ = oracle_quantize(b)
    x = inputs.activation_bf16(1, K, 9, 41, F + act)
    h = _run(A, W, x, act)
    _check_vs_oracle(h, c, s, t, x, np.arange(F), act, what)


def test_glu_31b_gate_up_sampled_rows(A):
    F, K = 21504, 5376
    say("glu 31B-like gate|up")
    b = _bundles(F, K, 0, 42)
    W, _ = gpu_quantize(A, b, K)
    x = inputs.activation_bf16(1, K, 9, 42, 0)
    h = _run(A, W, x, O.ACT_GELU_TANH)
    g = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, F - 1], g.choice(F, 254, replace=False)]))
    rows_all = np.concatenate([rows, rows + F])
    c, s, t, _ = oracle_quantize(b, rows=rows_all)
    n = len(rows)
    gg = O.gemv_nvfp4(c, s, t, x, [n, 2 * n], rows=np.arange(n))
    uu = O.gemv_nvfp4(c, s, t, x, [n, 2 * n], rows=np.arange(n, 2 * n))
    href = O.bf16_to_f32(O.glu(gg, uu, O.ACT_GELU_TANH)).astype(np.float64)
    hg = O.bf16_to_f32(h[rows]).astype(np.float64)
    ad_g = O.abs_dot(c, s, t, x, [n, 2 * n], rows=np.arange(n))[0]
    ad_u = O.abs_dot(c, s, t, x, [n, 2 * n], rows=np.arange(n, 2 * n))[0]
    bound = 2.0 ** -8 * np.abs(href) + 2.0 ** -14 * (ad_g * np.abs(uu) + ad_u * np.abs(O.activation(gg, 0))) + 1e-30
    assert np.all(np.abs(hg - href) <= bound)
    assert np.linalg.norm(hg - href) / np.linalg.norm(href) <= 1e-3


def test_glu_rejects_non_pair_layouts(A):
    W = A.NVFP4Weight.empty(96, 64, [32, 96])
    x = torch.zeros(64, dtype=torch.int16, device="cuda")
    h = torch.zeros(48, dtype=torch.int16, device="cuda")
    with pytest.raises(A.AttnqError):
        A.attnq_gemv_nvfp4_glu(W, x, 0, h)
    W2 = A.NVFP4Weight.empty(96, 64, [48, 96])
    with pytest.raises(A.AttnqError):
        A.attnq_gemv_nvfp4_glu(W2, x, 7, h)
