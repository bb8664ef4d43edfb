"""GPU parity of the load path through the C ABI: attnq_reconstruct and attnq_quantize_nvfp4
against the oracle, bit for bit (codes, block scales, tensor scales, W_eff)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import assert_same_bits, dev, gpu_quantize, host, host_u16, oracle_quantize, say
from nvfp4_weight_only_rtn_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def _check_quant(A, bundles, K, what):
    say(what)
    W, seg_end = gpu_quantize(A, bundles, K)
    c, s, t, oseg = oracle_quantize(bundles)
    assert seg_end == oseg
    assert_same_bits(host(W.codes), c, what + " codes")
    assert_same_bits(host(W.scales), s, what + " scales")
    assert_same_bits(host(W.tensor_scale).view(np.uint32), t.view(np.uint32), what + " tensor scales")
    return W


def test_quantize_single_projection_passthrough(A):
    # 1024x1152 bf16 ~ N(0, 0.02^2), s = 1, no low-rank pair
    _check_quant(A, [inputs.theta_bundle(1024, 1152, 0, cfg=0, layer=0, proj=0, passthrough=True)], 1152,
                 "quantize 1024x1152 passthrough")


def test_quantize_small_decoder_layer(A):
    # 1B-like layer: fused q|k|v 1024+256+256 x 1152, o 1152x1024, gate|up 2x6912x1152, down 1152x6912;
    # s ~ U(0.9, 1.1), rank-4 U, V ~ N(0, 1e-3^2)
    L = 0
    qkv = [inputs.theta_bundle(n, 1152, 4, cfg=1, layer=L, proj=p) for p, n in enumerate((1024, 256, 256))]
    _check_quant(A, qkv, 1152, "1B-like fused qkv")
    _check_quant(A, [inputs.theta_bundle(1152, 1024, 4, cfg=1, layer=L, proj=3)], 1024, "1B-like o_proj")
    gu = [inputs.theta_bundle(6912, 1152, 4, cfg=1, layer=L, proj=p) for p in (4, 5)]
    _check_quant(A, gu, 1152, "1B-like gate|up")
    _check_quant(A, [inputs.theta_bundle(1152, 6912, 4, cfg=1, layer=L, proj=6)], 6912, "1B-like down")


@pytest.mark.parametrize("r,uv", [(1, 1e-2), (16, 1e-3), (16, 1e-2), (33, 1e-2), (64, 1e-2)])
def test_quantize_ranks(A, r, uv):
    b = inputs.theta_bundle(200, 320, r, cfg=9, layer=20, proj=r, uv_sigma=uv)
    _check_quant(A, [b], 320, f"rank {r} uv {uv} 200x320")


@pytest.mark.parametrize("N,K", [(1, 32), (3, 64), (17, 96), (129, 2080), (4097, 32)])
def test_quantize_ragged_shapes(A, N, K):
    _check_quant(A, [inputs.theta_bundle(N, K, 0, cfg=9, layer=21, proj=N, passthrough=True)], K,
                 f"ragged {N}x{K}")


def _adversarial(seed, n, K, scale=0.02):
    g = np.random.default_rng(seed)
    w = (g.standard_normal((n, K)) * scale).astype(np.float32)
    w[0, :16] = 0.0
    w[0, 16:32] = 0.0
    w[0, 20] = 7 * scale
    w[0, 32:48] = -0.0
    w[1, :16] = np.float32(1e-4 * scale) * g.standard_normal(16)
    w[1, 16:32] = np.linspace(-1, 1, 16) * scale
    w[1, 32:48] = g.standard_normal(16) * scale      # signed zeros inside a block with a non-zero scale
    w[1, 33] = -0.0
    w[1, 35] = 0.0
    w[2, :] = g.choice([-1, 1], K) * np.exp2(g.integers(-30, 0, K)) * scale
    # exact E2M1 midpoints relative to the block step of a block whose bamax sits at 448 * 6 * ts
    return O.f32_to_bf16_rne(w)


def test_quantize_adversarial_blocks(A):
    W = _adversarial(5, 8, 128)
    _check_quant(A, [(W, None, None, None)], 128, "adversarial blocks")


def test_quantize_exact_ties(A):
    d = 448 * 2.0 ** -10
    q = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5, -0.0]
    W = inputs.bits_from_floats([[v * d for v in q] * 4] * 3)
    _check_quant(A, [(W, None, None, None)], 64, "exact E2M1 ties")


def test_quantize_tiny_magnitudes_use_fp32_denormals(A):
    # amax ~ 1e-36: ts and every d are fp32 denormals; the GPU must not flush them
    W = _adversarial(6, 4, 64, scale=1e-37)
    _check_quant(A, [(W, None, None, None)], 64, "denormal tensor scale")


def test_quantize_zero_and_nonfinite_segments(A):
    z = np.zeros((16, 64), np.uint16)
    z[3, 7] = 0x8000
    bad = inputs.normal_bf16((16, 64), 0.02, 9, 22, 0, 0).copy()
    bad[5, 9] = 0x7FC0
    inf = inputs.normal_bf16((16, 64), 0.02, 9, 22, 1, 0).copy()
    inf[0, 0] = 0xFF80
    ok = inputs.normal_bf16((16, 64), 0.02, 9, 22, 2, 0)
    W = _check_quant(A, [(z, None, None, None), (bad, None, None, None), (inf, None, None, None), (ok, None, None, None)],
                     64, "zero / NaN / -inf / normal segments")
    ts = host(W.tensor_scale)
    assert ts[0] == 0 and np.isnan(ts[1]) and np.isnan(ts[2]) and np.isfinite(ts[3])


def test_quantize_leaves_other_segments_alone(A):
    say("segment isolation")
    b = inputs.theta_bundle(32, 64, 0, cfg=9, layer=23, proj=0, passthrough=True)
    W = A.NVFP4Weight.empty(96, 64, [32, 64, 96])
    W.codes.fill_(0xAB); W.scales.fill_(0xCD); W.tensor_scale.fill_(-1.0)
    A.attnq_quantize_nvfp4(dev(b[0]), None, None, None, W, seg=1)
    torch.cuda.synchronize()
    c, s, t = O.quantize(b[0])
    codes, scales, ts = host(W.codes), host(W.scales), host(W.tensor_scale)
    assert (codes[:32] == 0xAB).all() and (codes[64:] == 0xAB).all()
    assert (scales[:32] == 0xCD).all() and (scales[64:] == 0xCD).all()
    assert ts[0] == -1.0 and ts[2] == -1.0 and ts[1] == t[0]
    assert np.array_equal(codes[32:64], c) and np.array_equal(scales[32:64], s)


def test_quantize_is_deterministic(A):
    b = [inputs.theta_bundle(6912, 1152, 4, cfg=1, layer=1, proj=4)]
    say("determinism 6912x1152 r4")
    W1, _ = gpu_quantize(A, b, 1152)
    W2, _ = gpu_quantize(A, b, 1152)
    assert torch.equal(W1.codes, W2.codes) and torch.equal(W1.scales, W2.scales)
    assert torch.equal(W1.tensor_scale, W2.tensor_scale)


def test_quantize_empty_is_noop(A):
    say("empty quantize")
    W = A.NVFP4Weight.empty(0, 64, [0])
    A.attnq_quantize_nvfp4(torch.empty((0, 64), dtype=torch.int16, device="cuda"), None, None, None, W, 0)
    torch.cuda.synchronize()
    assert host(W.tensor_scale)[0] == 0.0


@pytest.mark.parametrize("case", ["passthrough", "scale_only", "rank4", "rank16_stress", "rank40", "rank64"])
def test_reconstruct_bit_exact(A, case):
    N, K = 300, 448
    if case == "passthrough":
        b = inputs.theta_bundle(N, K, 0, cfg=9, layer=24, proj=0, passthrough=True)
    elif case == "scale_only":
        b = inputs.theta_bundle(N, K, 0, cfg=9, layer=24, proj=1)
    elif case == "rank4":
        b = inputs.theta_bundle(N, K, 4, cfg=9, layer=24, proj=2)
    elif case == "rank16_stress":
        b = inputs.theta_bundle(N, K, 16, cfg=9, layer=24, proj=3, uv_sigma=1e-2)
    elif case == "rank40":                      # two staged chunks of k, the second partial
        b = inputs.theta_bundle(N, K, 40, cfg=9, layer=24, proj=5, uv_sigma=1e-2)
    else:
        b = inputs.theta_bundle(N, K, 64, cfg=9, layer=24, proj=4, uv_sigma=1e-2)
    say(f"reconstruct {case} {N}x{K}")
    out = torch.empty((N, K), dtype=torch.int16, device="cuda")
    A.attnq_reconstruct(*[dev(a) for a in b], out)
    torch.cuda.synchronize()
    ref = O.reconstruct(*b)
    assert_same_bits(host_u16(out), ref, f"W_eff {case}")
    if case == "passthrough":
        assert np.array_equal(host_u16(out), b[0])
