"""GPU parity of the rank-16 load path on whole tiles (N a multiple of 32, K of 128, r = 16): the
matrix-core rebuild with its two passes (attnq_quantize_nvfp4), the staged variant that rebuilds
once into a workspace (attnq_quantize_nvfp4_staged), and attnq_reconstruct, all against the
oracle bit for bit (AttnQuant landing page, "How it works"; "GPU acceleration", "NVFP4
quantization").

With U = V = 0 the rebuild is exactly s*W0 (every rank step adds +0 to an accumulator of +0),
so adversarial blocks, exact E2M1 ties, signed zeros, NaN/inf and tiny segments reach the
rank-16 kernels with values chosen exactly. A segment whose tensor scale is below 2^-117 takes
the per-block path inside the quantize kernel; the cases around that switch are included.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import assert_same_bits, dev, host, host_u16, say
from nvfp4_weight_only_rtn_amd import inputs

pytestmark = pytest.mark.gpu

R = 16


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def _zero_uv(W0, s=None):
    N, K = W0.shape
    if s is None:
        s = np.full(N, 0x3F80, np.uint16)                 # 1.0
    return W0, s, np.zeros((N, R), np.uint16), np.zeros((K, R), np.uint16)


def _run(A, bundles, K, what, staged):
    seg_end, n = [], 0
    for b in bundles:
        n += b[0].shape[0]
        seg_end.append(n)
    W = A.NVFP4Weight.empty(n, K, seg_end)
    W.codes.fill_(0x5A)
    W.scales.fill_(0xA5)
    ws = A.staged_workspace(max(b[0].shape[0] for b in bundles), K, R) if staged else None
    say(f"{what} ({'staged' if staged else 'two rebuilds'})")
    for i, b in enumerate(bundles):
        d = [dev(a) for a in b]
        if staged:
            A.attnq_quantize_nvfp4_staged(*d, W, ws, seg=i)
        else:
            A.attnq_quantize_nvfp4(*d, W, seg=i)
    torch.cuda.synchronize()
    codes, scales, ts = [], [], []
    for b in bundles:
        c, sc, t = O.quantize_segment(O.reconstruct(*b))
        codes.append(c); scales.append(sc); ts.append(t)
    assert_same_bits(host(W.codes), np.concatenate(codes), what + " codes")
    assert_same_bits(host(W.scales), np.concatenate(scales), what + " scales")
    assert_same_bits(host(W.tensor_scale).view(np.uint32), np.array(ts, np.float32).view(np.uint32), what + " ts")
    return W, ws


@pytest.fixture(params=[False, True], ids=["two_rebuilds", "staged"])
def staged(request):
    return request.param


# whole-tile shapes: one strip and one walker; several strips; more row tiles than walkers
# (4096 rows x 5376 columns: 128 row tiles on 48 walkers of 42 strips), a narrow and a wide K
@pytest.mark.parametrize("N,K,uv", [(32, 128, 1e-3), (64, 256, 1e-2), (352, 640, 1e-2), (4096, 5376, 1e-3),
                                    (96, 21504, 1e-3)])
def test_rank16_against_oracle(A, staged, N, K, uv):
    b = inputs.theta_bundle(N, K, R, cfg=9, layer=50, proj=N % 97, uv_sigma=uv)
    _run(A, [b], K, f"rank16 {N}x{K} uv {uv}", staged)


def test_rank16_fused_segments(A, staged):
    # a q|k|v-like fused weight: three rank-16 segments of one K, each with its own tensor scale
    segs = [inputs.theta_bundle(n, 384, R, cfg=9, layer=51, proj=p, uv_sigma=1e-2) for p, n in enumerate((128, 32, 64))]
    _run(A, segs, 384, "rank16 fused q|k|v-like", staged)


def _adversarial_rows(seed, n, K, scale):
    g = np.random.default_rng(seed)
    w = (g.standard_normal((n, K)) * scale).astype(np.float32)
    w[0, :16] = 0.0                                       # an all-zero block
    w[0, 20] = 7 * scale
    w[0, 32:48] = -0.0                                    # negative zeros (s*W0 + 0 gives +0)
    w[1, :16] = np.float32(1e-4 * scale) * g.standard_normal(16)
    w[1, 16:32] = np.linspace(-1, 1, 16) * scale
    w[2, :] = g.choice([-1, 1], K) * np.exp2(g.integers(-30, 0, K)) * scale
    return O.f32_to_bf16_rne(w)


def test_rank16_adversarial_blocks(A, staged):
    W0 = _adversarial_rows(7, 64, 256, 0.02)
    s = inputs.uniform_bf16((64,), 0.9, 1.1, 9, 52, 0, inputs.T_S)
    _run(A, [_zero_uv(W0, s)], 256, "rank16 adversarial blocks", staged)


def test_rank16_exact_ties(A, staged):
    d = 448 * 2.0 ** -10
    q = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5, 4]
    W0 = inputs.bits_from_floats([[v * d for v in q] * 8] * 32)
    _run(A, [_zero_uv(W0)], 128, "rank16 exact E2M1 ties", staged)


@pytest.mark.parametrize("scale", [1e-37, 1e-32, 3e-32, 1e-31])
def test_rank16_small_tensor_scales(A, staged, scale):
    # amax from about 2^-119 to 2^-100: ts on both sides of the 2^-117 switch to the per-block path,
    # fp32 denormal divisors below it
    W0 = _adversarial_rows(8, 32, 128, scale)
    _run(A, [_zero_uv(W0)], 128, f"rank16 tiny segment {scale}", staged)


def test_rank16_zero_nan_inf_segments(A, staged):
    z = np.zeros((32, 128), np.uint16)
    z[3, 7] = 0x8000
    bad = inputs.normal_bf16((32, 128), 0.02, 9, 53, 0, 0).copy()
    bad[5, 9] = 0x7FC0
    inf = inputs.normal_bf16((32, 128), 0.02, 9, 53, 1, 0).copy()
    inf[31, 127] = 0xFF80
    ok = inputs.normal_bf16((32, 128), 0.02, 9, 53, 2, 0)
    W, _ = _run(A, [_zero_uv(z), _zero_uv(bad), _zero_uv(inf), _zero_uv(ok)], 128, "rank16 zero/NaN/-inf/normal", staged)
    ts = host(W.tensor_scale)
    assert ts[0] == 0 and np.isnan(ts[1]) and np.isnan(ts[2]) and np.isfinite(ts[3])


def test_staged_workspace_holds_the_rebuild(A):
    N, K = 256, 640
    b = inputs.theta_bundle(N, K, R, cfg=9, layer=54, proj=0, uv_sigma=1e-2)
    W, ws = _run(A, [b], K, "staged workspace", True)
    assert ws.numel() == A.attnq_quantize_nvfp4_staged_workspace(N, K, R) == 2 * N * K
    assert np.array_equal(ws.cpu().numpy().view(np.uint16).reshape(N, K), O.reconstruct(*b))


def test_staged_other_ranks_and_ragged_shapes(A):
    # the staged call on the generic walk: ranks 4, 40 and a ragged 200 x 320 rank-16 weight
    for (N, K, r) in ((200, 320, 16), (96, 256, 4), (64, 384, 40)):
        b = inputs.theta_bundle(N, K, r, cfg=9, layer=55, proj=r, uv_sigma=1e-2)
        W = A.NVFP4Weight.empty(N, K)
        ws = A.staged_workspace(N, K, r)
        say(f"staged generic {N}x{K} r{r}")
        A.attnq_quantize_nvfp4_staged(*[dev(a) for a in b], W, ws)
        torch.cuda.synchronize()
        c, sc, t = O.quantize(O.reconstruct(*b))
        assert_same_bits(host(W.codes), c, f"staged {N}x{K} r{r} codes")
        assert_same_bits(host(W.scales), sc, f"staged {N}x{K} r{r} scales")
        assert_same_bits(host(W.tensor_scale).view(np.uint32), np.asarray(t, np.float32).view(np.uint32), "ts")


def test_staged_rank0_needs_no_workspace(A):
    b = inputs.theta_bundle(64, 256, 0, cfg=9, layer=56, proj=0)
    assert A.attnq_quantize_nvfp4_staged_workspace(64, 256, 0) == 0
    W = A.NVFP4Weight.empty(64, 256)
    say("staged rank 0")
    A.attnq_quantize_nvfp4_staged(*[dev(a) for a in b], W, None)
    torch.cuda.synchronize()
    c, sc, t = O.quantize(O.reconstruct(*b))
    assert np.array_equal(host(W.codes), c) and np.array_equal(host(W.scales), sc)


def test_staged_repeats_and_matches_two_rebuilds(A):
    b = inputs.theta_bundle(1024, 1152, R, cfg=9, layer=57, proj=0, uv_sigma=1e-2)
    d = [dev(a) for a in b]
    W1 = A.NVFP4Weight.empty(1024, 1152)
    W2 = A.NVFP4Weight.empty(1024, 1152)
    ws = A.staged_workspace(1024, 1152, R)
    say("staged vs two rebuilds 1024x1152")
    A.attnq_quantize_nvfp4(*d, W1)
    for _ in range(3):
        A.attnq_quantize_nvfp4_staged(*d, W2, ws)
        torch.cuda.synchronize()
        assert torch.equal(W1.codes, W2.codes) and torch.equal(W1.scales, W2.scales)
        assert torch.equal(W1.tensor_scale.view(torch.int32), W2.tensor_scale.view(torch.int32))


@pytest.mark.parametrize("N,K,uv", [(32, 128, 1e-2), (352, 640, 1e-2), (96, 5376, 1e-3)])
def test_rank16_reconstruct(A, N, K, uv):
    b = inputs.theta_bundle(N, K, R, cfg=9, layer=58, proj=N % 31, uv_sigma=uv)
    out = torch.empty((N, K), dtype=torch.int16, device="cuda")
    say(f"rank16 reconstruct {N}x{K}")
    A.attnq_reconstruct(*[dev(a) for a in b], out)
    torch.cuda.synchronize()
    assert_same_bits(host_u16(out), O.reconstruct(*b), f"rank16 W_eff {N}x{K}")


def test_rank16_reconstruct_keeps_nan_and_signed_zero_rules(A):
    W0 = _adversarial_rows(9, 32, 128, 0.02).copy()
    W0[4, 5] = 0x7FC1                                     # a NaN with a payload
    W0[6, 7] = 0xFF80                                     # -inf
    b = _zero_uv(W0)
    out = torch.empty((32, 128), dtype=torch.int16, device="cuda")
    say("rank16 reconstruct NaN / -inf / signed zeros")
    A.attnq_reconstruct(*[dev(a) for a in b], out)
    torch.cuda.synchronize()
    assert_same_bits(host_u16(out), O.reconstruct(*b), "rank16 W_eff special values")


def _single_staged(A, b, K, seg_ends, seg):
    W = A.NVFP4Weight.empty(seg_ends[-1], K, seg_ends)
    W.codes.fill_(0x5A)
    W.scales.fill_(0xA5)
    A.attnq_quantize_nvfp4_staged(*[dev(a) for a in b], W, A.staged_workspace(b[0].shape[0], K, b[2].shape[1] if b[2] is not None else 0), seg=seg)
    return W


def _run_batch(A, entries, fill=None):
    """entries: (bundle, weight, seg); returns after the batched call."""
    bundles = [tuple(dev(a) for a in b) for b, _, _ in entries]
    ws = A.staged_batch_workspace(bundles)
    if ws is not None and fill is not None:
        ws.fill_(fill)
    A.attnq_quantize_nvfp4_staged_batch(bundles, [W for _, W, _ in entries], [s for _, _, s in entries], ws)
    torch.cuda.synchronize()


def _segment(W, seg):
    start = 0 if seg == 0 else W.seg_end[seg - 1]
    return host(W.codes)[start:W.seg_end[seg]], host(W.scales)[start:W.seg_end[seg]], host(W.tensor_scale)[seg:seg + 1]


def test_staged_batch_against_oracle_and_single_calls(A):
    """One batch of eight bundles: rank-16 whole-tile bundles of several shapes (rebuilt in one grid,
    runs crossing strips and bundles), three of them the segments of one fused weight; a ragged
    rank-16 bundle, a rank-4 one and a rank-0 one with row scales (each rebuilt on its own); against
    the oracle and against the single staged call, bit for bit."""
    qkv = A.NVFP4Weight.empty(384, 384, [256, 320, 384])
    qkv.codes.fill_(0x5A)
    qkv.scales.fill_(0xA5)
    specs = [((256, 384, 16), qkv, 0), ((64, 384, 16), qkv, 1), ((64, 384, 16), qkv, 2), ((352, 640, 16), None, 0),
             ((32, 128, 16), None, 0), ((200, 320, 16), None, 0), ((96, 256, 4), None, 0), ((64, 256, 0), None, 0)]
    entries = []
    for j, ((N, K, r), W, seg) in enumerate(specs):
        b = inputs.theta_bundle(N, K, r, cfg=9, layer=60, proj=j, uv_sigma=1e-2)    # r = 0: W0 and s
        if W is None:
            W = A.NVFP4Weight.empty(N, K)
            W.codes.fill_(0x5A)
            W.scales.fill_(0xA5)
        entries.append((b, W, seg))
    say("staged batch of 8 bundles")
    _run_batch(A, entries, fill=0xFF)
    for j, (b, W, seg) in enumerate(entries):
        c, sc, ts = _segment(W, seg)
        oc, osc, ot = O.quantize_segment(O.reconstruct(*b))
        what = f"batch bundle {j} {b[0].shape}"
        assert_same_bits(c, oc, what + " codes")
        assert_same_bits(sc, osc, what + " scales")
        assert_same_bits(ts.view(np.uint32), np.array([ot], np.float32).view(np.uint32), what + " ts")
        S = _single_staged(A, b, W.K, W.seg_end, seg)
        torch.cuda.synchronize()
        sc2 = _segment(S, seg)
        assert np.array_equal(c, sc2[0]) and np.array_equal(sc, sc2[1]) and np.array_equal(ts.view(np.uint32), sc2[2].view(np.uint32))


def test_staged_batch_layer_like_equals_single_calls(A):
    """q, k, v (segments of one weight) and o of a 31B-like attention block at rank 16 in one batch,
    twice (the workspace refilled in between), against the single staged calls bit for bit."""
    K = 5376
    qkv = A.NVFP4Weight.empty(6144, K, [4096, 5120, 6144])
    o = A.NVFP4Weight.empty(5376, 4096)
    entries = [(inputs.theta_bundle(n, K, 16, cfg=9, layer=61, proj=j, uv_sigma=1e-3), qkv, j)
               for j, n in enumerate((4096, 1024, 1024))]
    entries.append((inputs.theta_bundle(5376, 4096, 16, cfg=9, layer=61, proj=3, uv_sigma=1e-3), o, 0))
    say("staged batch q|k|v + o")
    _run_batch(A, entries, fill=0x00)
    first = [_segment(W, seg) for _, W, seg in entries]
    _run_batch(A, entries, fill=0x7F)
    for j, (b, W, seg) in enumerate(entries):
        again = _segment(W, seg)
        S = _single_staged(A, b, W.K, W.seg_end, seg)
        torch.cuda.synchronize()
        single = _segment(S, seg)
        for x, y, z in zip(first[j], again, single):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)) and np.array_equal(x.view(np.uint8), z.view(np.uint8)), j
