"""Pins of the oracle's reconstruction W_eff = s*W0 + U V^T (AttnQuant landing page,
"How it works"; weightless "GPU and cache acceleration", "Precompute-outside").

- passthrough (s = 1, no low-rank pair) rebuilds W0 bit for bit (Throughput, "Where the
  throughput comes from": the passthrough decomposition reconstructs the original weights
  bit-for-bit);
- s only: equals the bf16 rounding of the exact product, computed in float64 and rounded by
  torch's cast;
- exact small-integer cases: when every intermediate is exactly representable, the result is
  the bf16 rounding of the exact rational value (catches a transposed or dropped factor);
- rank r on the real distributions: within one bf16 ulp of the float64 closed form.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle as O
from nvfp4_weight_only_rtn_amd import inputs


def _torch_bf16(a64: np.ndarray) -> np.ndarray:
    # a64 must hold fp32-exact values (checked) so torch's cast rounds once
    a32 = a64.astype(np.float32)
    assert np.array_equal(a32.astype(np.float64), a64)
    return torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_passthrough_is_bit_exact():
    W0, _, _, _ = inputs.theta_bundle(64, 96, 0, cfg=9, layer=0, proj=0, passthrough=True)
    assert np.array_equal(O.reconstruct(W0), W0)
    ones = np.full(64, 0x3F80, dtype=np.uint16)
    assert np.array_equal(O.reconstruct(W0, ones), W0)
    zU = np.zeros((64, 4), np.uint16)
    zV = np.zeros((96, 4), np.uint16)
    assert np.array_equal(O.reconstruct(W0, ones, zU, zV), W0)   # no zeros in W0, so no -0 issue


def test_passthrough_keeps_negative_zero_only_without_delta():
    W0 = inputs.bits_from_floats([[-0.0, 0.0, 1.5, -2.0] * 8])
    assert np.array_equal(O.reconstruct(W0), W0)
    zU = np.zeros((1, 2), np.uint16)
    zV = np.zeros((32, 2), np.uint16)
    out = O.reconstruct(W0, None, zU, zV)        # -0 + (+0) = +0 under round-to-nearest
    assert out[0, 0] == 0x0000 and out[0, 1] == 0x0000
    assert np.array_equal(out[0, 2:4], W0[0, 2:4])


def test_row_scale_only_matches_exact_product():
    W0, s, _, _ = inputs.theta_bundle(128, 64, 0, cfg=9, layer=1, proj=0)
    exact = O.bf16_to_f32(s).astype(np.float64)[:, None] * O.bf16_to_f32(W0).astype(np.float64)
    assert np.array_equal(O.reconstruct(W0, s), _torch_bf16(exact))


def test_exact_small_integer_lowrank_matches_rational_value():
    # every value is a small integer times a power of two, so every fp32 step is exact;
    # the result must be the single bf16 rounding of the exact rational W_eff.
    g = np.random.default_rng(3)
    N, K, r = 5, 32, 3
    W0f = g.integers(-200, 200, (N, K)) / 64.0
    sf = g.integers(1, 8, N) / 4.0
    Uf = g.integers(-7, 8, (N, r)) / 8.0
    Vf = g.integers(-7, 8, (K, r)) / 16.0
    W0, s, U, V = (inputs.bits_from_floats(a) for a in (W0f, sf, Uf, Vf))
    got = O.reconstruct(W0, s, U, V)
    exact = np.empty((N, K), dtype=np.float64)
    for i in range(N):
        for j in range(K):
            v = Fraction(sf[i]) * Fraction(W0f[i, j]) + sum(Fraction(Uf[i, k]) * Fraction(Vf[j, k]) for k in range(r))
            exact[i, j] = float(v)
    assert np.array_equal(got, _torch_bf16(exact))


def test_lowrank_within_one_bf16_ulp_of_fp64_closed_form():
    for r in (4, 16):
        W0, s, U, V = inputs.theta_bundle(96, 160, r, cfg=9, layer=2, proj=r, uv_sigma=1e-2)
        got = O.bf16_to_f32(O.reconstruct(W0, s, U, V)).astype(np.float64)
        f = lambda a: O.bf16_to_f32(a).astype(np.float64)
        exact = f(s)[:, None] * f(W0) + f(U) @ f(V).T
        # one bf16 ulp at |exact|: 2^(floor(log2|exact|) - 7)
        ulp = np.exp2(np.floor(np.log2(np.abs(exact))) - 7)
        assert np.all(np.abs(got - exact) <= ulp)
        # and the delta really changes a visible fraction of the weights
        base = O.reconstruct(W0, s)
        assert np.mean(O.reconstruct(W0, s, U, V) != base) > 0.05
