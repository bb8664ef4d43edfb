"""Pins of the oracle's rounding sequence for W_eff = s*W0 + U V^T at rank r > 0 (AttnQuant landing
page, "How it works"; weightless "GPU and cache acceleration", "Precompute-outside").

The reading fixed for the rebuild is: acc = +0; for k = 0 .. r-1 ascending, acc = fl32(acc + U[i,k]
V[j,k]); w = fl32(s_i W0[i,j] + acc); W_eff = bf16_rne(w). The closed-form pins elsewhere (exact
small integers, one bf16 ulp of the float64 value) hold for other orders too, so this module pins
the order itself, with arithmetic that owes nothing to numpy's float32:

* exact rational arithmetic (fractions.Fraction) with a round-to-nearest-even step written from
  the IEEE 754 definition (round to p significant bits, ties to the even significand), itself
  checked against numpy's float64 -> float32 cast and torch's float32 -> bfloat16 cast;
* a worked example, derived by hand below, in which the documented order gives another bf16
  value than adding s*W0 first or summing exactly with one rounding;
* every element of "cancellation" bundles (W0 = -bf16(U[:,0] V[:,0]^T), so s*W0 + acc leaves a
  residual made of the low-order bits of acc), where the order decides hundreds of elements;
  the test also shows that each alternative order differs from the documented one there;
* an independent scalar loop in numpy float32 scalars, element by element in the documented
  order, on stress bundles of rank 3, 16 and 40 with U, V ~ N(0, 1e-2^2).
"""
from fractions import Fraction
import struct

import numpy as np
import pytest
import torch

import oracle as O
from nvfp4_weight_only_rtn_amd import inputs


# ---------------------------------------------------------------------------------------------
# exact arithmetic with explicit IEEE rounding steps
# ---------------------------------------------------------------------------------------------
EMIN = -126    # smallest normal exponent of binary32 and of bfloat16


def round_sig(q: Fraction, p: int) -> Fraction:
    """q rounded to nearest with p significant bits, ties to an even significand; below 2^EMIN the
    quantum stays 2^(EMIN - p + 1) (gradual underflow). No overflow in these tests."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()    # 2^e <= a < 2^(e+2)
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, EMIN)
    quantum = Fraction(2) ** (e - p + 1)
    n = a / quantum
    whole = n.numerator // n.denominator
    frac = n - whole
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    assert whole * quantum < Fraction(2) ** 127
    return (1 if q > 0 else -1) * whole * quantum


def fl32(q: Fraction) -> Fraction:
    return round_sig(q, 24)


def bf16_round(q: Fraction) -> Fraction:
    return round_sig(q, 8)


def value_of_bf16(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0])


def bits_of_bf16_value(q: Fraction) -> int:
    (u,) = struct.unpack("<I", struct.pack("<f", float(q)))
    assert u & 0xFFFF == 0, "not a bf16 value"
    return u >> 16


def rebuild(order: str, s: Fraction, w0: Fraction, u, v) -> Fraction:
    """One element of W_eff (before the bf16 step) in a given rounding order, all steps exact
    rational arithmetic followed by an explicit fp32 rounding."""
    terms = [uk * vk for uk, vk in zip(u, v)]           # bf16 x bf16: exact in fp32 anyway
    if order == "documented":                           # acc from +0, k ascending, then s*W0 + acc
        acc = Fraction(0)
        for t in terms:
            acc = fl32(acc + t)
        return fl32(s * w0 + acc)
    if order == "base_first":                           # w = s*W0, then w += U[k] V[k]
        w = fl32(s * w0)
        for t in terms:
            w = fl32(w + t)
        return w
    if order == "exact_once":                           # the exact sum, rounded once
        return fl32(s * w0 + sum(terms))
    if order == "descending":                           # acc with k descending
        acc = Fraction(0)
        for t in reversed(terms):
            acc = fl32(acc + t)
        return fl32(s * w0 + acc)
    raise ValueError(order)


ALTERNATIVES = ("base_first", "exact_once", "descending")


def exact_rebuild_bits(W0, s, U, V, order="documented") -> np.ndarray:
    N, K = W0.shape
    r = U.shape[1]
    w0 = [[value_of_bf16(b) for b in row] for row in W0]
    sv = [value_of_bf16(b) for b in s]
    u = [[value_of_bf16(b) for b in row] for row in U]
    v = [[value_of_bf16(b) for b in row] for row in V]
    # Fraction keeps no sign of zero. With no zero among the inputs, every zero on the way is an
    # exact cancellation of two nonzero operands, which round-to-nearest returns as +0.
    assert r > 0 and all(x != 0 for a in (w0, u, v) for row in a for x in row) and all(x != 0 for x in sv)
    out = np.empty((N, K), dtype=np.uint16)
    for i in range(N):
        for j in range(K):
            w = rebuild(order, sv[i], w0[i][j], u[i], v[j])
            out[i, j] = 0x0000 if w == 0 else bits_of_bf16_value(bf16_round(w))
    return out


# ---------------------------------------------------------------------------------------------
# the rounding helpers against library casts
# ---------------------------------------------------------------------------------------------
def test_round_sig_matches_library_casts():
    rng = np.random.default_rng(11)
    a = rng.standard_normal(4000) * np.exp2(rng.integers(-140, 40, 4000).astype(np.float64))
    # exact binary32 ties: a float32 value plus half its ulp (or half the subnormal quantum)
    f = rng.standard_normal(1000).astype(np.float32) * np.float32(2.0) ** rng.integers(-130, 30, 1000).astype(np.float32)
    ulp = np.spacing(np.abs(f)).astype(np.float64)
    ties = f.astype(np.float64) + np.sign(f.astype(np.float64)) * ulp / 2
    for x in np.concatenate([a, ties[np.isfinite(ties) & (f != 0)]]):
        assert fl32(Fraction(float(x))) == Fraction(float(np.float32(x))), x
    # bf16: torch's float32 -> bfloat16 cast on float32 values, ties included
    g = rng.standard_normal(4000).astype(np.float32) * np.float32(2.0) ** rng.integers(-120, 40, 4000).astype(np.float32)
    bits = g.view(np.uint32)
    tie_bits = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    vals = np.concatenate([g, tie_bits.view(np.float32)])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, w in zip(vals, want):
        assert bits_of_bf16_value(bf16_round(Fraction(float(x)))) == int(w), x


# ---------------------------------------------------------------------------------------------
# a worked example
# ---------------------------------------------------------------------------------------------
def test_worked_example_where_the_order_decides():
    """s = 1, W0 = 1, U = [-3/32, 113 * 2^-22], V row = [233/32, 171 * 2^-18] (all bf16 values).
    The terms are t0 = -699/1024 and t1 = 19323 * 2^-40 (about 1.76e-8).

    Documented order: acc = t0 (exact); acc + t1 lies in [1/2, 1), whose fp32 ulp is 2^-24, and t1
    is below half of it, so acc stays -699/1024. w = fl32(1 - 699/1024) = 325/1024 exactly. 325
    needs nine significant bits, so bf16 sees a tie between 324/1024 and 326/1024 and keeps the
    even significand: 81/256 = 0.31640625 = 0x3EA2.

    s*W0 first: w = fl32(1 + t0) = 325/1024, then 325/1024 + t1 lies in [1/4, 1/2) with fp32 ulp
    2^-25, and t1 exceeds half of it, so w = 325/1024 + 2^-25, which is above the bf16 tie:
    163/512 = 0.318359375 = 0x3EA3. The exact sum rounded once gives the same 0x3EA3."""
    one = 0x3F80
    W0 = np.array([[one]], dtype=np.uint16)
    s = np.array([one], dtype=np.uint16)
    U = inputs.bits_from_floats([[-3 / 32, 113 * 2.0 ** -22]])
    V = inputs.bits_from_floats([[233 / 32, 171 * 2.0 ** -18]])
    assert O.reconstruct(W0, s, U, V)[0, 0] == 0x3EA2
    assert exact_rebuild_bits(W0, s, U, V)[0, 0] == 0x3EA2
    assert exact_rebuild_bits(W0, s, U, V, "base_first")[0, 0] == 0x3EA3
    assert exact_rebuild_bits(W0, s, U, V, "exact_once")[0, 0] == 0x3EA3


# ---------------------------------------------------------------------------------------------
# every element of bundles where the order matters
# ---------------------------------------------------------------------------------------------
def _torch_bf16(a32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cancellation_bundle(N: int, K: int, r: int, layer: int):
    """U, V ~ N(0, 1) in column 0 and N(0, 1) * 2^-12 in the others; s ~ U(0.9, 1.1) is replaced by
    ones so that W0 = -bf16(U[:,0] V[:,0]^T) cancels the leading term to within one bf16 step."""
    U = _f32(inputs.normal_bf16((N, r), 1.0, 9, layer, r, inputs.T_U)).copy()
    V = _f32(inputs.normal_bf16((K, r), 1.0, 9, layer, r, inputs.T_V)).copy()
    U[:, 1:] *= np.float32(2.0 ** -12)
    V[:, 1:] *= np.float32(2.0 ** -12)
    U, V = _torch_bf16(U), _torch_bf16(V)
    lead = _f32(U)[:, 0][:, None].astype(np.float64) * _f32(V)[:, 0][None, :].astype(np.float64)
    W0 = _torch_bf16(-lead.astype(np.float32))          # the product is exact in fp32
    s = np.full(N, 0x3F80, dtype=np.uint16)
    return W0, s, U, V


@pytest.mark.parametrize("r", [3, 16, 40])
def test_exact_rounding_sequence_on_cancellation_bundles(r):
    W0, s, U, V = cancellation_bundle(8, 32, r, layer=r)
    want = exact_rebuild_bits(W0, s, U, V)
    assert np.array_equal(O.reconstruct(W0, s, U, V), want)
    # the bundle discriminates: each alternative order changes some of its elements
    for order in ALTERNATIVES:
        assert np.any(exact_rebuild_bits(W0, s, U, V, order) != want), order


# ---------------------------------------------------------------------------------------------
# an independent scalar loop on the stress distributions
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("r,N,K", [(3, 48, 96), (16, 32, 64), (40, 24, 64)])
def test_scalar_float32_loop_on_stress_bundles(r, N, K):
    W0, s, U, V = inputs.theta_bundle(N, K, r, cfg=9, layer=20, proj=r, uv_sigma=1e-2)
    w0, sv, u, v = _f32(W0), _f32(s), _f32(U), _f32(V)
    w = np.empty((N, K), dtype=np.float32)
    for i in range(N):
        for j in range(K):
            acc = np.float32(0.0)
            for k in range(r):
                acc = np.float32(acc + np.float32(u[i, k] * v[j, k]))
            w[i, j] = np.float32(np.float32(sv[i] * w0[i, j]) + acc)
    assert np.array_equal(O.reconstruct(W0, s, U, V), _torch_bf16(w))
