"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each one.

Every mutation below is a slip someone could make while writing the oracle from the pages:
a swapped nibble order, the wrong tensor-scale divisor, ties rounded away from even, a dropped
low-rank term, a transposed factor, a sign slip or a dropped block in the GEMV. Each must make
at least one of the pins in the other oracle test modules fail.
"""
import numpy as np

import oracle as O
import oracle.attnq_oracle as OM
import test_oracle_gemv as PG
import test_oracle_quantize as PQ
import test_oracle_reconstruct as PR


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_swapped_nibbles_are_caught(monkeypatch, golden_dir):
    orig = OM.quantize_segment

    def swapped(W):
        c, s, t = orig(W)
        return ((c >> 4) | (c << 4)).astype(np.uint8), s, t
    monkeypatch.setattr(OM, "quantize_segment", swapped)
    assert _fails(PQ.test_hand_worked_example, golden_dir)


def test_wrong_tensor_scale_divisor_is_caught(monkeypatch, golden_dir):
    monkeypatch.setattr(OM, "TS_DIVISOR", np.float32(448.0))
    assert _fails(PQ.test_amax_block_takes_the_largest_scale_and_code)
    assert _fails(PQ.test_hand_worked_example, golden_dir)


def test_ties_away_from_even_are_caught(monkeypatch):
    def away(aq):
        a = np.asarray(aq, dtype=np.float32)
        conds = [a < 0.25, a < 0.75, a < 1.25, a < 1.75, a < 2.5, a < 3.5, a < 5.0]
        return np.select(conds, [0, 1, 2, 3, 4, 5, 6], default=7).astype(np.uint8)
    monkeypatch.setattr(OM, "e2m1_encode_magnitude", away)
    assert _fails(PQ.test_brute_force_midpoint_ties)


def test_dropped_rank_term_is_caught(monkeypatch):
    orig = OM.reconstruct

    def dropped(W0, s=None, U=None, V=None):
        if U is None:
            return orig(W0, s)
        return orig(W0, s, U[:, :-1], V[:, :-1])
    monkeypatch.setattr(OM, "reconstruct", dropped)
    monkeypatch.setattr(O, "reconstruct", dropped)
    assert _fails(PR.test_exact_small_integer_lowrank_matches_rational_value)


def test_transposed_factor_is_caught(monkeypatch):
    orig = OM.reconstruct

    def swapped(W0, s=None, U=None, V=None):
        if U is None:
            return orig(W0, s)
        # V indexed by row instead of column: only defined when reading V[:N]
        N = W0.shape[0]
        K = W0.shape[1]
        Vw = np.resize(V[:N][::-1], (K, V.shape[1]))
        return orig(W0, s, U, Vw)
    monkeypatch.setattr(OM, "reconstruct", swapped)
    monkeypatch.setattr(O, "reconstruct", swapped)
    assert _fails(PR.test_exact_small_integer_lowrank_matches_rational_value)


def test_scale_applied_to_wrong_rows_is_caught(monkeypatch):
    orig = OM.row_segment_scale

    def shifted(N, seg_end, ts):
        return orig(N, seg_end, np.roll(np.asarray(ts), 1))
    monkeypatch.setattr(OM, "row_segment_scale", shifted)
    assert _fails(PG.test_gemv_equals_exact_rational_sum)


def test_gemv_sign_slip_is_caught(monkeypatch):
    orig = OM.e2m1_decode

    def nosign(codes):
        return np.abs(orig(codes))
    monkeypatch.setattr(OM, "e2m1_decode", nosign)
    assert _fails(PG.test_gemv_equals_exact_rational_sum)


def test_dropped_block_is_caught(monkeypatch):
    orig = OM.unpack_codes

    def drop_last_block(codes):
        out = orig(codes).copy()
        out[..., -16:] = 0
        return out
    monkeypatch.setattr(OM, "unpack_codes", drop_last_block)
    assert _fails(PG.test_gemv_equals_exact_rational_sum)


def _lowrank_mutant(monkeypatch, slip):
    """Replace the oracle's low-rank product by a version with one slip written in."""
    def mutated(codes, scales, ts, s_bf16, U_bf16, V_bf16, x_bf16, seg_end=None, rows=None):
        y = OM.gemv_nvfp4(codes, scales, ts, x_bf16, seg_end)
        sv = OM.bf16_to_f32(np.asarray(s_bf16)).astype(np.float64)
        x = OM.bf16_to_f32(x_bf16).astype(np.float64).reshape(-1)
        U = OM.bf16_to_f32(np.asarray(U_bf16)).astype(np.float64)
        V = OM.bf16_to_f32(np.asarray(V_bf16)).astype(np.float64).reshape((-1, x.size, U.shape[1]))
        seg = OM.row_segment_index(len(y), seg_end)
        out = slip(y, sv, x, U, V, seg)
        return out if rows is None else out[np.asarray(rows)]
    monkeypatch.setattr(OM, "gemv_nvfp4_lowrank", mutated)
    monkeypatch.setattr(O, "gemv_nvfp4_lowrank", mutated)


def _delta(U, V, x, seg):
    return np.sum(U * np.stack([V[g].T @ x for g in range(V.shape[0])])[seg], axis=1)


def test_lowrank_scale_on_the_delta_is_caught(monkeypatch):
    import test_oracle_lowrank as PL
    _lowrank_mutant(monkeypatch, lambda y, s, x, U, V, seg: s * (y + _delta(U, V, x, seg)))
    assert _fails(PL.test_lowrank_equals_exact_rational_sum)


def test_lowrank_reversed_factor_rows_are_caught(monkeypatch):
    import test_oracle_lowrank as PL
    _lowrank_mutant(monkeypatch, lambda y, s, x, U, V, seg: s * y + _delta(U, V[:, ::-1], x, seg))
    assert _fails(PL.test_lowrank_equals_exact_rational_sum)


def test_lowrank_delta_sign_slip_is_caught(monkeypatch):
    import test_oracle_lowrank as PL
    _lowrank_mutant(monkeypatch, lambda y, s, x, U, V, seg: s * y - _delta(U, V, x, seg))
    assert _fails(PL.test_lowrank_equals_exact_rational_sum)


def test_lowrank_dropped_rank_is_caught(monkeypatch):
    import test_oracle_lowrank as PL
    _lowrank_mutant(monkeypatch, lambda y, s, x, U, V, seg: s * y + _delta(U[:, :-1], V[:, :, :-1], x, seg))
    assert _fails(PL.test_lowrank_equals_exact_rational_sum)


def test_lowrank_first_segment_factors_everywhere_are_caught(monkeypatch):
    import test_oracle_lowrank as PL
    _lowrank_mutant(monkeypatch, lambda y, s, x, U, V, seg: s * y + _delta(U, V, x, np.zeros_like(seg)))
    assert _fails(PL.test_lowrank_equals_exact_rational_sum)


# ---------------------------------------------------------------------------------------------
# the rebuild's rounding sequence (s*W0 + U V^T at rank r > 0)
# ---------------------------------------------------------------------------------------------
def _rebuild_mutant(monkeypatch, combine):
    """Replace the oracle's rebuild at r > 0 by one whose fp32 sequence is `combine(base, u, v)`."""
    orig = OM.reconstruct

    def mutated(W0, s=None, U=None, V=None):
        if U is None or U.shape[1] == 0:
            return orig(W0, s)
        w0 = OM.bf16_to_f32(W0)
        sv = np.ones(w0.shape[0], np.float32) if s is None else OM.bf16_to_f32(s)
        base = (sv[:, None] * w0).astype(np.float32)
        return OM.f32_to_bf16_rne(combine(base, OM.bf16_to_f32(U), OM.bf16_to_f32(V)))
    monkeypatch.setattr(OM, "reconstruct", mutated)
    monkeypatch.setattr(O, "reconstruct", mutated)


def _order_pins_fail():
    import test_oracle_reconstruct_order as PO
    return (_fails(PO.test_worked_example_where_the_order_decides) or
            _fails(PO.test_exact_rounding_sequence_on_cancellation_bundles, 16))


def test_rebuild_with_base_added_first_is_caught(monkeypatch):
    def base_first(base, u, v):
        w = base.copy()
        for k in range(u.shape[1]):
            w = (w + u[:, k][:, None] * v[:, k][None, :]).astype(np.float32)
        return w
    _rebuild_mutant(monkeypatch, base_first)
    assert _order_pins_fail()


def test_rebuild_summed_in_float64_and_rounded_once_is_caught(monkeypatch):
    def once(base, u, v):
        return (base.astype(np.float64) + u.astype(np.float64) @ v.astype(np.float64).T).astype(np.float32)
    _rebuild_mutant(monkeypatch, once)
    assert _order_pins_fail()


def test_rebuild_with_rank_terms_descending_is_caught(monkeypatch):
    def descending(base, u, v):
        acc = np.zeros(base.shape, np.float32)
        for k in reversed(range(u.shape[1])):
            acc = (acc + u[:, k][:, None] * v[:, k][None, :]).astype(np.float32)
        return (base + acc).astype(np.float32)
    _rebuild_mutant(monkeypatch, descending)
    assert _fails(__import__("test_oracle_reconstruct_order").test_exact_rounding_sequence_on_cancellation_bundles, 16)


# ---------------------------------------------------------------------------------------------
# the gate|up pairing of the fused epilogue
# ---------------------------------------------------------------------------------------------
def test_gate_and_up_swapped_is_caught(monkeypatch):
    import test_oracle_glu as PGL
    orig = OM.gemv_nvfp4_glu

    def swapped(codes, scales, ts, x_bf16, rows=None):
        g, u = orig(codes, scales, ts, x_bf16, rows)
        return u, g
    monkeypatch.setattr(OM, "gemv_nvfp4_glu", swapped)
    monkeypatch.setattr(O, "gemv_nvfp4_glu", swapped)
    assert _fails(PGL.test_hand_built_gate_up_pairs)


def test_gate_up_pairs_shifted_is_caught(monkeypatch):
    import test_oracle_glu as PGL
    orig = OM.gemv_nvfp4_glu

    def shifted(codes, scales, ts, x_bf16, rows=None):
        g, u = orig(codes, scales, ts, x_bf16, rows)
        return g, np.roll(u, 1)
    monkeypatch.setattr(OM, "gemv_nvfp4_glu", shifted)
    monkeypatch.setattr(O, "gemv_nvfp4_glu", shifted)
    assert _fails(PGL.test_hand_built_gate_up_pairs)
