"""Helpers for the GPU parity tests: device upload of the seeded inputs, calls through the C ABI
binding, and the comparison rules against the oracle.

Comparison rules:
* packed codes, block scales and tensor scales: bit-exact;
* reconstructed W_eff: bit-exact;
* GEMV / small-M outputs (fp32 accumulation): the contract is relative L2 <= 1e-3 against the
  float64 oracle; the tests also hold every element to
  |y - y_ref| <= 2^-16 * sum_k |x_k w_k|, a bound far above fp32 summation error for any
  order (about K/64 + 20 roundings of 2^-24) yet below the contribution of a single dropped or
  mis-scaled 16-element block, and the vector to an internal relative L2 of 1e-5, taken against
  the larger of |y_ref| and 2^-10 |sum_k |x_k w_k|| (the scale of the rounding error).
"""
import sys

import numpy as np
import torch

import oracle as O

REL_L2_CONTRACT = 1e-3
REL_L2_INTERNAL = 1e-5
INTERNAL_FLOOR = 2.0 ** -10
ELEM_BOUND = 2.0 ** -16


def say(msg: str) -> None:
    """Name the case before a GPU step, unbuffered (a crash keeps the last line)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(a: np.ndarray | None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def gpu_quantize(A, bundles, K):
    """Quantize one or more theta bundles (one per segment) into one fused NVFP4 weight."""
    seg_end, n = [], 0
    for (W0, s, U, V) in bundles:
        n += W0.shape[0]
        seg_end.append(n)
    W = A.NVFP4Weight.empty(n, K, seg_end)
    keep = []
    for i, (W0, s, U, V) in enumerate(bundles):
        d = [dev(W0), dev(s), dev(U), dev(V)]
        keep.append(d)
        A.attnq_quantize_nvfp4(*d, W, seg=i)
    torch.cuda.synchronize()
    return W, seg_end


def oracle_quantize(bundles, rows=None):
    """Oracle codes/scales/ts for the fused weight (optionally only `rows` of the fused rows)."""
    codes, scales, ts, seg_end, n = [], [], [], [], 0
    for (W0, s, U, V) in bundles:
        We = O.reconstruct(W0, s, U, V)
        seg_rows = None
        if rows is not None:
            rows = np.asarray(rows)
            seg_rows = rows[(rows >= n) & (rows < n + W0.shape[0])] - n
        c, sc, t = O.quantize_segment(We, rows=seg_rows)
        codes.append(c); scales.append(sc); ts.append(t)
        n += W0.shape[0]
        seg_end.append(n)
    return np.concatenate(codes), np.concatenate(scales), np.array(ts, dtype=np.float32), seg_end


def assert_same_bits(a: np.ndarray, b: np.ndarray, what: str) -> None:
    if not np.array_equal(a.view(np.uint8) if a.dtype != np.uint8 else a, b.view(np.uint8) if b.dtype != np.uint8 else b):
        diff = np.argwhere(a != b)
        raise AssertionError(f"{what}: {len(diff)} mismatches, first at {diff[:5].tolist()}")


def assert_close_products(y: np.ndarray, y_ref: np.ndarray, absdot: np.ndarray, what: str) -> None:
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = ELEM_BOUND * absdot
    bad = np.argwhere(~(err <= bound))
    assert len(bad) == 0, f"{what}: {len(bad)} elements over the fp32 bound, first {bad[:5].tolist()} " \
                          f"err {err.ravel()[:1]} bound {bound.ravel()[:1]}"
    nref = np.linalg.norm(y_ref)
    rel = np.linalg.norm(y - y_ref) / nref if nref > 0 else np.linalg.norm(y - y_ref)
    assert rel <= REL_L2_CONTRACT, f"{what}: rel-L2 {rel} over the 1e-3 contract"
    # The internal gate is relative to the larger of |y_ref| and 2^-10 |sum_k |x_k w_k||: the rounding
    # error of any fp32 summation order scales with the latter, so a vector whose entries cancel
    # to 10^4 times below it (a single output row, say) is held to the arithmetic, not to its norm.
    floor = INTERNAL_FLOOR * np.linalg.norm(np.asarray(absdot, dtype=np.float64))
    rel_int = np.linalg.norm(y - y_ref) / max(nref, floor) if max(nref, floor) > 0 else np.linalg.norm(y - y_ref)
    assert rel_int <= REL_L2_INTERNAL, f"{what}: rel-L2 {rel_int} over the 1e-5 internal gate"
