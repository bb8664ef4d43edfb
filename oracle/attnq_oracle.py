"""CPU oracle for load-time NVFP4 weight-only RTN quantization and the decode GEMVs.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path (the HIP library and its Python binding) never does, and shares
no code, table or helper with it.

What it computes, and where each step is defined:

* Reconstruction ``W_eff = s*W0 + U*V^T`` -- AttnQuant landing page, "How it
  works" (each projection is a theta bundle: shared block W0, per-row scale s,
  low-rank pair U, V, rebuilt once at load); weightless "GPU and cache
  acceleration", "Architecture decisions / Precompute-outside" (the same sum
  written ``s*W0 + U@V.T``).
* NVFP4 round-to-nearest quantization -- "GPU acceleration", "NVFP4
  quantization" (packed uint8 weights plus float8 block scales, quantized once
  at load); landing page, "Results" (round-to-nearest, no calibration);
  "Throughput", "What quantization actually saves" (storage cost: four bits
  per element plus an E4M3 scale byte for every 16-element block, 0.5625
  B/element). The E2M1 value grid and the FP32 per-tensor scale are not
  printed on the pages; they are the NVFP4 format itself (E2M1 = 1 sign,
  2 exponent, 1 mantissa bit).
* The decode GEMV ``y = x * W_eff^T`` consuming fp4 directly -- "GPU
  acceleration", "Where GPU time goes" (weight-reading GEMVs, no dequant
  kernel) and "Throughput", "The NVFP4 MLP kernels are the least
  bandwidth-efficient on the step".
* The fused gate|up projection with its activation, ``h = act(gate) * up``
  rounded to bf16 as the input of the down projection -- weightless "GPU and
  cache acceleration", "Future work" (gate/up fusion on the Q/K/V pattern).
  The pages do not name the activation; GELU with the tanh approximation,
  SiLU and the identity are offered. Reading: the activation and product are
  evaluated in float64 on the float64 GEMV outputs and rounded once to bf16
  (PARITY PINNED by closed forms, odd-part identities, a library cross-check
  and a hand-built two-segment weight whose gate/up pairing is checked, in
  tests/test_oracle_glu.py).
* The runtime low-rank product over a shared NVFP4 block, ``y = s * (x .
  deq(W0)^T) + U (V_g^T x)`` with the weight never rebuilt -- "Throughput",
  "The runtime reconstruction path does not reach dense parity" (W0 and the
  low-rank delta applied on every forward pass); weightless "GPU and cache
  acceleration", "Custom-op kernel" (the W0 dot product and the low-rank
  delta fused) and "Future work / Trained weight sharing" (a shared NVFP4 W0
  plus a bf16 low-rank pair). Each segment of a fused weight is one
  projection with its own factors (PARITY PINNED by exact rational sums and
  mutations in tests/test_oracle_lowrank.py and test_oracle_mutations.py).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* theta tensors and W_eff are bf16; reconstruction accumulates in fp32 with
  ``acc = 0; acc += U[i,k]*V[j,k]`` for k ascending, then ``s_i*W0[i,j] + acc``
  rounded once to fp32 and once to bf16; with r == 0 the add is skipped.
  bf16 x bf16 products are exact in fp32, so a fused multiply-add gives the
  same bits. (PARITY PINNED: this sequence is checked element by element
  against exact rational arithmetic with explicit IEEE rounding steps on
  bundles where the order decides the result, and by a hand-derived example,
  in tests/test_oracle_reconstruct_order.py.)
* quantization starts from the bf16 W_eff (also when reconstruction is fused).
* tensor scale ``ts = fl32(amax / 2688)`` (2688 = 6 * 448, the E2M1 maximum
  times the E4M3 maximum), one per projection ("segment"), stored as the
  dequantization multiplier.
* block scale ``S = e4m3_rne_satfinite(fl32(bamax / fl32(6*ts)))``; element
  ``q = fl32(w / fl32(e4m3(S)*ts))`` rounded to the E2M1 grid with ties to the
  even code, saturating at 6; sign copied from w; S == 0 forces magnitude 0.
* blocks run along K (16 consecutive elements of a row); two codes per byte,
  the even element in the low nibble.
* a segment whose amax is not finite gets ts = NaN, every block scale 0x7F
  (the E4M3 NaN code) and every code byte 0.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# format constants (NVFP4 = E2M1 elements, E4M3FN block scales, FP32 tensor scale)
# ---------------------------------------------------------------------------
BLOCK = 16                       # elements per block scale ("per 16 elements")
E2M1_MAX = 6.0
E4M3_MAX = 448.0
TS_DIVISOR = np.float32(E2M1_MAX * E4M3_MAX)   # 2688
E4M3_NAN_CODE = 0x7F

# E2M1 magnitude for each 3-bit code: exponent bias 1, one mantissa bit, code 1 subnormal.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# ---------------------------------------------------------------------------
# bf16 <-> fp32
# ---------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32: bf16 is the top half of an fp32 word."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round-to-nearest-even on the 16 dropped bits; NaN stays a quiet NaN."""
    a = np.asarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    upper = bits >> np.uint64(16)
    lower = bits & np.uint64(0xFFFF)
    # round up when the dropped half is above the midpoint, or exactly at it with an odd kept LSB
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & np.uint64(1)) == 1))
    out = (upper + round_up.astype(np.uint64)) & np.uint64(0xFFFF)
    nan = np.isnan(a)
    out = np.where(nan, upper | np.uint64(0x0040), out)
    return out.astype(np.uint16)


def f64_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits with one round-to-nearest-even step. The float32 intermediate is
    rounded to odd (truncate toward zero, then set the last bit if anything was dropped), which
    keeps the second rounding exact because float32 carries 16 more bits than bf16."""
    a = np.asarray(a, dtype=np.float64)
    t = a.astype(np.float32)
    away = np.abs(t.astype(np.float64)) > np.abs(a)
    t = np.where(away, np.nextafter(t, np.float32(0)), t).astype(np.float32)
    inexact = t.astype(np.float64) != a
    bits = t.view(np.uint32) | np.where(inexact & np.isfinite(a), np.uint32(1), np.uint32(0))
    return f32_to_bf16_rne(bits.astype(np.uint32).view(np.float32))


# ---------------------------------------------------------------------------
# E4M3FN (OCP 8-bit float: bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN)
# ---------------------------------------------------------------------------
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes -> float64 values (exact)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    sub = m * 2.0 ** -9
    v = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode_rne_satfinite(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3FN code, round to nearest with ties to the even code, saturating to +-448.

    Works on the exact value of each fp32 input (float64 holds it exactly):
    below 2^-6 the grid step is 2^-9 (subnormals); in the binade [2^e, 2^(e+1))
    it is 2^(e-3). Values at or past 448 saturate to 448 (code 0x7E).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    sign = np.signbit(x).astype(np.uint8) << 7
    ax = np.abs(x)
    nan = np.isnan(ax)
    sat = (~nan) & (ax >= E4M3_MAX)
    rest = (~nan) & (~sat)

    sub = rest & (ax < 2.0 ** -6)
    q_sub = np.rint(np.where(sub, ax, 0.0) * 2.0 ** 9)   # rint: half to even; code == q for subnormals
    norm = rest & (ax >= 2.0 ** -6)
    _, ex = np.frexp(np.where(norm, ax, 1.0))   # ax = f * 2^ex, f in [0.5, 1)
    ue = ex - 1                                 # ax in [2^ue, 2^(ue+1))
    q = np.rint(np.where(norm, ax, 1.0) / np.exp2(ue - 3.0))   # in [8, 16]; even q <=> even code
    carry = q >= 16
    ue = np.where(carry, ue + 1, ue)
    mant = np.where(carry, 0, q - 8).astype(np.int64)
    code_norm = ((ue + 7) << 3) | mant

    out = np.where(sub, q_sub.astype(np.int64), out)
    out = np.where(norm, code_norm, out)
    out = np.where(sat, 0x7E, out)
    out = np.where(nan, E4M3_NAN_CODE, out)
    return (out.astype(np.uint8) | np.where(nan, 0, sign).astype(np.uint8))


# ---------------------------------------------------------------------------
# E2M1 (NVFP4 element: 1 sign, 2 exponent, 1 mantissa bit)
# ---------------------------------------------------------------------------
def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_encode_magnitude(aq: np.ndarray) -> np.ndarray:
    """|q| (float32, >= 0) -> 3-bit magnitude code, nearest grid value, ties to the even code.

    Grid 0, 0.5, 1, 1.5, 2, 3, 4, 6; the midpoints 0.25, 1.25, 2.5, 5 tie down
    to an even code, 0.75, 1.75, 3.5 tie up to an even code; above 5 saturates
    to 6 (code 7). A NaN quotient can only come from 0/0 (a zero weight in a block whose step
    d underflowed to zero) and encodes as 0.
    """
    a = np.asarray(aq, dtype=np.float32)
    conds = [np.isnan(a), a <= 0.25, a < 0.75, a <= 1.25, a < 1.75, a <= 2.5, a < 3.5, a <= 5.0]
    return np.select(conds, [0, 0, 1, 2, 3, 4, 5, 6], default=7).astype(np.uint8)


# ---------------------------------------------------------------------------
# reconstruction (landing page "How it works"; weightless "Precompute-outside")
# ---------------------------------------------------------------------------
def reconstruct(W0: np.ndarray, s: np.ndarray | None = None, U: np.ndarray | None = None,
                V: np.ndarray | None = None) -> np.ndarray:
    """W_eff = s*W0 + U V^T as bf16 bits; all inputs are bf16 bit arrays.

    W0 [N, K], s [N] (None means 1), U [N, r], V [K, r] (None means r = 0).
    """
    w0 = bf16_to_f32(W0)
    N, K = w0.shape
    sv = np.ones(N, dtype=np.float32) if s is None else bf16_to_f32(s)
    base = sv[:, None] * w0                       # exact: 8-bit x 8-bit significands
    r = 0 if U is None else U.shape[1]
    if r == 0:
        return f32_to_bf16_rne(base)
    u = bf16_to_f32(U)
    v = bf16_to_f32(V)
    assert u.shape == (N, r) and v.shape == (K, r)
    acc = np.zeros((N, K), dtype=np.float32)
    for k in range(r):                            # k ascending, one fp32 rounding per step
        acc = acc + u[:, k][:, None] * v[:, k][None, :]
    return f32_to_bf16_rne(base + acc)


# ---------------------------------------------------------------------------
# NVFP4 RTN quantization ("NVFP4 quantization"; "What quantization actually saves")
# ---------------------------------------------------------------------------
def quantize_segment(W_eff: np.ndarray, rows=None):
    """One projection (segment): bf16 bits [n, K] -> (codes u8 [n, K/2], scales u8 [n, K/16], ts f32).

    rows: optional row indices; the amax is still taken over the whole segment, but codes and
    scales are returned for those rows only (for sampled checks of large weights).
    """
    W_eff = np.asarray(W_eff)
    n_all, K = W_eff.shape
    assert K % BLOCK == 0
    if n_all == 0:
        return np.zeros((0, K // 2), np.uint8), np.zeros((0, K // BLOCK), np.uint8), np.float32(0.0)
    amax = np.float32(np.abs(bf16_to_f32(W_eff)).max())   # exact; NaN propagates
    w = bf16_to_f32(W_eff if rows is None else W_eff[np.asarray(rows)])
    n = w.shape[0]
    absw = np.abs(w)
    codes = np.zeros((n, K // 2), dtype=np.uint8)
    if not np.isfinite(amax):
        scales = np.full((n, K // BLOCK), E4M3_NAN_CODE, dtype=np.uint8)
        return codes, scales, np.float32(np.nan)

    ts = np.float32(amax / TS_DIVISOR)                     # fp32 division, RNE
    six_ts = np.float32(np.float32(E2M1_MAX) * ts)
    bamax = absw.reshape(n, K // BLOCK, BLOCK).max(axis=2)
    if amax == 0:
        sb = np.zeros_like(bamax)
    else:
        with np.errstate(divide="ignore", over="ignore"):
            sb = (bamax / six_ts).astype(np.float32)
    S = e4m3_encode_rne_satfinite(sb)
    d = (e4m3_decode(S).astype(np.float32) * ts).astype(np.float32)   # e4m3 value is exact in fp32
    d_el = np.repeat(d, BLOCK, axis=1)
    zero_scale = np.repeat(S == 0, BLOCK, axis=1)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (w / np.where(zero_scale, np.float32(1.0), d_el)).astype(np.float32)
    mag = np.where(zero_scale, 0, e2m1_encode_magnitude(np.abs(q))).astype(np.uint8)
    code = (np.signbit(w).astype(np.uint8) << 3) | mag
    codes[:] = code[:, 0::2] | (code[:, 1::2] << 4)
    return codes, S, ts


def quantize(W_eff: np.ndarray, seg_end=None):
    """Quantize a (possibly fused) [N, K] bf16 weight whose rows split into segments.

    seg_end: exclusive, ascending row ends, last == N (None = one segment).
    Returns codes [N, K/2] u8, scales [N, K/16] u8, tensor_scale [n_seg] f32.
    """
    N, K = W_eff.shape
    seg_end = [N] if seg_end is None else list(seg_end)
    codes = np.zeros((N, K // 2), dtype=np.uint8)
    scales = np.zeros((N, K // BLOCK), dtype=np.uint8)
    ts = np.zeros(len(seg_end), dtype=np.float32)
    start = 0
    for i, end in enumerate(seg_end):
        c, s, t = quantize_segment(W_eff[start:end])
        codes[start:end], scales[start:end], ts[i] = c, s, t
        start = end
    return codes, scales, ts


def packed_bytes(N: int, K: int, n_seg: int = 1) -> int:
    """Storage of one NVFP4 weight: K/2 code bytes + K/16 scale bytes per row, 4 B per tensor scale."""
    return N * K // 2 + N * K // BLOCK + 4 * n_seg


# ---------------------------------------------------------------------------
# dequantization and the decode products (fp64 reference)
# ---------------------------------------------------------------------------
def unpack_codes(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = c & 0x0F
    out[..., 1::2] = c >> 4
    return out


def row_segment_scale(N: int, seg_end, ts: np.ndarray) -> np.ndarray:
    """Per-row tensor scale for a fused weight (row i takes the scale of its segment)."""
    seg_end = [N] if seg_end is None else list(seg_end)
    out = np.empty(N, dtype=np.float64)
    start = 0
    for i, end in enumerate(seg_end):
        out[start:end] = np.float64(ts[i])
        start = end
    return out


def dequantize(codes, scales, ts, seg_end=None, rows=None) -> np.ndarray:
    """Exact dequantized weights in float64: e2m1(code) * e4m3(S) * ts (at most 30 significant bits)."""
    codes = np.asarray(codes)
    N = codes.shape[0]
    rts = row_segment_scale(N, seg_end, np.asarray(ts))
    if rows is not None:
        codes, scales, rts = codes[rows], np.asarray(scales)[rows], rts[rows]
    el = e2m1_decode(unpack_codes(codes))
    sc = np.repeat(e4m3_decode(scales), BLOCK, axis=-1)
    return el * sc * rts[:, None]


def dequantize_f32(codes, scales, ts, seg_end=None) -> np.ndarray:
    """fp32 dequantization fl32(fl32(e2m1*e4m3) * ts); the inner product is exact in fp32."""
    codes = np.asarray(codes)
    N = codes.shape[0]
    rts = row_segment_scale(N, seg_end, np.asarray(ts)).astype(np.float32)
    el = e2m1_decode(unpack_codes(codes)).astype(np.float32)
    sc = np.repeat(e4m3_decode(scales).astype(np.float32), BLOCK, axis=-1)
    return ((el * sc).astype(np.float32) * rts[:, None]).astype(np.float32)


def gemv_nvfp4(codes, scales, ts, x_bf16, seg_end=None, rows=None, chunk_rows=4096) -> np.ndarray:
    """y[n] = sum_k x[k] * deq[n, k], accumulated in float64 (every product is exact in fp64)."""
    x = bf16_to_f32(x_bf16).astype(np.float64).reshape(-1)
    codes = np.asarray(codes)
    idx = np.arange(codes.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty(len(idx), dtype=np.float64)
    for a in range(0, len(idx), chunk_rows):
        sel = idx[a:a + chunk_rows]
        out[a:a + len(sel)] = dequantize(codes, scales, ts, seg_end, rows=sel) @ x
    return out


def gemm_nvfp4_small_m(codes, scales, ts, X_bf16, seg_end=None, rows=None, chunk_rows=4096) -> np.ndarray:
    """Y[m, n] = sum_k X[m, k] * deq[n, k] in float64; each row m is the GEMV of X[m]."""
    X = bf16_to_f32(X_bf16).astype(np.float64)
    codes = np.asarray(codes)
    idx = np.arange(codes.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((X.shape[0], len(idx)), dtype=np.float64)
    for a in range(0, len(idx), chunk_rows):
        sel = idx[a:a + chunk_rows]
        out[:, a:a + len(sel)] = X @ dequantize(codes, scales, ts, seg_end, rows=sel).T
    return out


def gemv_bf16(W_bf16, x_bf16, rows=None, chunk_rows=8192) -> np.ndarray:
    """y[n] = sum_k x[k] * W[n, k] in float64 (tied bf16 lm_head)."""
    x = bf16_to_f32(x_bf16).astype(np.float64).reshape(-1)
    W = np.asarray(W_bf16)
    idx = np.arange(W.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty(len(idx), dtype=np.float64)
    for a in range(0, len(idx), chunk_rows):
        sel = idx[a:a + chunk_rows]
        out[a:a + len(sel)] = bf16_to_f32(W[sel]).astype(np.float64) @ x
    return out


def abs_dot(codes, scales, ts, X_bf16, seg_end=None, rows=None) -> np.ndarray:
    """sum_k |X[m,k] * deq[n,k]|: the scale of the fp32 rounding error of any summation order."""
    X = np.abs(bf16_to_f32(X_bf16).astype(np.float64)).reshape(-1, np.asarray(codes).shape[1] * 2)
    D = np.abs(dequantize(codes, scales, ts, seg_end, rows=rows))
    return X @ D.T


def abs_dot_bf16(W_bf16, x_bf16, rows=None) -> np.ndarray:
    x = np.abs(bf16_to_f32(x_bf16).astype(np.float64)).reshape(-1)
    W = np.asarray(W_bf16) if rows is None else np.asarray(W_bf16)[rows]
    return np.abs(bf16_to_f32(W).astype(np.float64)) @ x


# ---------------------------------------------------------------------------
# gate|up epilogue: h = act(gate) * up, the input of the down projection
# ---------------------------------------------------------------------------
ACT_GELU_TANH, ACT_SILU, ACT_IDENTITY = 0, 1, 2


def activation(g: np.ndarray, act: int) -> np.ndarray:
    """The epilogue activation in float64: GELU with the tanh approximation
    0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))), SiLU g / (1 + exp(-g)), or the identity."""
    g = np.asarray(g, dtype=np.float64)
    if act == ACT_GELU_TANH:
        return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))
    if act == ACT_SILU:
        return g / (1.0 + np.exp(-g))
    if act == ACT_IDENTITY:
        return g
    raise ValueError(f"unknown activation {act}")


def glu(y_gate: np.ndarray, y_up: np.ndarray, act: int) -> np.ndarray:
    """h[j] = bf16(act(gate[j]) * up[j]): float64 arithmetic, one rounding to bf16 (bits)."""
    return f64_to_bf16_rne(activation(y_gate, act) * np.asarray(y_up, dtype=np.float64))


def gemv_nvfp4_glu(codes, scales, ts, x_bf16, rows=None) -> np.ndarray:
    """The fused gate|up projection of a two-segment weight [gate; up] (F rows each) followed by
    the epilogue: returns (gate, up) float64 GEMV outputs for the pair rows `rows` (default all)."""
    N = np.asarray(codes).shape[0]
    F = N // 2
    j = np.arange(F) if rows is None else np.asarray(rows)
    seg_end = [F, N]
    g = gemv_nvfp4(codes, scales, ts, x_bf16, seg_end, rows=j)
    u = gemv_nvfp4(codes, scales, ts, x_bf16, seg_end, rows=j + F)
    return g, u


# ---------------------------------------------------------------------------
# runtime low-rank product over a shared NVFP4 block
# ---------------------------------------------------------------------------
def gemv_nvfp4_lowrank(codes, scales, ts, s_bf16, U_bf16, V_bf16, x_bf16, seg_end=None, rows=None) -> np.ndarray:
    """y = s * (x . deq(W0)^T) + U (V_g^T x) in float64 for a row of segment g, never rebuilding the
    weight ("Throughput", the runtime reconstruction path; weightless "Custom-op kernel" and
    "Trained weight sharing"). Each segment is one projection with its own factors.
    s is bf16 bits [N] or None (s = 1); U [N, r] and V [n_seg, K, r] (or [K, r] for one segment)
    bf16 bits, or None (r = 0)."""
    N = np.asarray(codes).shape[0]
    idx = np.arange(N) if rows is None else np.asarray(rows)
    y = gemv_nvfp4(codes, scales, ts, x_bf16, seg_end, rows=idx)
    if s_bf16 is not None:
        y = y * bf16_to_f32(np.asarray(s_bf16)[idx]).astype(np.float64)
    if U_bf16 is not None and np.asarray(U_bf16).shape[1] > 0:
        x = bf16_to_f32(x_bf16).astype(np.float64).reshape(-1)
        V = bf16_to_f32(np.asarray(V_bf16)).astype(np.float64)
        V = V.reshape((-1,) + V.shape[-2:])
        t = np.stack([V[g].T @ x for g in range(V.shape[0])])               # [n_seg, r]
        seg = row_segment_index(N, seg_end)[idx]
        U = bf16_to_f32(np.asarray(U_bf16)[idx]).astype(np.float64)
        y = y + np.sum(U * t[seg], axis=1)
    return y


def row_segment_index(N: int, seg_end) -> np.ndarray:
    """The segment each fused row belongs to."""
    ends = [N] if seg_end is None else list(seg_end)
    return np.searchsorted(np.asarray(ends), np.arange(N), side="right")


def abs_lowrank(s_bf16, U_bf16, V_bf16, x_bf16, absdot_w0, seg_end=None) -> np.ndarray:
    """|s| * sum_k |x_k w0_k| + sum_j |U_j| (sum_k |x_k V_g,kj|) for the rows of absdot_w0 (s, U and
    seg_end describe the same rows): the magnitude scale of the fp32 rounding error of the
    low-rank product, for any summation order."""
    out = np.asarray(absdot_w0, dtype=np.float64).copy()
    if s_bf16 is not None:
        out = out * np.abs(bf16_to_f32(np.asarray(s_bf16)).astype(np.float64))
    if U_bf16 is not None and np.asarray(U_bf16).shape[1] > 0:
        x = np.abs(bf16_to_f32(x_bf16).astype(np.float64)).reshape(-1)
        V = np.abs(bf16_to_f32(np.asarray(V_bf16)).astype(np.float64))
        V = V.reshape((-1,) + V.shape[-2:])
        t = np.stack([V[g].T @ x for g in range(V.shape[0])])
        seg = row_segment_index(len(out), seg_end)
        out = out + np.sum(np.abs(bf16_to_f32(np.asarray(U_bf16)).astype(np.float64)) * t[seg], axis=1)
    return out
