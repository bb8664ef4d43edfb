"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no reconstruction, no quantization, no dot products).
Both the HIP path and the CPU oracle consume what it produces, so neither
side can bias the other's inputs.

Recipe (the decode workloads the pages describe are Gemma 3 1B / Gemma 4 31B
projections; weights and activations here are synthetic stand-ins of the same
shapes):

* every tensor is drawn, in row-major order, in blocks of 2^20 elements; block b comes from
  ``numpy.random.PCG64`` seeded by ``SeedSequence([20261202, cfg, layer, proj, tensor, b])``
  (blocks are filled in parallel; the values do not depend on the thread count);
* values are drawn in float32, scaled, then rounded to bf16 by torch's
  float32 -> bfloat16 cast (round-to-nearest-even), and handed out as the raw
  uint16 bit patterns;
* W0 ~ N(0, 0.02^2), x ~ N(0, 1), s ~ U(0.9, 1.1), U, V ~ N(0, 1e-3^2).

For the full 31B-like token stream (24 G weight elements) host generation is
too slow for a benchmark run, so ``device_normal_bf16`` draws the same
distributions on the GPU with torch's own seeded generator. Those tensors are
only ever timed, never compared with the oracle.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

ROOT_SEED = 20261202

# tensor ids inside SeedSequence
T_W0, T_S, T_U, T_V, T_X = 0, 1, 2, 3, 4


GEN_BLOCK = 1 << 20
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _rng(cfg: int, layer: int, proj: int, tensor: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, cfg, layer, proj, tensor, block])))


def _draw(shape, fill, key) -> np.ndarray:
    """float32 array of `shape`; block b of the flat array is fill(generator_b, out_view)."""
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    nblk = (out.size + GEN_BLOCK - 1) // GEN_BLOCK

    def one(b):
        fill(_rng(*key, b), out[b * GEN_BLOCK:(b + 1) * GEN_BLOCK])
    if nblk <= 1:
        for b in range(nblk):
            one(b)
    else:
        list(_pool().map(one, range(nblk)))
    return out.reshape(shape)


def _to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns via torch's RNE cast (a library routine)."""
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, sigma: float, cfg: int, layer: int, proj: int, tensor: int) -> np.ndarray:
    def fill(g, o):
        g.standard_normal(out=o, dtype=np.float32)
        o *= np.float32(sigma)
    return _to_bf16_bits(_draw(shape, fill, (cfg, layer, proj, tensor)))


def uniform_bf16(shape, lo: float, hi: float, cfg: int, layer: int, proj: int, tensor: int) -> np.ndarray:
    def fill(g, o):
        o[:] = g.uniform(lo, hi, size=o.size)
    return _to_bf16_bits(_draw(shape, fill, (cfg, layer, proj, tensor)))


def theta_bundle(N: int, K: int, r: int, cfg: int, layer: int, proj: int,
                 passthrough: bool = False, w_sigma: float = 0.02, uv_sigma: float = 1e-3):
    """One projection's (W0, s, U, V) as bf16 bit arrays.

    passthrough=True gives s = None and r = 0 (the identity reconstruction).
    """
    W0 = normal_bf16((N, K), w_sigma, cfg, layer, proj, T_W0)
    if passthrough:
        return W0, None, None, None
    s = uniform_bf16((N,), 0.9, 1.1, cfg, layer, proj, T_S)
    if r == 0:
        return W0, s, None, None
    U = normal_bf16((N, r), uv_sigma, cfg, layer, proj, T_U)
    V = normal_bf16((K, r), uv_sigma, cfg, layer, proj, T_V)
    return W0, s, U, V


def activation_bf16(M: int, K: int, cfg: int, layer: int, proj: int) -> np.ndarray:
    """Decode-step activations, [M, K] (M = 1 for batch-1 decode)."""
    return normal_bf16((M, K), 1.0, cfg, layer, proj, T_X)


def bits_from_floats(values) -> np.ndarray:
    """Exact bf16 bit patterns for literal values that are bf16-representable (fixtures)."""
    a = np.asarray(values, dtype=np.float32)
    b = _to_bf16_bits(a)
    back = (b.astype(np.uint32) << 16).view(np.float32)
    if not np.array_equal(back.view(np.uint32), a.view(np.uint32)):
        raise ValueError("literal is not exactly representable in bf16")
    return b


def device_normal_bf16(shape, sigma: float, seed: int, device) -> torch.Tensor:
    """bf16 tensor ~ N(0, sigma^2) drawn on `device` with torch's seeded generator."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(sigma)
    return t.to(torch.bfloat16)


def device_uniform_bf16(shape, lo: float, hi: float, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(hi - lo).add_(lo)
    return t.to(torch.bfloat16)
