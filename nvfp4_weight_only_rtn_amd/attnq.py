"""Thin ctypes binding of libattnq.so (include/attnq.h), same names as the C calls.

Argument marshalling only: tensors are turned into device pointers and sizes, the call is
made on the current HIP stream (or the one given), and a non-zero status raises AttnqError.
Every step of the computation runs in the library's HIP kernels. If libattnq.so has not been
built, importing this module fails: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattnq.so")
MAX_SEGMENTS = 4
MAX_BATCH = 8
LAYOUT_ROW_MAJOR = 0
ACT_GELU_TANH, ACT_SILU, ACT_IDENTITY = 0, 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m nvfp4_weight_only_rtn_amd.build` "
                      "(or __graft_entry__.build()) before using the attnq binding")

_lib = ctypes.CDLL(LIB_PATH)


class _Theta(ctypes.Structure):
    _fields_ = [("W0", ctypes.c_void_p), ("s", ctypes.c_void_p), ("U", ctypes.c_void_p), ("V", ctypes.c_void_p),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("r", ctypes.c_int32)]


class _NVFP4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("n_seg", ctypes.c_int32),
                ("seg_end", ctypes.c_int32 * MAX_SEGMENTS), ("layout", ctypes.c_int32)]


_S = ctypes.c_int
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "attnq_reconstruct": [ctypes.POINTER(_Theta), _P, _P],
    "attnq_quantize_nvfp4": [ctypes.POINTER(_Theta), ctypes.POINTER(_NVFP4), _I, _P],
    "attnq_quantize_nvfp4_staged": [ctypes.POINTER(_Theta), ctypes.POINTER(_NVFP4), _I, _P, ctypes.c_int64, _P],
    "attnq_quantize_nvfp4_staged_batch": [ctypes.POINTER(_Theta), ctypes.POINTER(_NVFP4), ctypes.POINTER(_I), _I, _P,
                                          ctypes.c_int64, _P],
    "attnq_gemv_nvfp4": [ctypes.POINTER(_NVFP4), _P, _P, _P],
    "attnq_gemv_nvfp4_splitk": [ctypes.POINTER(_NVFP4), _P, _P, _P, ctypes.c_int64, _P],
    "attnq_gemv_nvfp4_splitk_noalloc": [ctypes.POINTER(_NVFP4), _P, _P, _P],
    "attnq_gemv_nvfp4_glu": [ctypes.POINTER(_NVFP4), _P, _I, _P, _P],
    "attnq_gemv_nvfp4_lowrank": [ctypes.POINTER(_NVFP4), _P, _P, _P, _I, _P, _P, _P, _P],
    "attnq_gemv_nvfp4_lowrank_splitk": [ctypes.POINTER(_NVFP4), _P, _P, _P, _I, _P, _P, _P, ctypes.c_int64, _P, _P],
    "attnq_gemv_bf16": [_P, _I, _I, _P, _P, _P],
    "attnq_gemm_nvfp4_small_m": [ctypes.POINTER(_NVFP4), _P, _I, _I, _P, _I, _P],
    "attnq_read_ceiling": [_P, ctypes.c_int64, _P, ctypes.c_int64, _P, _P],
    "attnq_gemm_nvfp4_small_m_splitk": [ctypes.POINTER(_NVFP4), _P, _I, _I, _P, _I, _P, ctypes.c_int64, _P],
}
for _name, _args in _SIGS.items():
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = _S
_lib.attnq_gemv_nvfp4_lowrank_workspace.argtypes = [_I, _I, _I]
_lib.attnq_gemv_nvfp4_lowrank_workspace.restype = ctypes.c_int64
_lib.attnq_quantize_nvfp4_staged_workspace.argtypes = [_I, _I, _I]
_lib.attnq_quantize_nvfp4_staged_workspace.restype = ctypes.c_int64
_lib.attnq_quantize_nvfp4_staged_batch_workspace.argtypes = [ctypes.POINTER(_Theta), _I]
_lib.attnq_quantize_nvfp4_staged_batch_workspace.restype = ctypes.c_int64
_lib.attnq_gemv_nvfp4_splitk_workspace.argtypes = [_I, _I]
_lib.attnq_gemv_nvfp4_splitk_workspace.restype = ctypes.c_int64
_lib.attnq_gemm_nvfp4_small_m_splitk_workspace.argtypes = [_I, _I, _I]
_lib.attnq_gemm_nvfp4_small_m_splitk_workspace.restype = ctypes.c_int64
_lib.attnq_status_string.argtypes = [_S]
_lib.attnq_status_string.restype = ctypes.c_char_p

STATUS = {0: "ATTNQ_OK", 1: "ATTNQ_ERR_NULL", 2: "ATTNQ_ERR_SHAPE", 3: "ATTNQ_ERR_ALIGN",
          4: "ATTNQ_ERR_SEGMENT", 5: "ATTNQ_ERR_LAYOUT", 6: "ATTNQ_ERR_HIP"}


class AttnqError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(_lib.attnq_status_string(status).decode())


def _check(status: int) -> None:
    if status != 0:
        raise AttnqError(status)


def _ptr(t: torch.Tensor | None, itemsize: int | None = None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("attnq expects contiguous tensors")
    if itemsize is not None and t.element_size() != itemsize:
        raise TypeError(f"expected {itemsize}-byte elements, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class NVFP4Weight:
    """Caller-owned device buffers of one NVFP4 weight (attnq_nvfp4): codes, scales, tensor scales."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, tensor_scale: torch.Tensor, seg_end):
        self.codes, self.scales, self.tensor_scale = codes, scales, tensor_scale
        self.seg_end = [int(v) for v in seg_end]
        self.N = codes.shape[0]
        self.K = codes.shape[1] * 2
        self._desc = _NVFP4(_ptr(codes, 1), _ptr(scales, 1), _ptr(tensor_scale, 4), self.N, self.K,
                            len(self.seg_end), (ctypes.c_int32 * MAX_SEGMENTS)(*(self.seg_end + [0] * (MAX_SEGMENTS - len(self.seg_end)))),
                            LAYOUT_ROW_MAJOR)

    @classmethod
    def empty(cls, N: int, K: int, seg_end=None, device="cuda") -> "NVFP4Weight":
        seg_end = [N] if seg_end is None else list(seg_end)
        return cls(torch.empty((N, K // 2), dtype=torch.uint8, device=device),
                   torch.empty((N, K // 16), dtype=torch.uint8, device=device),
                   torch.empty((len(seg_end),), dtype=torch.float32, device=device), seg_end)

    @property
    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel() + 4 * self.tensor_scale.numel()

    def desc(self) -> _NVFP4:
        return self._desc


def _theta(W0, s, U, V) -> _Theta:
    N, K = W0.shape
    r = 0 if U is None else U.shape[1]
    return _Theta(_ptr(W0, 2), _ptr(s, 2), _ptr(U, 2), _ptr(V, 2), N, K, r)


def attnq_reconstruct(W0, s, U, V, W_eff, stream=None) -> None:
    th = _theta(W0, s, U, V)
    _check(_lib.attnq_reconstruct(ctypes.byref(th), _ptr(W_eff, 2), _stream(stream)))


def attnq_quantize_nvfp4(W0, s, U, V, dst: NVFP4Weight, seg: int = 0, stream=None) -> None:
    th = _theta(W0, s, U, V)
    _check(_lib.attnq_quantize_nvfp4(ctypes.byref(th), ctypes.byref(dst.desc()), seg, _stream(stream)))


def attnq_quantize_nvfp4_staged_workspace(N: int, K: int, r: int) -> int:
    return int(_lib.attnq_quantize_nvfp4_staged_workspace(N, K, r))


def staged_workspace(N: int, K: int, r: int, device="cuda") -> torch.Tensor | None:
    """A workspace for attnq_quantize_nvfp4_staged on an [N][K] projection of rank r (None if not
    needed); torch's allocations are 256-byte aligned."""
    n = attnq_quantize_nvfp4_staged_workspace(N, K, r)
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def attnq_quantize_nvfp4_staged(W0, s, U, V, dst: NVFP4Weight, ws, seg: int = 0, stream=None) -> None:
    th = _theta(W0, s, U, V)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.attnq_quantize_nvfp4_staged(ctypes.byref(th), ctypes.byref(dst.desc()), seg, _ptr(ws), nbytes,
                                            _stream(stream)))


def _theta_array(bundles):
    return (_Theta * max(1, len(bundles)))(*[_theta(*b) for b in bundles])


def attnq_quantize_nvfp4_staged_batch_workspace(bundles) -> int:
    """bundles: (W0, s, U, V) tuples."""
    return int(_lib.attnq_quantize_nvfp4_staged_batch_workspace(_theta_array(bundles), len(bundles)))


def staged_batch_workspace(bundles, device="cuda") -> torch.Tensor | None:
    n = attnq_quantize_nvfp4_staged_batch_workspace(bundles)
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def attnq_quantize_nvfp4_staged_batch(bundles, dsts, segs, ws, stream=None) -> None:
    """bundles: (W0, s, U, V) tuples; bundle i goes into segment segs[i] of dsts[i]."""
    n = len(bundles)
    descs = (_NVFP4 * max(1, n))(*[d.desc() for d in dsts])
    seg_arr = (_I * max(1, n))(*segs)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.attnq_quantize_nvfp4_staged_batch(_theta_array(bundles), descs, seg_arr, n, _ptr(ws), nbytes,
                                                  _stream(stream)))


def attnq_gemv_nvfp4(W: NVFP4Weight, x, y, stream=None) -> None:
    _check(_lib.attnq_gemv_nvfp4(ctypes.byref(W.desc()), _ptr(x, 2), _ptr(y, 4), _stream(stream)))


def attnq_gemv_nvfp4_splitk_workspace(N: int, K: int) -> int:
    return int(_lib.attnq_gemv_nvfp4_splitk_workspace(N, K))


def splitk_workspace(N: int, K: int, device="cuda") -> torch.Tensor | None:
    """A zero-filled workspace for attnq_gemv_nvfp4_splitk on [N][K] weights (None if not needed);
    torch's allocations are 256-byte aligned."""
    n = attnq_gemv_nvfp4_splitk_workspace(N, K)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n > 0 else None


def attnq_gemv_nvfp4_splitk(W: NVFP4Weight, x, y, ws, stream=None) -> None:
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.attnq_gemv_nvfp4_splitk(ctypes.byref(W.desc()), _ptr(x, 2), _ptr(y, 4), _ptr(ws), nbytes,
                                        _stream(stream)))


def attnq_gemv_nvfp4_splitk_noalloc(W: NVFP4Weight, x, y, stream=None) -> None:
    _check(_lib.attnq_gemv_nvfp4_splitk_noalloc(ctypes.byref(W.desc()), _ptr(x, 2), _ptr(y, 4), _stream(stream)))


def attnq_gemv_nvfp4_glu(W: NVFP4Weight, x, act: int, h, stream=None) -> None:
    _check(_lib.attnq_gemv_nvfp4_glu(ctypes.byref(W.desc()), _ptr(x, 2), act, _ptr(h, 2), _stream(stream)))


def attnq_gemv_nvfp4_lowrank_workspace(K: int, n_seg: int, r: int) -> int:
    return int(_lib.attnq_gemv_nvfp4_lowrank_workspace(K, n_seg, r))


def attnq_gemv_nvfp4_lowrank(W0: NVFP4Weight, s, U, V, x, ws, y, stream=None) -> None:
    r = 0 if U is None else U.shape[1]
    if r and (ws is None or ws.numel() < attnq_gemv_nvfp4_lowrank_workspace(W0.K, len(W0.seg_end), r)):
        raise ValueError("attnq_gemv_nvfp4_lowrank: workspace smaller than attnq_gemv_nvfp4_lowrank_workspace()")
    _check(_lib.attnq_gemv_nvfp4_lowrank(ctypes.byref(W0.desc()), _ptr(s, 2), _ptr(U, 2), _ptr(V, 2), r, _ptr(x, 2),
                                         _ptr(ws, 4), _ptr(y, 4), _stream(stream)))


def attnq_gemv_nvfp4_lowrank_splitk(W0: NVFP4Weight, s, U, V, x, ws, split_ws, y, stream=None) -> None:
    r = 0 if U is None else U.shape[1]
    if r and (ws is None or ws.numel() < attnq_gemv_nvfp4_lowrank_workspace(W0.K, len(W0.seg_end), r)):
        raise ValueError("attnq_gemv_nvfp4_lowrank_splitk: workspace smaller than attnq_gemv_nvfp4_lowrank_workspace()")
    nbytes = 0 if split_ws is None else split_ws.numel() * split_ws.element_size()
    _check(_lib.attnq_gemv_nvfp4_lowrank_splitk(ctypes.byref(W0.desc()), _ptr(s, 2), _ptr(U, 2), _ptr(V, 2), r,
                                                _ptr(x, 2), _ptr(ws, 4), _ptr(split_ws), nbytes, _ptr(y, 4),
                                                _stream(stream)))


def attnq_gemv_bf16(W, x, y, stream=None) -> None:
    N, K = W.shape
    _check(_lib.attnq_gemv_bf16(_ptr(W, 2), N, K, _ptr(x, 2), _ptr(y, 4), _stream(stream)))


def attnq_gemm_nvfp4_small_m(W: NVFP4Weight, X, Y, stream=None) -> None:
    M = X.shape[0]
    _check(_lib.attnq_gemm_nvfp4_small_m(ctypes.byref(W.desc()), _ptr(X, 2), M, X.stride(0) if M else W.K,
                                         _ptr(Y, 4), Y.stride(0) if M else W.N, _stream(stream)))


def attnq_read_ceiling(a, b, sink, stream=None) -> None:
    """Streaming read of tensors a and b (b may be None), nothing written: the read ceiling."""
    na = a.numel() * a.element_size()
    nb = 0 if b is None else b.numel() * b.element_size()
    _check(_lib.attnq_read_ceiling(_ptr(a), na, _ptr(b), nb, _ptr(sink, 4), _stream(stream)))


def attnq_gemm_nvfp4_small_m_splitk_workspace(N: int, K: int, M: int) -> int:
    return int(_lib.attnq_gemm_nvfp4_small_m_splitk_workspace(N, K, M))


def small_m_workspace(N: int, K: int, M: int, device="cuda") -> torch.Tensor | None:
    """A workspace for attnq_gemm_nvfp4_small_m_splitk (None if the shape needs none)."""
    n = attnq_gemm_nvfp4_small_m_splitk_workspace(N, K, M)
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def attnq_gemm_nvfp4_small_m_splitk(W: NVFP4Weight, X, Y, ws, stream=None) -> None:
    M = X.shape[0]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.attnq_gemm_nvfp4_small_m_splitk(ctypes.byref(W.desc()), _ptr(X, 2), M, X.stride(0) if M else W.K,
                                                _ptr(Y, 4), Y.stride(0) if M else W.N, _ptr(ws), nbytes,
                                                _stream(stream)))


def raw_library() -> ctypes.CDLL:
    """The loaded library object (for ABI tests that call entry points with raw arguments)."""
    return _lib
