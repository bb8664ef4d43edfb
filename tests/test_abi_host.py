"""Host-side checks of the C ABI: the library loads, exports every call include/attnq.h
declares, the ctypes descriptors match the C struct layout, and argument validation returns
the documented status codes. No call here reaches a kernel launch: every argument set fails
validation, which runs on the host before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnq.h")

A = pytest.importorskip("nvfp4_weight_only_rtn_amd.attnq", reason="libattnq.so not built")

# invalid-pointer calls are only made where no GPU can be reached by mistake
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="host-only validation test")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ATTNQ_API\s+[\w\s\*]+?\b(attnq_\w+)\s*\(", text)))


def test_header_declares_every_call():
    names = _declared_functions()
    for n in ["attnq_reconstruct", "attnq_quantize_nvfp4", "attnq_quantize_nvfp4_staged",
              "attnq_quantize_nvfp4_staged_workspace", "attnq_gemv_nvfp4", "attnq_gemv_bf16",
              "attnq_gemm_nvfp4_small_m", "attnq_gemv_nvfp4_glu", "attnq_gemv_nvfp4_lowrank",
              "attnq_gemv_nvfp4_lowrank_workspace", "attnq_gemv_nvfp4_lowrank_splitk", "attnq_gemv_nvfp4_splitk",
              "attnq_gemv_nvfp4_splitk_workspace", "attnq_gemv_nvfp4_splitk_noalloc", "attnq_read_ceiling",
              "attnq_gemm_nvfp4_small_m_splitk", "attnq_gemm_nvfp4_small_m_splitk_workspace", "attnq_status_string",
              "attnq_quantize_nvfp4_staged_batch", "attnq_quantize_nvfp4_staged_batch_workspace"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = A.raw_library()
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(attnq_\w+)", out))
    assert exported == set(_declared_functions())


def test_lowrank_workspace_sizes():
    ws = A.attnq_gemv_nvfp4_lowrank_workspace
    assert ws(5376, 1, 0) == 0
    assert ws(5376, 1, 16) == 6 * 16               # chunks of 1024 rows
    assert ws(21504, 1, 16) == 21 * 16
    assert ws(5376, 3, 64) == 3 * 21 * 64          # chunks of 256 rows
    assert ws(96, 2, 3) == 2 * 1 * 3               # 5461 rows per chunk
    assert ws(32, 1, 1) == 1
    for bad in [(0, 1, 4), (40, 1, 4), (64, 0, 4), (64, 5, 4), (64, 1, 65), (64, 1, -1)]:
        assert ws(*bad) == -1


def test_splitk_workspace_sizes():
    ws = A.attnq_gemv_nvfp4_splitk_workspace
    # rows under 16384 elements are not split
    assert ws(5376, 4096) == 0 and ws(43008, 5376) == 0 and ws(100, 16384 - 32) == 0
    # one 832-byte record (a ticket slot and 12 partial slots of 64 B) per tile of 16 rows, for every
    # split shape: down 5376 x 21504 (672 chunks -> 6 slices of 112) has 336 tiles
    assert ws(5376, 21504) == 336 * 832
    assert ws(1, 16384) == 832                         # 512 chunks -> 4 slices of 128
    assert ws(17, 24576) == 2 * 832                    # 768 chunks -> 6 slices of 128
    assert ws(100, 49152) == 7 * 832                   # 1536 chunks -> 12 slices of 128
    assert ws(100, 49152 + 32) == 0                    # would need 13 slices: not split
    assert ws(0, 21504) == 0
    for bad in [(-1, 21504), (64, 0), (64, 48)]:
        assert ws(*bad) == -1


def test_small_m_splitk_workspace_sizes():
    ws = A.attnq_gemm_nvfp4_small_m_splitk_workspace
    # fp32 partials [row group of 64][strip or slice][token][64 rows]
    # weights of at least 16384 rows walk whole strips of 32, 24 or 16 chunks:
    # gate|up 43008 x 5376 at M = 8: 672 groups, 168 chunks -> 7 strips of 24
    assert ws(43008, 5376, 8) == 672 * 7 * 8 * 64 * 4
    assert ws(43008, 5376, 3) == 672 * 7 * 3 * 64 * 4     # M = 3, 4 walk too on rows of up to 6144
    # 16384 x 4096 at M = 16: 256 groups, 128 chunks -> 4 strips of 32
    assert ws(16384, 4096, 16) == 256 * 4 * 16 * 64 * 4
    assert ws(16384, 1024, 8) == 0                     # one strip: Y stored directly
    assert ws(300000, 4096, 8) == 4688 * 4 * 8 * 64 * 4
    assert ws(16384, 512 * 3, 2) == 0                  # rows of up to 6144 at M <= 2: the batch-1 walk
    # rows that do not split into whole strips take the one-shot slices (two steps of 1024 elements
    # each at 4 < M <= 8 on weights of at least 16384 rows: 129 chunks -> 5 steps -> 3 slices)
    assert ws(16400, 4096 + 32, 7) == 257 * 3 * 7 * 64 * 4
    # narrower weights with long rows: down 5376 x 21504 at M = 4 takes the slices (84 groups, 21
    # slices), at M = 8 the walk (84 row groups, 21 strips of 32 chunks: the same partial count)
    assert ws(5376, 21504, 4) == 84 * 21 * 4 * 64 * 4
    assert ws(5376, 21504, 8) == 84 * 21 * 8 * 64 * 4
    assert ws(5376, 21504, 16) == 84 * 21 * 16 * 64 * 4
    assert ws(5376, 4096, 16) == 0                     # fewer rows and short rows: the older kernels
    assert ws(6144, 5376, 4) == 0                      # M <= 4 on rows of up to 6144: the batch-1 walk
    assert ws(0, 4096, 8) == 0 and ws(64, 4096, 0) == 0
    for bad in [(-1, 4096, 8), (64, 48, 8), (64, 4096, 17), (64, 4096, -1)]:
        assert ws(*bad) == -1


def test_status_strings():
    for code, name in A.STATUS.items():
        assert A.raw_library().attnq_status_string(code).decode().startswith(name)
    assert b"unknown" in A.raw_library().attnq_status_string(99)


def test_ctypes_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(f"""
#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(attnq_theta), offsetof(attnq_theta, W0),
         offsetof(attnq_theta, s), offsetof(attnq_theta, U), offsetof(attnq_theta, V),
         offsetof(attnq_theta, N), offsetof(attnq_theta, K), offsetof(attnq_theta, r));
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(attnq_nvfp4), offsetof(attnq_nvfp4, codes),
         offsetof(attnq_nvfp4, scales), offsetof(attnq_nvfp4, tensor_scale), offsetof(attnq_nvfp4, N),
         offsetof(attnq_nvfp4, K), offsetof(attnq_nvfp4, n_seg), offsetof(attnq_nvfp4, seg_end),
         offsetof(attnq_nvfp4, layout));
  return 0;
}}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(src), "-o", str(exe)], check=True)
    c_theta, c_nv = [list(map(int, l.split())) for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split("\n")[:2]]
    T, NV = A._Theta, A._NVFP4
    assert c_theta == [ctypes.sizeof(T)] + [getattr(T, f).offset for f in ("W0", "s", "U", "V", "N", "K", "r")]
    assert c_nv == [ctypes.sizeof(NV)] + [getattr(NV, f).offset for f in
                                           ("codes", "scales", "tensor_scale", "N", "K", "n_seg", "seg_end", "layout")]


# ---------------------------------------------------------------- validation (host only)
FAKE = 0x10000          # aligned, never dereferenced: every call below fails validation first


def _nv(N=64, K=64, n_seg=1, seg_end=None, layout=0, codes=FAKE, scales=FAKE, ts=FAKE):
    seg_end = [N] if seg_end is None else seg_end
    return A._NVFP4(codes, scales, ts, N, K, n_seg, (ctypes.c_int32 * 4)(*(seg_end + [0] * (4 - len(seg_end)))), layout)


def _th(N=64, K=64, r=0, W0=FAKE, s=None, U=None, V=None):
    return A._Theta(W0, s, U, V, N, K, r)


@no_gpu
def test_reconstruct_validation():
    lib = A.raw_library()
    assert lib.attnq_reconstruct(None, FAKE, None) == 1
    assert lib.attnq_reconstruct(ctypes.byref(_th(W0=None)), FAKE, None) == 1
    assert lib.attnq_reconstruct(ctypes.byref(_th()), None, None) == 1
    assert lib.attnq_reconstruct(ctypes.byref(_th(K=48)), FAKE, None) == 2       # K % 32 != 0
    assert lib.attnq_reconstruct(ctypes.byref(_th(K=0)), FAKE, None) == 2
    assert lib.attnq_reconstruct(ctypes.byref(_th(N=-1)), FAKE, None) == 2
    assert lib.attnq_reconstruct(ctypes.byref(_th(r=65, U=FAKE, V=FAKE)), FAKE, None) == 2
    assert lib.attnq_reconstruct(ctypes.byref(_th(r=4)), FAKE, None) == 1        # r > 0 needs U, V
    assert lib.attnq_reconstruct(ctypes.byref(_th(W0=FAKE + 2)), FAKE, None) == 3
    assert lib.attnq_reconstruct(ctypes.byref(_th()), FAKE + 8, None) == 3


@no_gpu
def test_quantize_validation():
    lib = A.raw_library()
    q = lib.attnq_quantize_nvfp4
    assert q(ctypes.byref(_th()), None, 0, None) == 1
    assert q(ctypes.byref(_th()), ctypes.byref(_nv(layout=1)), 0, None) == 5
    assert q(ctypes.byref(_th(K=96)), ctypes.byref(_nv()), 0, None) == 2          # K mismatch
    assert q(ctypes.byref(_th()), ctypes.byref(_nv()), 1, None) == 4              # seg out of range
    assert q(ctypes.byref(_th(N=10)), ctypes.byref(_nv()), 0, None) == 4          # row count mismatch
    nv = _nv(N=64, n_seg=3, seg_end=[32, 48, 64])
    assert q(ctypes.byref(_th(N=32)), ctypes.byref(nv), 1, None) == 4             # seg 1 has 16 rows
    assert q(ctypes.byref(_th()), ctypes.byref(_nv(n_seg=2, seg_end=[40, 30])), 0, None) == 4
    assert q(ctypes.byref(_th()), ctypes.byref(_nv(n_seg=2, seg_end=[32, 60])), 0, None) == 4
    assert q(ctypes.byref(_th()), ctypes.byref(_nv(n_seg=5)), 0, None) == 4
    assert q(ctypes.byref(_th()), ctypes.byref(_nv(codes=FAKE + 4)), 0, None) == 3
    assert q(ctypes.byref(_th()), ctypes.byref(_nv(scales=FAKE + 2)), 0, None) == 3


def test_quantize_staged_workspace_sizes():
    ws = A.attnq_quantize_nvfp4_staged_workspace
    assert ws(5376, 21504, 16) == 2 * 5376 * 21504           # bf16 W_eff of the whole projection
    assert ws(21504, 5376, 1) == 2 * 21504 * 5376
    assert ws(64, 64, 0) == 0                                # rank 0: nothing to rebuild
    assert ws(0, 64, 16) == 0 and ws(64, 0, 16) == 0


@no_gpu
def test_quantize_staged_validation():
    lib = A.raw_library()
    q = lib.attnq_quantize_nvfp4_staged
    need = A.attnq_quantize_nvfp4_staged_workspace(64, 64, 4)
    r4 = _th(r=4, U=FAKE, V=FAKE)
    assert q(ctypes.byref(r4), ctypes.byref(_nv()), 0, None, need, None) == 1     # r > 0 needs a workspace
    assert q(ctypes.byref(r4), ctypes.byref(_nv()), 0, FAKE, need - 1, None) == 2  # too small
    assert q(ctypes.byref(r4), ctypes.byref(_nv()), 0, FAKE + 16, need, None) == 3  # not 256-byte aligned
    assert q(ctypes.byref(_th(K=96, r=4, U=FAKE, V=FAKE)), ctypes.byref(_nv()), 0, FAKE, 1 << 20, None) == 2
    assert q(ctypes.byref(r4), ctypes.byref(_nv()), 1, FAKE, need, None) == 4      # seg out of range
    assert q(ctypes.byref(_th(r=4)), ctypes.byref(_nv()), 0, FAKE, need, None) == 1  # U, V missing
    assert q(None, ctypes.byref(_nv()), 0, FAKE, need, None) == 1


def _th_array(*ths):
    return (A._Theta * max(1, len(ths)))(*ths)


def test_quantize_staged_batch_workspace_sizes():
    ws = A.raw_library().attnq_quantize_nvfp4_staged_batch_workspace
    assert ws(_th_array(), 0) == 0
    # bundle i's W_eff at the sum of the earlier ones, each rounded up to 256 bytes
    ths = [_th(N=64, K=256, r=16, U=FAKE, V=FAKE), _th(N=3, K=32, r=4, U=FAKE, V=FAKE), _th(N=64, K=64, r=0),
           _th(N=5376, K=21504, r=16, U=FAKE, V=FAKE)]
    assert ws(_th_array(*ths), 4) == 2 * 64 * 256 + 256 + 0 + 2 * 5376 * 21504
    assert ws(_th_array(*ths[2:3]), 1) == 0
    assert ws(_th_array(*([ths[0]] * 8)), 8) == 8 * 2 * 64 * 256
    assert ws(_th_array(*([ths[0]] * 9)), 9) == -1           # at most ATTNQ_MAX_BATCH bundles
    assert ws(None, 2) == -1 and ws(_th_array(), -1) == -1


@no_gpu
def test_quantize_staged_batch_validation():
    lib = A.raw_library()
    q = lib.attnq_quantize_nvfp4_staged_batch
    r4 = _th(r=4, U=FAKE, V=FAKE)
    need = A.attnq_quantize_nvfp4_staged_workspace(64, 64, 4)
    segs2 = (ctypes.c_int32 * 2)(0, 1)
    fused = _nv(N=128, n_seg=2, seg_end=[64, 128])
    two = (A._NVFP4 * 2)(fused, fused)
    ths = _th_array(r4, r4)
    assert q(ths, two, segs2, 0, None, 0, None) == 0                      # nothing to do
    assert q(ths, two, segs2, 9, FAKE, 1 << 30, None) == 2                 # count above ATTNQ_MAX_BATCH
    assert q(ths, two, segs2, -1, FAKE, 1 << 30, None) == 2
    assert q(None, two, segs2, 2, FAKE, 1 << 30, None) == 1
    assert q(ths, None, segs2, 2, FAKE, 1 << 30, None) == 1
    assert q(ths, two, None, 2, FAKE, 1 << 30, None) == 1
    assert q(ths, two, (ctypes.c_int32 * 2)(0, 0), 2, FAKE, 1 << 30, None) == 4   # one segment named twice
    assert q(ths, two, (ctypes.c_int32 * 2)(0, 2), 2, FAKE, 1 << 30, None) == 4   # seg out of range
    assert q(ths, two, segs2, 2, None, 2 * need, None) == 1                # rank > 0 needs a workspace
    assert q(ths, two, segs2, 2, FAKE, 2 * need - 1, None) == 2            # too small
    assert q(ths, two, segs2, 2, FAKE + 16, 2 * need, None) == 3           # not 256-byte aligned
    assert q(_th_array(r4, _th(r=4)), two, segs2, 2, FAKE, 1 << 30, None) == 1    # second bundle lacks U, V
    assert q(_th_array(r4, _th(N=32, r=4, U=FAKE, V=FAKE)), two, segs2, 2, FAKE, 1 << 30, None) == 4  # row count


@no_gpu
def test_gemv_and_gemm_validation():
    lib = A.raw_library()
    nv = _nv()
    assert lib.attnq_gemv_nvfp4(ctypes.byref(nv), None, FAKE, None) == 1
    assert lib.attnq_gemv_nvfp4(ctypes.byref(nv), FAKE + 8, FAKE, None) == 3
    assert lib.attnq_gemv_nvfp4(ctypes.byref(nv), FAKE, FAKE + 2, None) == 3
    assert lib.attnq_gemv_nvfp4(ctypes.byref(_nv(K=16)), FAKE, FAKE, None) == 2
    big = _nv(N=1 << 20, K=8192 + 64)                                             # N * K/2 > 2^32 code bytes
    assert lib.attnq_gemv_nvfp4(ctypes.byref(big), FAKE, FAKE, None) == 2
    assert lib.attnq_gemm_nvfp4_small_m(ctypes.byref(big), FAKE, 4, 8192 + 64, FAKE, 1 << 20, None) == 2
    assert lib.attnq_quantize_nvfp4(ctypes.byref(_th(N=1 << 20, K=8192 + 64)), ctypes.byref(big), 0, None) == 2
    assert lib.attnq_gemv_bf16(FAKE, 10, 40, FAKE, FAKE, None) == 2
    assert lib.attnq_gemv_bf16(FAKE, -1, 64, FAKE, FAKE, None) == 2
    assert lib.attnq_gemv_bf16(None, 10, 64, FAKE, FAKE, None) == 1
    assert lib.attnq_gemv_bf16(FAKE + 4, 10, 64, FAKE, FAKE, None) == 3
    glu = lib.attnq_gemv_nvfp4_glu
    pair = _nv(N=64, n_seg=2, seg_end=[32, 64])
    assert glu(ctypes.byref(nv), FAKE, 0, FAKE, None) == 4                        # one segment
    assert glu(ctypes.byref(_nv(N=64, n_seg=2, seg_end=[16, 64])), FAKE, 0, FAKE, None) == 4  # unequal halves
    assert glu(ctypes.byref(pair), FAKE, 3, FAKE, None) == 2                      # unknown activation
    assert glu(ctypes.byref(pair), FAKE, -1, FAKE, None) == 2
    assert glu(ctypes.byref(pair), None, 0, FAKE, None) == 1
    assert glu(ctypes.byref(pair), FAKE, 0, None, None) == 1
    assert glu(ctypes.byref(pair), FAKE + 8, 0, FAKE, None) == 3
    assert glu(ctypes.byref(pair), FAKE, 1, FAKE + 1, None) == 3                  # h needs 2-byte alignment
    lr = lib.attnq_gemv_nvfp4_lowrank
    assert lr(ctypes.byref(nv), FAKE, FAKE, FAKE, 65, FAKE, FAKE, FAKE, None) == 2       # r > 64
    assert lr(ctypes.byref(nv), FAKE, FAKE, FAKE, -1, FAKE, FAKE, FAKE, None) == 2
    assert lr(ctypes.byref(nv), FAKE, None, FAKE, 4, FAKE, FAKE, FAKE, None) == 1        # U missing
    assert lr(ctypes.byref(nv), FAKE, FAKE, None, 4, FAKE, FAKE, FAKE, None) == 1        # V missing
    assert lr(ctypes.byref(nv), FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, None) == 1        # t missing
    assert lr(ctypes.byref(nv), FAKE, FAKE, FAKE, 4, None, FAKE, FAKE, None) == 1        # x missing
    assert lr(ctypes.byref(nv), FAKE, FAKE, FAKE, 4, FAKE, FAKE, None, None) == 1        # y missing
    assert lr(ctypes.byref(nv), FAKE, FAKE, FAKE, 4, FAKE + 8, FAKE, FAKE, None) == 3    # x 16-byte
    assert lr(ctypes.byref(nv), FAKE, FAKE, FAKE, 4, FAKE, FAKE + 2, FAKE, None) == 3    # t 4-byte
    assert lr(ctypes.byref(nv), FAKE + 1, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None) == 3    # s 2-byte
    assert lr(ctypes.byref(nv), FAKE, FAKE + 1, FAKE, 4, FAKE, FAKE, FAKE, None) == 3    # U 2-byte
    assert lr(ctypes.byref(nv), FAKE, FAKE, FAKE + 8, 4, FAKE, FAKE, FAKE, None) == 3    # V 16-byte
    assert lr(ctypes.byref(_nv(K=16)), FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None) == 2
    sk = lib.attnq_gemv_nvfp4_splitk
    down = _nv(N=64, K=21504)
    need = A.attnq_gemv_nvfp4_splitk_workspace(64, 21504)
    assert sk(ctypes.byref(down), FAKE, FAKE, None, need, None) == 1             # workspace needed
    assert sk(ctypes.byref(down), FAKE, FAKE, FAKE, need - 1, None) == 2         # too small
    assert sk(ctypes.byref(down), FAKE, FAKE, FAKE + 128, need, None) == 3       # 256-byte alignment
    assert sk(ctypes.byref(down), None, FAKE, FAKE, need, None) == 1
    assert sk(ctypes.byref(down), FAKE + 8, FAKE, FAKE, need, None) == 3
    assert sk(ctypes.byref(_nv(K=16)), FAKE, FAKE, FAKE, need, None) == 2
    assert sk(ctypes.byref(_nv(layout=1)), FAKE, FAKE, FAKE, need, None) == 5
    lrs = lib.attnq_gemv_nvfp4_lowrank_splitk                                      # (W0, s, U, V, r, x, t, split_ws, bytes, y)
    assert lrs(ctypes.byref(down), FAKE, FAKE, FAKE, 4, FAKE, FAKE, None, need, FAKE, None) == 1       # split_ws needed
    assert lrs(ctypes.byref(down), FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, need - 1, FAKE, None) == 2   # too small
    assert lrs(ctypes.byref(down), FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE + 128, need, FAKE, None) == 3  # 256-byte
    assert lrs(ctypes.byref(down), FAKE, FAKE, FAKE, 65, FAKE, FAKE, FAKE, need, FAKE, None) == 2      # r > 64
    assert lrs(ctypes.byref(down), FAKE, None, FAKE, 4, FAKE, FAKE, FAKE, need, FAKE, None) == 1       # U missing
    assert lrs(ctypes.byref(down), FAKE, FAKE, FAKE, 4, FAKE, None, FAKE, need, FAKE, None) == 1       # t missing
    assert lrs(ctypes.byref(down), FAKE, FAKE, FAKE, 4, FAKE + 8, FAKE, FAKE, need, FAKE, None) == 3   # x 16-byte
    assert lrs(ctypes.byref(down), FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, need, FAKE + 2, None) == 3   # y 4-byte
    assert lrs(ctypes.byref(_nv(K=16)), FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, need, FAKE, None) == 2
    assert lrs(ctypes.byref(nv), FAKE + 1, FAKE, FAKE, 4, FAKE, FAKE, None, 0, FAKE, None) == 3       # unsplit: s 2-byte
    na = lib.attnq_gemv_nvfp4_splitk_noalloc
    assert na(ctypes.byref(_nv(N=20176, K=16384)), FAKE, FAKE, None) == 2       # 1261 tiles > 1 MiB of records
    assert na(ctypes.byref(_nv(N=20160, K=49152 + 32)), FAKE, FAKE + 2, None) == 3   # unsplit shape: checks still run
    assert na(ctypes.byref(down), None, FAKE, None) == 1
    assert na(ctypes.byref(down), FAKE + 8, FAKE, None) == 3
    assert na(ctypes.byref(_nv(layout=1)), FAKE, FAKE, None) == 5
    smk = lib.attnq_gemm_nvfp4_small_m_splitk
    gu = _nv(N=43008, K=5376, n_seg=2, seg_end=[21504, 43008])
    need = A.attnq_gemm_nvfp4_small_m_splitk_workspace(43008, 5376, 8)
    assert smk(ctypes.byref(gu), FAKE, 8, 5376, FAKE, 43008, None, need, None) == 1        # workspace needed
    assert smk(ctypes.byref(gu), FAKE, 8, 5376, FAKE, 43008, FAKE, need - 1, None) == 2    # too small
    assert smk(ctypes.byref(gu), FAKE, 8, 5376, FAKE, 43008, FAKE + 64, need, None) == 3   # 256-byte alignment
    assert smk(ctypes.byref(gu), FAKE, 17, 5376, FAKE, 43008, FAKE, need, None) == 2       # M > 16
    assert smk(ctypes.byref(gu), FAKE, 8, 5370, FAKE, 43008, FAKE, need, None) == 2        # ldx % 8
    assert smk(ctypes.byref(gu), None, 8, 5376, FAKE, 43008, FAKE, need, None) == 1
    rc = lib.attnq_read_ceiling
    assert rc(FAKE, 24, None, 0, FAKE, None) == 2                                 # not a multiple of 16
    assert rc(FAKE, -16, None, 0, FAKE, None) == 2
    assert rc(FAKE, 64, None, 16, FAKE, None) == 1                                # b missing
    assert rc(FAKE, 64, None, 0, None, None) == 1                                 # sink missing
    assert rc(FAKE + 8, 64, None, 0, FAKE, None) == 3
    assert rc(FAKE, 63 << 30, None, 0, FAKE, None) == 2                          # 32-bit piece indices
    g = lib.attnq_gemm_nvfp4_small_m
    assert g(ctypes.byref(nv), FAKE, 17, 64, FAKE, 64, None) == 2                 # M > 16
    assert g(ctypes.byref(nv), FAKE, 4, 32, FAKE, 64, None) == 2                  # ldx < K
    assert g(ctypes.byref(nv), FAKE, 4, 68, FAKE, 64, None) == 2                  # ldx % 8
    assert g(ctypes.byref(nv), FAKE, 4, 64, FAKE, 32, None) == 2                  # ldy < N
    assert g(ctypes.byref(nv), FAKE, 4, 1 << 29, FAKE, 64, None) == 2             # X extent 3 * 2^29 + K >= 2^30
    assert g(ctypes.byref(nv), None, 4, 64, FAKE, 64, None) == 1
