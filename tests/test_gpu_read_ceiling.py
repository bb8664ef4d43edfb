"""The read-ceiling measurement call (attnq_read_ceiling) reads every 16-byte piece of both ranges:
it stores its xor-fold only when a thread's fold equals 0x9E3779B9, so a single planted piece
holding that value must reach the sink, from either range and in both walk shapes (grid-stride
below 1 GiB, contiguous stretches from 1 GiB up), while all-zero data leaves the sink alone."""
import pytest
import torch

from gpu_helpers import say

pytestmark = pytest.mark.gpu
MAGIC = 0x9E3779B9


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def _sink():
    return torch.full((1,), 7, dtype=torch.int32, device="cuda")


def _plant(buf, piece):
    words = buf.view(torch.int32)
    words[4 * piece] = MAGIC - (1 << 32)          # the same 32 bits as a signed int32


def _sink_value(s):
    return int(s.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("nbytes_a,nbytes_b,piece", [(1024, 0, 5), (32, 32, 3), (12_386_304, 4096, 774_143),
                                                     (1 << 30, 0, (1 << 26) - 1), ((1 << 30) - 4096, 8192, 1 << 26)])
def test_every_piece_is_read(A, nbytes_a, nbytes_b, piece):
    say(f"read ceiling {nbytes_a}+{nbytes_b} planted piece {piece}")
    a = torch.zeros(nbytes_a, dtype=torch.uint8, device="cuda")
    b = torch.zeros(nbytes_b, dtype=torch.uint8, device="cuda") if nbytes_b else None
    na = nbytes_a // 16
    _plant(a if piece < na else b, piece if piece < na else piece - na)
    s = _sink()
    A.attnq_read_ceiling(a, b, s)
    torch.cuda.synchronize()
    assert _sink_value(s) == MAGIC
    a.zero_()
    if b is not None:
        b.zero_()
    s = _sink()
    A.attnq_read_ceiling(a, b, s)
    torch.cuda.synchronize()
    assert _sink_value(s) == 7
