"""The allocation-free split-K entry point (attnq_gemv_nvfp4_splitk_noalloc, scratch in a device array
inside the library) against the workspace entry point it varies (attnq_gemv_nvfp4_splitk): bit for
bit, on two calls in a row, the second with a smaller weight, and against the float64 oracle; a
weight beyond the array's 20160 rows is refused."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import assert_close_products, dev, gpu_quantize, host, oracle_quantize, say
from nvfp4_weight_only_rtn_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def test_noalloc_equals_the_workspace_call_on_two_calls(A):
    for i, (segs, K) in enumerate((((2000, 1376), 21504), ((301,), 16384))):    # the second call is smaller
        bs = [inputs.theta_bundle(n, K, 0, cfg=9, layer=60 + i, proj=j, passthrough=True) for j, n in enumerate(segs)]
        x = inputs.activation_bf16(1, K, 9, 60 + i, 0)
        say(f"no-alloc split-K call {i}: {segs}x{K}")
        W, seg_end = gpu_quantize(A, bs, K)
        xd = dev(x.reshape(-1))
        y_ws = torch.full((W.N,), np.nan, dtype=torch.float32, device="cuda")
        y_na = torch.full((W.N,), np.nan, dtype=torch.float32, device="cuda")
        A.attnq_gemv_nvfp4_splitk(W, xd, y_ws, A.splitk_workspace(W.N, K))
        A.attnq_gemv_nvfp4_splitk_noalloc(W, xd, y_na)
        torch.cuda.synchronize()
        assert np.array_equal(host(y_na).view(np.uint32), host(y_ws).view(np.uint32)), i
        c, s, t, _ = oracle_quantize(bs)
        assert_close_products(host(y_na), O.gemv_nvfp4(c, s, t, x, seg_end), O.abs_dot(c, s, t, x, seg_end)[0],
                              f"no-alloc call {i}")


def test_noalloc_refuses_weights_beyond_its_scratch(A):
    W = A.NVFP4Weight.empty(20176, 16384, [20176])
    with pytest.raises(A.AttnqError):
        A.attnq_gemv_nvfp4_splitk_noalloc(W, torch.zeros(16384, dtype=torch.int16, device="cuda"),
                                          torch.empty(20176, dtype=torch.float32, device="cuda"))
