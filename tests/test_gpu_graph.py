"""Graph-capture safety of the library calls: every entry point that enqueues kernels is captured
once in a hipGraph (torch.cuda.CUDAGraph on a side stream, as the benchmark does) and the graph
is replayed several times. Between replays the outputs are overwritten with NaN and unrelated
eager work runs, with synchronizations; after every replay each output must equal the eager
result bit for bit (every kernel here is deterministic, and no call records a memset).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, gpu_quantize, say
from nvfp4_weight_only_rtn_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import nvfp4_weight_only_rtn_amd.attnq as A
    return A


def _setup(A):
    K = 1152
    qkv = [inputs.theta_bundle(n, K, 4, cfg=9, layer=80, proj=p) for p, n in enumerate((300, 100, 100))]
    W, _ = gpu_quantize(A, qkv, K)
    gu = [inputs.theta_bundle(512, K, 0, cfg=9, layer=81, proj=p, passthrough=True) for p in (0, 1)]
    Wg, _ = gpu_quantize(A, gu, K)
    Kl, r = 2080, 16
    W0, _ = gpu_quantize(A, [inputs.theta_bundle(1000, Kl, 0, cfg=9, layer=82, proj=0, passthrough=True)], Kl)
    s = dev(inputs.uniform_bf16((1000,), 0.9, 1.1, 9, 82, 1, inputs.T_S))
    U = dev(inputs.normal_bf16((1000, r), 0.02, 9, 82, 1, inputs.T_U))
    V = dev(inputs.normal_bf16((Kl, r), 0.02, 9, 82, 1, inputs.T_V))
    ws = torch.zeros((A.attnq_gemv_nvfp4_lowrank_workspace(Kl, 1, r),), dtype=torch.float32, device="cuda")
    th = [dev(a) for a in inputs.theta_bundle(640, K, 8, cfg=9, layer=83, proj=0)]
    Wq = A.NVFP4Weight.empty(640, K)
    x = dev(inputs.activation_bf16(1, K, 9, 80, 0).reshape(-1))
    xl = dev(inputs.activation_bf16(1, Kl, 9, 82, 0).reshape(-1))
    X4 = dev(inputs.activation_bf16(4, K, 9, 80, 4))
    X8 = dev(inputs.activation_bf16(8, K, 9, 80, 8))
    out = {
        "y": torch.empty((W.N,), dtype=torch.float32, device="cuda"),
        "h": torch.empty((Wg.N // 2,), dtype=torch.bfloat16, device="cuda"),
        "ylr": torch.empty((1000,), dtype=torch.float32, device="cuda"),
        "Y4": torch.empty((4, W.N), dtype=torch.float32, device="cuda"),
        "Y8": torch.empty((8, W.N), dtype=torch.float32, device="cuda"),
        "codes": Wq.codes, "scales": Wq.scales, "ts": Wq.tensor_scale,
    }

    def run():
        A.attnq_gemv_nvfp4(W, x, out["y"])
        A.attnq_gemv_nvfp4_glu(Wg, x, A.ACT_GELU_TANH, out["h"])
        A.attnq_gemv_nvfp4_lowrank(W0, s, U, V, xl, ws, out["ylr"])
        A.attnq_gemm_nvfp4_small_m(W, X4, out["Y4"])
        A.attnq_gemm_nvfp4_small_m(W, X8, out["Y8"])
        A.attnq_quantize_nvfp4(*th, Wq, seg=0)
    return run, out, (W, x)


def _poison(out):
    for t in out.values():
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(0xA5)


def test_graph_replays_match_eager(A):
    say("graph capture of every entry point")
    run, out, (W, x) = _setup(A)
    run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                    # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()

    scratch = torch.empty((W.N,), dtype=torch.float32, device="cuda")
    for rep in range(4):
        _poison(out)
        A.attnq_gemv_nvfp4(W, x, scratch)        # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            a = v.view(torch.int32) if v.element_size() == 4 else v.view(torch.int16) if v.element_size() == 2 else v
            b = ref[k].view(torch.int32) if v.element_size() == 4 else ref[k].view(torch.int16) if v.element_size() == 2 else ref[k]
            assert torch.equal(a, b), f"replay {rep}: {k} differs from the eager result"
    del graph
