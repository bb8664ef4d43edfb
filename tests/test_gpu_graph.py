"""Graph-capture safety of the library calls: every entry point that enqueues kernels (the
read-ceiling measurement aid aside) is captured once in a hipGraph (torch.cuda.CUDAGraph on a side
stream, as the benchmark does) and the graph is replayed several times. Between replays the outputs are overwritten with NaN and unrelated
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


def _setup_more(A):
    """The calls with workspaces, tickets or slot clears: reconstruct, the staged and batched staged
    quantization (rank-16 whole tiles and a rank-0 bundle), the split-K GEMV with a workspace and on
    the static scratch, the bf16 GEMV, and the small-M product on walking strips and on K slices."""
    K = 1152
    b16 = [inputs.theta_bundle(64, K, 16, cfg=9, layer=84, proj=p) for p in (0, 1)]
    b0 = inputs.theta_bundle(96, K, 0, cfg=9, layer=84, proj=2)
    bundles = [tuple(dev(a) for a in b) for b in b16 + [b0]]
    Wb = A.NVFP4Weight.empty(64 + 64 + 96, K, [64, 128, 224])
    ws_b = A.staged_batch_workspace(bundles)
    th = bundles[0]
    Ws = A.NVFP4Weight.empty(64, K)
    ws_s = A.staged_workspace(64, K, 16)
    We = torch.empty((64, K), dtype=torch.bfloat16, device="cuda")
    Kd = 21504
    Wd, _ = gpu_quantize(A, [inputs.theta_bundle(64, Kd, 0, cfg=9, layer=85, proj=0, passthrough=True)], Kd)
    xd = dev(inputs.activation_bf16(1, Kd, 9, 85, 0).reshape(-1))
    ws_d = A.splitk_workspace(64, Kd)
    Kw = 8192                                        # 377 rows, M = 6: walking strips (8 of 32 chunks)
    Ww, _ = gpu_quantize(A, [inputs.theta_bundle(377, Kw, 0, cfg=9, layer=86, proj=0, passthrough=True)], Kw)
    Xw = dev(inputs.activation_bf16(6, Kw, 9, 86, 6))
    ws_w = A.small_m_workspace(377, Kw, 6)
    Kl = 21504 + 32                                  # 129 rows, M = 4: one-shot K slices
    Wl, _ = gpu_quantize(A, [inputs.theta_bundle(129, Kl, 0, cfg=9, layer=87, proj=0, passthrough=True)], Kl)
    Xl = dev(inputs.activation_bf16(4, Kl, 9, 87, 4))
    ws_l = A.small_m_workspace(129, Kl, 4)
    assert ws_w is not None and ws_l is not None and ws_d is not None
    Wh = dev(inputs.normal_bf16((300, K), 0.02, 9, 88, 0, inputs.T_W0))
    xh = dev(inputs.activation_bf16(1, K, 9, 88, 0).reshape(-1))
    out = {
        "We": We, "s_codes": Ws.codes, "s_scales": Ws.scales, "s_ts": Ws.tensor_scale,
        "b_codes": Wb.codes, "b_scales": Wb.scales, "b_ts": Wb.tensor_scale,
        "yd": torch.empty((64,), dtype=torch.float32, device="cuda"),
        "yd_na": torch.empty((64,), dtype=torch.float32, device="cuda"),
        "yh": torch.empty((300,), dtype=torch.float32, device="cuda"),
        "Yw": torch.empty((6, 377), dtype=torch.float32, device="cuda"),
        "Yl": torch.empty((4, 129), dtype=torch.float32, device="cuda"),
    }

    def run():
        A.attnq_reconstruct(*th, We)
        A.attnq_quantize_nvfp4_staged(*th, Ws, ws_s, seg=0)
        A.attnq_quantize_nvfp4_staged_batch(bundles, [Wb, Wb, Wb], [0, 1, 2], ws_b)
        A.attnq_gemv_nvfp4_splitk(Wd, xd, out["yd"], ws_d)
        A.attnq_gemv_nvfp4_splitk_noalloc(Wd, xd, out["yd_na"])
        A.attnq_gemv_bf16(Wh, xh, out["yh"])
        A.attnq_gemm_nvfp4_small_m_splitk(Ww, Xw, out["Yw"], ws_w)
        A.attnq_gemm_nvfp4_small_m_splitk(Wl, Xl, out["Yl"], ws_l)
    return run, out, (Wd, xd)


@pytest.mark.parametrize("setup", [_setup, _setup_more], ids=["gemv_glu_lowrank_small_m_quantize", "workspace_calls"])
def test_graph_replays_match_eager(A, setup):
    say(f"graph capture: {setup.__name__}")
    run, out, (W, x) = setup(A)
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
