"""Benchmark: NVFP4 weight streaming for batch-1 decode of a 31B-like model on one MI355X.

One step = one token of the whole-model weight stream: 60 layers x {fused q|k|v 6144x5376,
o 5376x4096, fused gate|up 43008x5376, down 5376x21504} NVFP4 GEMVs plus the tied bf16
lm_head 262144x5376 GEMV -- 241 kernel launches, replayed as one hipGraph. Every layer has
its own weights (16.4 GB per token, far above the 256 MB last-level cache), already resident
in HBM when timing starts.

The weights are built on the GPU by the load path itself: seeded bf16 W0 drawn on the device,
then attnq_quantize_nvfp4 (passthrough reconstruction). The load path is also timed on its
own workload -- all 410 theta bundles at rank 16 with s ~ U(0.9, 1.1) (420 segment
quantizations: in 10 layers k's bundle also fills the v rows), through the staged call
(attnq_quantize_nvfp4_staged, one shared workspace) and the two-rebuild call -- and so is the
small-M verify product (M = 4 and 8) on one layer; both are reported as extra fields.

Three more token streams are timed the same way and reported under "streams": the chained token
in which each layer's gate|up launch applies the activation epilogue (attnq_gemv_nvfp4_glu)
and its down projection reads that bf16 output; the coverage-matched mix with the attention
projections left in bf16 (attnq_gemv_bf16) and the MLP in NVFP4; and the runtime low-rank token,
26 shared NVFP4 blocks in contiguous bands of layers, each layer applying its own rank-16
s, U, V in the GEMV epilogue (attnq_gemv_nvfp4_lowrank_splitk; the down projection on the split-K GEMV). Consecutive layers of one band read the
same block, so part of that stream's block bytes may come from the last-level cache.

Output: one JSON line (metric, value, trials, roofline, per-projection and stream figures). Options:
  --steps K --warmup W       timed / untimed steps (defaults 20 / 5)
  --gpus N                   only N = 1 is supported (one GPU)
  --no-cpu-baseline          skip the oracle timing
  --no-load-path             skip the rank-16 load-path timing (saves ~48 GB of W0)
  --eager                    time plain stream launches instead of the hipGraph replay
  --calibrate-copy           also run a 1 GiB device copy (for counter calibration)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HIDDEN = 5376
N_LAYERS = 60
QKV_SEGS = (4096, 1024, 1024)
O_SHAPE = (HIDDEN, 4096)
GU_SEGS = (21504, 21504)
DOWN_SHAPE = (HIDDEN, 21504)
VOCAB = 262144
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
VALU_FP32_PEAK_TFLOPS = 157.3  # published fp32 vector peak (packed), for the load path note
PROJ_NAMES = ("qkv", "o", "gate_up", "down")
LOWRANK_BANDS = 26             # shared NVFP4 blocks for the 60 layers, in contiguous bands
LOWRANK_RANK = 16

# HBM traffic of one fused gate|up launch from the FETCH_SIZE / WRITE_SIZE passes recorded in
# profiles/gemv_nvfp4_31b_token_traffic.md (FETCH scaled x1.9999, WRITE x1.0 by a 1 GiB copy).
# Valid only for the kernel code it was measured on: reported as null once that changes.
GATE_UP_TRAFFIC = {"sources_sha256_16": "42c01147214a0f99", "bytes": 130371401}


def gemv_sources_hash() -> str:
    """Hash of the GEMV kernel sources with comments and whitespace removed, so that the guard
    follows the code, not its commentary."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "nvfp4_weight_only_rtn_amd", "csrc")
    code = "".join(open(os.path.join(csrc, f)).read() for f in ("gemv.hip", "attnq_device.h"))
    code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = re.sub(r"\s+", " ", code)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def nvfp4_bytes(N: int, K: int, n_seg: int) -> int:
    """Algorithmic HBM bytes of one NVFP4 GEMV: codes + scales + tensor scales + x + y."""
    return N * K // 2 + N * K // 16 + 4 * n_seg + 2 * K + 4 * N


def bf16_bytes(N: int, K: int) -> int:
    return 2 * N * K + 2 * K + 4 * N


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Model:
    """Device-resident NVFP4 weights of the 31B-like stack plus per-projection x / y buffers."""

    def __init__(self, A, dev):
        self.A = A
        self.layers = []
        seed = 1000
        for L in range(N_LAYERS):
            lay = {}
            for name, segs, K in (("qkv", QKV_SEGS, HIDDEN), ("o", (O_SHAPE[0],), O_SHAPE[1]),
                                  ("gate_up", GU_SEGS, HIDDEN), ("down", (DOWN_SHAPE[0],), DOWN_SHAPE[1])):
                N = sum(segs)
                ends = list(np.cumsum(segs))
                W = A.NVFP4Weight.empty(N, K, ends, device=dev)
                x = torch.randn(K, device=dev, generator=torch.Generator(device=dev).manual_seed(seed)).to(torch.bfloat16)
                seed += 1
                y = torch.empty(N, dtype=torch.float32, device=dev)
                lay[name] = (W, x, y, segs, K)
            self.layers.append(lay)
        from nvfp4_weight_only_rtn_amd import inputs
        self.lm_head = inputs.device_normal_bf16((VOCAB, HIDDEN), 0.02, seed=7, device=dev)
        self.x_head = torch.randn(HIDDEN, device=dev, generator=torch.Generator(device=dev).manual_seed(8)).to(torch.bfloat16)
        self.y_head = torch.empty(VOCAB, dtype=torch.float32, device=dev)
        # gate|up activation output per layer (the input of down in the chained stream)
        self.h = [torch.empty(GU_SEGS[0], dtype=torch.bfloat16, device=dev) for _ in range(N_LAYERS)]
        self.attn_bf16 = None
        self.lowrank = None
        # one zeroed workspace serves every down projection (attnq_gemv_nvfp4_splitk), in stream order
        self.ws = A.splitk_workspace(DOWN_SHAPE[0], DOWN_SHAPE[1], device=dev)

    def down(self, W, x, y):
        """The down projection (rows of 21504 elements): K split across workgroups."""
        self.A.attnq_gemv_nvfp4_splitk(W, x, y, self.ws)

    def quantize_passthrough(self, dev):
        """Fill every NVFP4 weight from a seeded device bf16 W0 (passthrough reconstruction)."""
        from nvfp4_weight_only_rtn_amd import inputs
        seed = 50_000
        for lay in self.layers:
            for name in PROJ_NAMES:
                W, _, _, segs, K = lay[name]
                for i, n in enumerate(segs):
                    W0 = inputs.device_normal_bf16((n, K), 0.02, seed=seed, device=dev)
                    seed += 1
                    self.A.attnq_quantize_nvfp4(W0, None, None, None, W, seg=i)
        torch.cuda.synchronize()

    def step(self):
        A = self.A
        for lay in self.layers:
            for name in PROJ_NAMES[:3]:
                W, x, y, _, _ = lay[name]
                A.attnq_gemv_nvfp4(W, x, y)
            self.down(*lay["down"][:3])
        A.attnq_gemv_bf16(self.lm_head, self.x_head, self.y_head)

    def glu_step(self):
        """The token with the gate|up epilogue: gate|up writes h = gelu_tanh(gate) * up (bf16), and
        down reads h, so each layer's down projection depends on its gate|up output."""
        A = self.A
        for L, lay in enumerate(self.layers):
            for name in ("qkv", "o"):
                W, x, y, _, _ = lay[name]
                A.attnq_gemv_nvfp4(W, x, y)
            W, x, _, _, _ = lay["gate_up"]
            A.attnq_gemv_nvfp4_glu(W, x, A.ACT_GELU_TANH, self.h[L])
            W, _, y, _, _ = lay["down"]
            self.down(W, self.h[L], y)
        A.attnq_gemv_bf16(self.lm_head, self.x_head, self.y_head)

    def build_bf16_attention(self, dev):
        """bf16 q|k|v and o weights for every layer (the mixed stream: attention left in bf16)."""
        from nvfp4_weight_only_rtn_amd import inputs
        self.attn_bf16 = []
        for L in range(N_LAYERS):
            qkv = inputs.device_normal_bf16((sum(QKV_SEGS), HIDDEN), 0.02, seed=70_000 + 2 * L, device=dev)
            o = inputs.device_normal_bf16(O_SHAPE, 0.02, seed=70_001 + 2 * L, device=dev)
            self.attn_bf16.append((qkv, o))

    def mixed_step(self):
        """Attention projections in bf16, MLP in NVFP4 (the pages' coverage-matched mix), tied bf16 head."""
        A = self.A
        for L, lay in enumerate(self.layers):
            qkv, o = self.attn_bf16[L]
            A.attnq_gemv_bf16(qkv, lay["qkv"][1], lay["qkv"][2])
            A.attnq_gemv_bf16(o, lay["o"][1], lay["o"][2])
            W, x, y, _, _ = lay["gate_up"]
            A.attnq_gemv_nvfp4(W, x, y)
            self.down(*lay["down"][:3])
        A.attnq_gemv_bf16(self.lm_head, self.x_head, self.y_head)

    def build_lowrank(self, dev):
        """Runtime low-rank stream: 26 shared NVFP4 blocks (the first 26 layers' weights), layer L
        reading block L * 26 // 60, each layer with its own per-segment s, U, V at rank 16."""
        from nvfp4_weight_only_rtn_amd import inputs
        r = LOWRANK_RANK
        seed = 80_000
        self.lowrank = []
        for L in range(N_LAYERS):
            band = L * LOWRANK_BANDS // N_LAYERS
            lay = {}
            for name in PROJ_NAMES:
                W, _, _, segs, K = self.layers[band][name]
                _, x, y, _, _ = self.layers[L][name]
                s = inputs.device_uniform_bf16((W.N,), 0.9, 1.1, seed=seed, device=dev)
                U = inputs.device_normal_bf16((W.N, r), 1e-3, seed=seed + 1, device=dev)
                V = inputs.device_normal_bf16((len(segs), K, r), 1e-3, seed=seed + 2, device=dev)
                t = torch.empty(self.A.attnq_gemv_nvfp4_lowrank_workspace(K, len(segs), r), dtype=torch.float32,
                                device=dev)
                seed += 3
                lay[name] = (W, s, U, V, t, x, y, self.A.splitk_workspace(W.N, K, device=dev))
            self.lowrank.append(lay)

    def lowrank_step(self):
        """Every projection as shared NVFP4 block + its own low-rank delta, never rebuilt
        (attnq_gemv_nvfp4_lowrank_splitk: the t = V^T x kernel, then the GEMV with the s / U t epilogue,
        the down projection on the split-K GEMV)."""
        A = self.A
        for lay in self.lowrank:
            for name in PROJ_NAMES:
                W, s, U, V, t, x, y, sws = lay[name]
                A.attnq_gemv_nvfp4_lowrank_splitk(W, s, U, V, x, t, sws, y)
        A.attnq_gemv_bf16(self.lm_head, self.x_head, self.y_head)

    def lowrank_bytes_per_step(self) -> int:
        """Per launch: the block's NVFP4 bytes + x + y, plus s (2N), U (2Nr), V (2 n_seg K r), the
        partial-sum kernel's x reads (2K per segment) and its partials written and read once (8 per value)."""
        r = LOWRANK_RANK
        total = 0
        for lay in self.lowrank:
            for name in PROJ_NAMES:
                W, s, U, V, t, x, y, _ = lay[name]
                n_seg = len(W.seg_end)
                total += nvfp4_bytes(W.N, W.K, n_seg) + 2 * W.N + 2 * W.N * r + 2 * n_seg * W.K * r + \
                    2 * W.K * n_seg + 8 * t.numel()
        return total + bf16_bytes(VOCAB, HIDDEN)

    def lowrank_resident_bytes(self) -> int:
        blocks = sum(self.layers[b][n][0].nbytes for b in range(LOWRANK_BANDS) for n in PROJ_NAMES)
        factors = sum(lay[n][1].numel() * 2 + lay[n][2].numel() * 2 + lay[n][3].numel() * 2
                      for lay in self.lowrank for n in PROJ_NAMES)
        return blocks + factors + 2 * VOCAB * HIDDEN

    def glu_bytes_per_step(self) -> int:
        total = 0
        for lay in self.layers:
            for name in PROJ_NAMES:
                W, _, _, segs, K = lay[name]
                total += nvfp4_bytes(W.N, K, len(segs))
            total -= 4 * GU_SEGS[0] * 2 - 2 * GU_SEGS[0]      # h (bf16 F) written instead of y (fp32 2F)
        return total + bf16_bytes(VOCAB, HIDDEN)

    def mixed_bytes_per_step(self) -> int:
        total = 0
        for lay in self.layers:
            for name in ("gate_up", "down"):
                W, _, _, segs, K = lay[name]
                total += nvfp4_bytes(W.N, K, len(segs))
            total += bf16_bytes(sum(QKV_SEGS), HIDDEN) + bf16_bytes(O_SHAPE[0], O_SHAPE[1])
        return total + bf16_bytes(VOCAB, HIDDEN)

    def bytes_per_step(self) -> int:
        total = 0
        for lay in self.layers:
            for name in PROJ_NAMES:
                W, _, _, segs, K = lay[name]
                total += nvfp4_bytes(W.N, K, len(segs))
        return total + bf16_bytes(VOCAB, HIDDEN)

    def weight_bytes_per_step(self) -> int:
        total = sum(lay[n][0].nbytes for lay in self.layers for n in PROJ_NAMES)
        return total + 2 * VOCAB * HIDDEN


def time_steps(fn, steps: int) -> float:
    """ms per step over exactly `steps` calls, bracketed by device synchronization."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def graph_timing(fn, warmup: int, steps: int) -> float:
    """ms per step of `fn` captured once as a hipGraph and replayed."""
    graph = graph_of(fn)
    for _ in range(max(1, warmup)):
        graph.replay()
    torch.cuda.synchronize()
    ms = time_steps(graph.replay, steps)
    del graph
    return ms


def dominant_kernel_timing(model: Model, reps: int):
    """Average duration of the fused gate|up NVFP4 GEMV (the largest byte share of a token): the 60
    layers' distinct gate|up launches (7.8 GB per pass, so every launch streams from HBM) captured
    as a hipGraph and replayed `reps` times between HIP events on the replay stream. Returns ms."""
    A = model.A
    launches = [lambda W=W, x=x, y=y: A.attnq_gemv_nvfp4(W, x, y) for (W, x, y, _, _) in
                (lay["gate_up"] for lay in model.layers)]
    return per_launch_us(launches, reps) * 1e-3, reps * len(launches)


def load_path_timing(A, dev, model: Model, reps: int = 1):
    """Rank-16 reconstruct + RTN quantize over all 410 theta bundles (420 segment writes), timed
    three ways: the batched staged call per layer (attnq_quantize_nvfp4_staged_batch: a layer's seven
    bundles in three launches, W_eff staged in one shared workspace), the staged call per bundle
    (attnq_quantize_nvfp4_staged: W_eff rebuilt once, then quantized from it) and the two-rebuild
    call (attnq_quantize_nvfp4: the rebuild is formed again in the quantize pass). Returns
    {"staged_batch": ms, "staged": ms, "two_rebuilds": ms}, elements, distinct bundles."""
    from nvfp4_weight_only_rtn_amd import inputs
    r = 16
    bundles = []      # (W, seg, W0, s, U, V)
    seed = 900_000
    elements = 0
    distinct = 0
    for L, lay in enumerate(model.layers):
        for name in PROJ_NAMES:
            W, _, _, segs, K = lay[name]
            prev = None
            for i, n in enumerate(segs):
                reuse_k_for_v = name == "qkv" and i == 2 and L % 6 == 5     # 10 layers without a v bundle
                if reuse_k_for_v:
                    W0, s, U, V = prev
                else:
                    W0 = inputs.device_normal_bf16((n, K), 0.02, seed=seed, device=dev)
                    s = inputs.device_uniform_bf16((n,), 0.9, 1.1, seed=seed + 1, device=dev)
                    U = inputs.device_normal_bf16((n, r), 1e-3, seed=seed + 2, device=dev)
                    V = inputs.device_normal_bf16((K, r), 1e-3, seed=seed + 3, device=dev)
                    seed += 4
                    distinct += 1
                prev = (W0, s, U, V)
                bundles.append((W, i, W0, s, U, V))
                elements += n * K
    torch.cuda.synchronize()

    ws = A.staged_workspace(max(b[2].shape[0] * b[2].shape[1] for b in bundles), 1, r)
    per_layer = len(bundles) // len(model.layers)            # a layer's bundles, in order
    layers = [bundles[i:i + per_layer] for i in range(0, len(bundles), per_layer)]
    batch_ws = torch.empty(max(A.attnq_quantize_nvfp4_staged_batch_workspace([b[2:] for b in lay]) for lay in layers),
                           dtype=torch.uint8, device=dev)

    def run_batch():
        for lay in layers:
            A.attnq_quantize_nvfp4_staged_batch([b[2:] for b in lay], [b[0] for b in lay], [b[1] for b in lay], batch_ws)

    def run_staged():
        for (W, i, W0, s, U, V) in bundles:
            A.attnq_quantize_nvfp4_staged(W0, s, U, V, W, ws, seg=i)

    def run_two():
        for (W, i, W0, s, U, V) in bundles:
            A.attnq_quantize_nvfp4(W0, s, U, V, W, seg=i)
    out = {}
    for name, run in (("staged_batch", run_batch), ("staged", run_staged), ("two_rebuilds", run_two)):
        run()                               # warm-up (first-touch of every buffer)
        out[name] = time_steps(run, reps)
    del bundles, ws, batch_ws, layers
    torch.cuda.empty_cache()
    return out, elements, distinct


def small_m_timing(A, model: Model, steps: int):
    """M = 4 (gamma 3 + 1) and M = 8 verify products over one 31B-like layer's four projections through
    attnq_gemm_nvfp4_small_m_splitk (one workspace for all of them), timed cold by walking 8 distinct
    layers in a hipGraph; per-projection figures are the same launches class by class."""
    out = {}
    for M in (4, 8):
        need = max(A.attnq_gemm_nvfp4_small_m_splitk_workspace(model.layers[0][n][0].N, model.layers[0][n][4], M)
                   for n in PROJ_NAMES)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        nbytes = flops = 0
        per = {}
        all_fns = []
        for name in PROJ_NAMES:
            W0, _, _, segs, K = model.layers[0][name]
            X = torch.randn((M, K), device="cuda").to(torch.bfloat16)
            Y = torch.empty((M, W0.N), dtype=torch.float32, device="cuda")
            nbytes += W0.nbytes + 2 * M * K + 4 * M * W0.N
            flops += 2 * M * W0.N * K
            fns = [lambda W=model.layers[L][name][0], X=X, Y=Y: A.attnq_gemm_nvfp4_small_m_splitk(W, X, Y, ws)
                   for L in range(8)]
            per[name] = round(per_launch_us(fns, steps), 2)
            all_fns.append(fns)
        layer_fns = [f for L in range(8) for f in (all_fns[p][L] for p in range(len(PROJ_NAMES)))]
        us = per_launch_us(layer_fns, steps) * len(PROJ_NAMES)
        out[f"M{M}"] = {"us_per_layer": round(us, 2), "TBps": round(nbytes / (us * 1e-6) / 1e12, 3),
                        "TFLOPs": round(flops / (us * 1e-6) / 1e12, 2), "per_projection_us": per}
    return out


def machine_state():
    """Other GPU processes (rocm-smi --showpids) and the clock levels (rocm-smi --showclocks), read
    before this process touches the GPU: a busy machine reads low, so the run records whether it was idle."""
    import subprocess
    out = {}
    try:
        r = subprocess.run(["rocm-smi", "--showpids"], capture_output=True, text=True, timeout=60)
        txt = r.stdout + r.stderr
        out["idle"] = "No KFD PIDs currently running" in txt
        if not out["idle"]:
            out["gpu_processes"] = [l.strip() for l in txt.splitlines() if l.strip() and l.strip()[0].isdigit()][:8]
    except Exception as e:                      # rocm-smi missing or failing: say so, do not stop
        out["idle"] = None
        out["idle_check_error"] = str(e)[:200]
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=60)
        out["clocks"] = [" ".join(l.split()) for l in r.stdout.splitlines() if "clock level" in l][:8]
    except Exception as e:
        out["clocks"] = f"unavailable: {str(e)[:200]}"
    return out


def summarize_trials(ms: list) -> dict:
    v = sorted(ms)
    return {"n": len(v), "median_ms": round(float(np.median(v)), 5), "min_ms": round(v[0], 5),
            "max_ms": round(v[-1], 5), "all_ms": [round(t, 5) for t in ms]}


EAGER = False          # --eager: every timing launches on the stream (counter passes see each dispatch)


def per_launch_us(fn_list, reps: int) -> float:
    """Average duration of back-to-back launches: the launches of `fn_list` (each item one launch on
    distinct buffers) captured once as a hipGraph, replayed `reps` times between two HIP events on
    the stream the graph runs on -- the conditions of the token stream (with --eager, launched on the
    stream instead)."""
    def run():
        for f in fn_list:
            f()
    if EAGER:
        run()
        return time_steps(run, reps) * 1e3 / len(fn_list)
    g = graph_of(run)
    ms = time_steps(g.replay, reps)
    del g
    return ms * 1e3 / len(fn_list)


def per_projection_timing(model: Model, reps: int):
    """Each projection class launched back to back over the 60 layers' distinct weights (cold), next to
    the read ceiling of the same bytes: attnq_read_ceiling over each weight's codes and scales. The
    token's ceiling is 60 x the per-layer ceilings + the lm_head's."""
    A = model.A
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = {}
    ceil_layer_us = 0.0
    for name in PROJ_NAMES:
        lays = [lay[name] for lay in model.layers]
        if name == "down":
            gemv = [lambda W=W, x=x, y=y: model.down(W, x, y) for (W, x, y, _, _) in lays]
            plain = [lambda W=W, x=x, y=y: A.attnq_gemv_nvfp4(W, x, y) for (W, x, y, _, _) in lays]
        else:
            gemv = [lambda W=W, x=x, y=y: A.attnq_gemv_nvfp4(W, x, y) for (W, x, y, _, _) in lays]
            plain = None
        reads = [lambda W=W: A.attnq_read_ceiling(W.codes, W.scales, sink) for (W, _, _, _, _) in lays]
        W0 = lays[0][0]
        nbytes = nvfp4_bytes(W0.N, W0.K, len(W0.seg_end))
        us = per_launch_us(gemv, reps)
        ceil = per_launch_us(reads, reps)
        ceil_layer_us += ceil
        out[name] = {"us": round(us, 3), "TBps": round(nbytes / (us * 1e-6) / 1e12, 3),
                     "read_ceiling_us": round(ceil, 3),
                     "ceiling_TBps": round((W0.codes.numel() + W0.scales.numel()) / (ceil * 1e-6) / 1e12, 3)}
        if plain is not None:
            out[name]["single_workgroup_k_us"] = round(per_launch_us(plain, reps), 3)
    head = [lambda: A.attnq_gemv_bf16(model.lm_head, model.x_head, model.y_head)]
    head_us = per_launch_us(head, reps)
    head_ceil = per_launch_us([lambda: A.attnq_read_ceiling(model.lm_head, None, sink)], reps)
    out["lm_head"] = {"us": round(head_us, 3), "TBps": round(bf16_bytes(VOCAB, HIDDEN) / (head_us * 1e-6) / 1e12, 3),
                      "read_ceiling_us": round(head_ceil, 3),
                      "ceiling_TBps": round(2 * VOCAB * HIDDEN / (head_ceil * 1e-6) / 1e12, 3)}
    token_ceiling_ms = (N_LAYERS * ceil_layer_us + head_ceil) * 1e-3
    return out, token_ceiling_ms


def single_projection_c0(A, dev, trials: int, steps: int):
    """One 1024 x 1152 projection (W0 ~ N(0, 0.02^2), s = 1, U = V = 0 at rank 4: passthrough), quantized
    by the library, then copied to 1600 distinct places (1.06 GB, beyond the 256 MB last-level
    cache); one step is one GEMV on each copy in turn, replayed as a hipGraph. Latency-bound: the
    headline is microseconds per GEMV."""
    from nvfp4_weight_only_rtn_amd import inputs
    N, K, copies = 1024, 1152, 1600
    W0 = inputs.device_normal_bf16((N, K), 0.02, seed=11, device=dev)
    zU = torch.zeros((N, 4), dtype=torch.bfloat16, device=dev)
    zV = torch.zeros((K, 4), dtype=torch.bfloat16, device=dev)
    ones = torch.ones(N, dtype=torch.bfloat16, device=dev)
    src = A.NVFP4Weight.empty(N, K, [N], device=dev)
    A.attnq_quantize_nvfp4(W0, ones, zU, zV, src, seg=0)
    Ws = []
    for _ in range(copies):
        W = A.NVFP4Weight.empty(N, K, [N], device=dev)
        W.codes.copy_(src.codes)
        W.scales.copy_(src.scales)
        W.tensor_scale.copy_(src.tensor_scale)
        Ws.append(W)
    x = torch.randn(K, device=dev, generator=torch.Generator(device=dev).manual_seed(12)).to(torch.bfloat16)
    y = torch.empty(N, dtype=torch.float32, device=dev)

    def run():
        for W in Ws:
            A.attnq_gemv_nvfp4(W, x, y)
    g = graph_of(run)
    ms = [time_steps(g.replay, steps) for _ in range(trials)]
    del g
    nbytes = nvfp4_bytes(N, K, 1)
    med = float(np.median(ms))
    return {"what": "1024x1152 NVFP4 GEMV, passthrough weight, 1600 rotated copies (1.06 GB) in one hipGraph",
            "us_per_gemv": round(med * 1e3 / copies, 4), "bytes_per_gemv": nbytes,
            "TBps": round(nbytes * copies / (med * 1e-3) / 1e12, 4),
            "trials_us_per_gemv": [round(t * 1e3 / copies, 4) for t in ms]}


def small_stack_c1(A, dev, trials: int, steps: int):
    """The 1B-like decoder stack: 26 layers of fused q|k|v 1536x1152 (1024 + 256 + 256), o 1152x1024,
    gate|up 2 x 6912 x 1152 and down 1152x6912, each rebuilt as s * W0 + U V^T (s ~ U(0.9, 1.1), rank-4
    U, V ~ N(0, 1e-3^2), W0 ~ N(0, 0.02^2)) and quantized by the library. Three distinct copies of
    the stack (1.18 GB) are streamed in turn so that the 392 MB of one token do not sit in the
    last-level cache; one step = one token through 26 layers (104 GEMVs)."""
    from nvfp4_weight_only_rtn_amd import inputs
    H, r = 1152, 4
    specs = (("qkv", (1024, 256, 256), H), ("o", (H,), 1024), ("gate_up", (6912, 6912), H), ("down", (H,), 6912))
    stacks = []
    seed = 300_000
    total = 0
    for c in range(3):
        layers = []
        for L in range(26):
            lay = []
            for name, segs, K in specs:
                W = A.NVFP4Weight.empty(sum(segs), K, list(np.cumsum(segs)), device=dev)
                for i, n in enumerate(segs):
                    W0 = inputs.device_normal_bf16((n, K), 0.02, seed=seed, device=dev)
                    sv = inputs.device_uniform_bf16((n,), 0.9, 1.1, seed=seed + 1, device=dev)
                    U = inputs.device_normal_bf16((n, r), 1e-3, seed=seed + 2, device=dev)
                    V = inputs.device_normal_bf16((K, r), 1e-3, seed=seed + 3, device=dev)
                    seed += 4
                    A.attnq_quantize_nvfp4(W0, sv, U, V, W, seg=i)
                x = torch.randn(K, device=dev, generator=torch.Generator(device=dev).manual_seed(seed)).to(torch.bfloat16)
                y = torch.empty(W.N, dtype=torch.float32, device=dev)
                lay.append((W, x, y))
                if c == 0:
                    total += nvfp4_bytes(W.N, K, len(segs))
            layers.append(lay)
        stacks.append(layers)
    torch.cuda.synchronize()

    def run():
        for layers in stacks:
            for lay in layers:
                for (W, x, y) in lay:
                    A.attnq_gemv_nvfp4(W, x, y)
    g = graph_of(run)
    ms = [time_steps(g.replay, steps) / 3 for _ in range(trials)]
    del g
    med = float(np.median(ms))
    return {"what": "1B-like stack, 26 layers x (q|k|v 1536x1152, o 1152x1024, gate|up 13824x1152, down 1152x6912), "
                    "rank-4 rebuild + RTN at load, 3 rotated copies",
            "ms_per_token": round(med, 5), "bytes_per_token": total,
            "TBps": round(total / (med * 1e-3) / 1e12, 4), "launches_per_token": 104,
            "trials_ms": [round(t, 5) for t in ms]}


def graph_of(fn):
    """`fn`'s launches captured once as a hipGraph (after one eager warm-up on a side stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    return g


def cpu_baseline():
    """The oracle as it stands, on one host thread (BLAS limited to one thread; numpy's elementwise work
    is single-threaded anyway), over a bounded sample of the same workload:
      * dequantize + float64 GEMV over the four projections of one 31B-like layer (q|k|v 6144x5376,
        o 5376x4096, gate|up 43008x5376, down 5376x21504: 226 MB NVFP4) -- the reported value;
      * the oracle's RTN quantization of the fused q|k|v (33.0 M elements), as elements per second;
      * the whole-token figure, SCALED: 60 x the layer's GEMV time + the bf16 lm_head GEMV over 16384
        of its 262144 rows x 16;
      * the load path, SCALED: the 410 bundles' 24.06 G elements at the measured quantization rate
        (rank 0 rebuild; the rank-16 rebuild adds its U V^T on top).
    The oracle's quantization of the layer sample is setup, run on threads and not timed."""
    import concurrent.futures as cf

    import oracle as O
    from nvfp4_weight_only_rtn_amd import inputs
    from threadpoolctl import threadpool_limits
    specs = (("qkv", QKV_SEGS, HIDDEN), ("o", (O_SHAPE[0],), O_SHAPE[1]),
             ("gate_up", GU_SEGS, HIDDEN), ("down", (DOWN_SHAPE[0],), DOWN_SHAPE[1]))
    jobs = [(p, i, n, K) for p, (_, segs, K) in enumerate(specs) for i, n in enumerate(segs)]
    W0s = {}

    def quantize(job):
        p, i, n, K = job
        W0 = inputs.theta_bundle(n, K, 0, cfg=2, layer=0, proj=10 * p + i, passthrough=True)[0]
        W0s[job] = W0
        return job, O.quantize_segment(W0)
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        done = dict(ex.map(quantize, jobs))
    work = []
    for p, (_, segs, K) in enumerate(specs):
        parts = [done[(p, i, n, K)] for i, n in enumerate(segs)]
        codes = np.concatenate([q[0] for q in parts])
        scales = np.concatenate([q[1] for q in parts])
        ts = np.array([q[2] for q in parts], dtype=np.float32)
        x = inputs.activation_bf16(1, K, 2, 0, p)
        work.append((codes, scales, ts, list(np.cumsum(segs)), x))
    nbytes = sum(c.nbytes + sc.nbytes + t.nbytes for c, sc, t, _, _ in work)
    head_rows = 16384
    head = inputs.normal_bf16((head_rows, HIDDEN), 0.02, 3, 60, 0, 0)
    x_head = inputs.activation_bf16(1, HIDDEN, 3, 60, 0)
    qkv_jobs = [(0, i, n, HIDDEN) for i, n in enumerate(QKV_SEGS)]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for codes, scales, ts, ends, x in work:
            O.gemv_nvfp4(codes, scales, ts, x, ends)
        t_layer = time.perf_counter() - t0
        t0 = time.perf_counter()
        O.gemv_bf16(head, x_head)
        t_head = (time.perf_counter() - t0) * (VOCAB // head_rows)
        t0 = time.perf_counter()
        for job in qkv_jobs:
            O.quantize_segment(W0s[job])
        t_quant = time.perf_counter() - t0
    q_elems = sum(n * HIDDEN for n in QKV_SEGS)
    q_rate = q_elems / t_quant
    return {"value": round(nbytes / t_layer / 1e12, 9), "unit": "TB/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle dequantize + float64 GEMV over one 31B-like layer (q|k|v 6144x5376, o 5376x4096, "
                      f"gate|up 43008x5376, down 5376x21504; {nbytes} NVFP4 bytes) in {t_layer:.2f} s on one "
                      f"thread (BLAS limited to 1; affinity {len(os.sched_getaffinity(0))} cpus)",
            "layer_gemv_s": round(t_layer, 3),
            "token_ms_scaled": round((N_LAYERS * t_layer + t_head) * 1e3, 1),
            "token_scaled_from": f"60 x the one-layer GEMV time + the bf16 lm_head GEMV timed on {head_rows} of "
                                 f"{VOCAB} rows ({t_head / (VOCAB // head_rows):.2f} s) x {VOCAB // head_rows}",
            "quantize_elements_per_s": round(q_rate, 1),
            "quantize_sample": f"oracle RTN quantization of the fused q|k|v ({q_elems} elements, 3 segments) in "
                               f"{t_quant:.2f} s",
            "load_path_s_scaled": round(24_056_954_880 / q_rate, 1)}


def calibrate_copy(dev):
    """1 GiB device-to-device copy, a kernel of known traffic for counter calibration."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"calibration copy: 3 x {n} bytes read and written")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-load-path", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the streams, small-M, C0 and C1 workloads")
    ap.add_argument("--extra", default="streams,small_m,c0,c1",
                    help="comma list of the other workloads to time (streams, small_m, c0, c1)")
    ap.add_argument("--no-machine-state", action="store_true",
                    help="skip the rocm-smi probes (for runs under a counter-collecting profiler, whose preload "
                         "would initialise the GPU in the rocm-smi child before it replaces itself)")
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="untimed token replays for at least this long before the warmup steps")
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the weight stream is a single-device path "
              "(more GPUs would shard rows; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    extra = set() if args.no_extra else {w for w in args.extra.split(",") if w}
    unknown = extra - {"streams", "small_m", "c0", "c1"}
    if unknown:
        print(f"unknown --extra workloads: {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)

    global EAGER
    EAGER = args.eager
    state = None if args.no_machine_state else machine_state()    # before this process touches the GPU
    log(f"machine: {state}")
    import nvfp4_weight_only_rtn_amd.attnq as A
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log("allocating the 31B-like stack")
    model = Model(A, dev)
    log("loading weights (device W0 -> attnq_quantize_nvfp4, passthrough)")
    t0 = time.perf_counter()
    model.quantize_passthrough(dev)
    log(f"passthrough load {time.perf_counter() - t0:.1f} s")

    for _ in range(args.warmup):
        model.step()
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        graph = graph_of(model.step)
        run = graph.replay
    else:
        run = model.step
    # settle: replays for at least --settle-ms before the warmup steps (after the set-up's idle
    # stretches the token ran about 2.5% slower for its first ~150 ms of replays)
    t_settle = time.perf_counter()
    n_settle = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            run()
        torch.cuda.synchronize()
        n_settle += 10
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for _ in range(args.warmup):
        run()
    # trials: each times exactly `steps` replays between synchronizations; the value is the median
    trial_ms = [time_steps(run, args.steps) for _ in range(max(1, args.trials))]
    trials = summarize_trials(trial_ms)
    ms = trials["median_ms"]
    eager_ms = time_steps(model.step, max(3, args.steps // 4))
    bytes_step = model.bytes_per_step()
    tbps = bytes_step / (ms * 1e-3) / 1e12
    log(f"{'graph' if graph else 'eager'} {ms:.4f} ms/token (trials {trials['all_ms']}), eager {eager_ms:.4f} ms/token, "
        f"{tbps:.3f} TB/s")

    dom_mean, dom_n = dominant_kernel_timing(model, max(3, args.steps // 2))
    W_gu = model.layers[0]["gate_up"][0]
    dom_bytes = nvfp4_bytes(W_gu.N, W_gu.K, 2)
    achieved = dom_bytes / (dom_mean * 1e-3) / 1e9

    log("per-projection times and read ceilings")
    per_proj, ceiling_ms = per_projection_timing(model, max(3, args.steps // 4))
    log(f"per projection: {per_proj}; token read ceiling {ceiling_ms:.4f} ms")

    streams = small_m = c0 = c1 = None
    if "streams" in extra:
        log("timing the chained stream (gate|up epilogue feeds down) and the bf16-attention mix")
        glu_ms = graph_timing(model.glu_step, args.warmup, args.steps)
        glu_bytes = model.glu_bytes_per_step()
        model.build_bf16_attention(dev)
        mixed_ms = graph_timing(model.mixed_step, args.warmup, args.steps)
        mixed_bytes = model.mixed_bytes_per_step()
        model.attn_bf16 = None
        model.build_lowrank(dev)
        lr_ms = graph_timing(model.lowrank_step, args.warmup, args.steps)
        lr_bytes = model.lowrank_bytes_per_step()
        lr_resident = model.lowrank_resident_bytes()
        model.lowrank = None
        torch.cuda.empty_cache()
        streams = {
            "glu_chained": {"what": "gate|up GEMV with the gelu-tanh epilogue writing bf16 h, down reading h",
                            "ms_per_token": round(glu_ms, 5), "bytes_per_token": glu_bytes,
                            "TBps": round(glu_bytes / (glu_ms * 1e-3) / 1e12, 4)},
            "bf16_attention": {"what": "q|k|v and o in bf16 (attnq_gemv_bf16), gate|up and down NVFP4, bf16 lm_head",
                               "ms_per_token": round(mixed_ms, 5), "bytes_per_token": mixed_bytes,
                               "TBps": round(mixed_bytes / (mixed_ms * 1e-3) / 1e12, 4)},
            "lowrank_banded": {"what": f"runtime low-rank: {LOWRANK_BANDS} shared NVFP4 blocks in contiguous bands of "
                                       f"layers, per-layer per-segment s, U, V at rank {LOWRANK_RANK} applied in the GEMV "
                                       "epilogue (attnq_gemv_nvfp4_lowrank_splitk, 2 launches per projection, the down projection on the "
                                       "split-K GEMV), bf16 lm_head",
                               "ms_per_token": round(lr_ms, 5), "bytes_per_token": lr_bytes,
                               "resident_weight_bytes": lr_resident,
                               "TBps": round(lr_bytes / (lr_ms * 1e-3) / 1e12, 4)},
        }
        log(f"streams: {streams}")
    if "small_m" in extra:
        small_m = small_m_timing(A, model, max(3, args.steps // 4))
        log(f"small-M: {small_m}")
    if "c0" in extra:
        log("single projection 1024x1152 over rotated copies")
        c0 = single_projection_c0(A, dev, args.trials, args.steps)
        log(f"C0 {c0}")
    if "c1" in extra:
        log("the 1B-like 26-layer stack")
        c1 = small_stack_c1(A, dev, args.trials, args.steps)
        log(f"C1 {c1}")
    # last of the GPU timings: after the load path's matrix-core and VALU load the token stream ran
    # about 2.5% slower for the rest of a run
    load = None
    if not args.no_load_path:
        log("timing the rank-16 load path over 410 bundles")
        lp_ms, elements, distinct = load_path_timing(A, dev, model)
        # algorithmic bytes per element -- staged: W0 read, W_eff written and read back (2 + 2 + 2),
        # 0.5625 B of codes and scales written; two rebuilds: W0 read twice + 0.5625 B written.
        # Rank-term flops: 2 * 16 per element per rebuild.
        per = {"staged_batch": (6.5625, 1), "staged": (6.5625, 1), "two_rebuilds": (4.5625, 2)}
        load = {"ms": round(lp_ms["staged_batch"], 3), "call": "attnq_quantize_nvfp4_staged_batch (one call per layer)",
                "elements": elements, "bundles": distinct, "segments": 420}
        for name, t in lp_ms.items():
            bpe, rebuilds = per[name]
            load[name] = {"ms": round(t, 3), "TBps_algorithmic": round(elements * bpe / (t * 1e-3) / 1e12, 3),
                          "rank_TFLOPs": round(elements * 32 * rebuilds / (t * 1e-3) / 1e12, 2)}
        log(f"load path: {load}")
        model.quantize_passthrough(dev)   # restore the passthrough weights for the stream

    if args.calibrate_copy:
        calibrate_copy(dev)

    out = {
        "metric": "NVFP4 GEMV achieved HBM TB/s (% of peak) + ms per token weight stream, 31B-like",
        "value": round(tbps, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": round(settle_ms, 1), "replays": n_settle,
                   "what": "untimed token replays before the warmup steps, until the device's rate has settled"},
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 weights (e2m1 + e4m3 block scales) x bf16 activations, fp32 accumulate",
        "data": "synthetic: seeded device bf16 W0 ~ N(0, 0.02^2) RTN-quantized by the library at load; x ~ N(0, 1)",
        "config": {"workload": "31B-like whole-model weight stream per token: 60 layers x (q|k|v 6144x5376, "
                               "o 5376x4096, gate|up 43008x5376, down 5376x21504 with K split across workgroups) "
                               "NVFP4 + bf16 lm_head 262144x5376, batch 1",
                   "launches_per_step": 4 * N_LAYERS + 1, "launch": "hipGraph replay" if graph else "stream",
                   "parallelism": "single GPU"},
        "trials": trials,
        "pct_of_hbm_peak": round(100 * tbps * 1e3 / HBM_PEAK_GBS, 2),
        "ms_per_token": round(ms, 5),
        "ms_per_token_eager": round(eager_ms, 5),
        "bytes_per_token": bytes_step,
        "weight_bytes_per_token": model.weight_bytes_per_step(),
        "read_ceiling": {"ms_per_token": round(ceiling_ms, 5),
                         "what": "sum over the token's launches of attnq_read_ceiling over the same weight bytes "
                                 "(60 x per-layer ceilings + lm_head), each timed back to back over distinct buffers",
                         "token_frac_of_ceiling": round(ceiling_ms / ms, 4)},
        "per_projection": per_proj,
        "roofline": {"bound": "hbm", "kernel": "k_gemv_nvfp4_oneshot<2,1,3,true,4,true,3,0> (fused gate|up 43008x5376)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (GATE_UP_TRAFFIC["bytes"] if gemv_sources_hash() == GATE_UP_TRAFFIC["sources_sha256_16"]
                                 else None),
                     "bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_mean * 1e3, 3),
                     "launches_timed": dom_n},
        "single_projection_1024x1152": c0,
        "stack_1b_like_26_layers": c1,
        "small_m": small_m,
        "streams": streams,
        "load_path": load,
        "machine": state,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
