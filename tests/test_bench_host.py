"""Host-side checks of the benchmark script (no GPU): its refusal of more than one GPU and of an
unknown workload name, its 31B-like shapes against the analytic byte counts of that configuration, and the consistency of
the HBM-traffic figure it reports with the committed counter summary."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_unknown_extra_workload_is_refused_before_the_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--extra", "small_m,nope", "--no-machine-state"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "nope" in r.stderr
    assert r.stdout == ""


# Weight bytes of the 31B-like configuration at 4.5 bits per NVFP4 element (4-bit E2M1 code plus
# one E4M3 byte per 16 elements) and 2 bytes per bf16 element, worked out by hand:
#   q|k|v 6144 x 5376 -> 18,579,456    o 5376 x 4096 -> 12,386,304
#   gate|up 43008 x 5376 -> 130,056,192    down 5376 x 21504 -> 65,028,096
#   layer 226,050,048; 60 layers 13,563,002,880; lm_head 262144 x 5376 bf16 2,818,572,288
SHAPE_BYTES = {"qkv": 18_579_456, "o": 12_386_304, "gate_up": 130_056_192, "down": 65_028_096}
LAYER_BYTES = 226_050_048
TOKEN_WEIGHT_BYTES = 60 * LAYER_BYTES + 2_818_572_288


def _shapes():
    return {"qkv": (sum(bench.QKV_SEGS), bench.HIDDEN, len(bench.QKV_SEGS)),
            "o": (bench.O_SHAPE[0], bench.O_SHAPE[1], 1),
            "gate_up": (sum(bench.GU_SEGS), bench.HIDDEN, len(bench.GU_SEGS)),
            "down": (bench.DOWN_SHAPE[0], bench.DOWN_SHAPE[1], 1)}


def test_benchmark_shapes_give_the_configurations_weight_bytes():
    shapes = _shapes()
    assert set(shapes) == set(bench.PROJ_NAMES)
    for name, (N, K, n_seg) in shapes.items():
        # algorithmic bytes = weight bytes + tensor scales (fp32 per segment) + x (bf16) + y (fp32)
        assert bench.nvfp4_bytes(N, K, n_seg) == SHAPE_BYTES[name] + 4 * n_seg + 2 * K + 4 * N, name
    assert sum(SHAPE_BYTES.values()) == LAYER_BYTES
    weights = bench.N_LAYERS * sum(SHAPE_BYTES[n] for n in bench.PROJ_NAMES) + 2 * bench.VOCAB * bench.HIDDEN
    assert weights == TOKEN_WEIGHT_BYTES
    assert bench.bf16_bytes(bench.VOCAB, bench.HIDDEN) == 2_818_572_288 + 2 * 5376 + 4 * 262144


def test_traffic_figure_matches_the_committed_counter_summary():
    """The gate|up traffic bench.py reports comes from the committed FETCH_SIZE / WRITE_SIZE
    summary: same source hash, same scaled bytes, and the same algorithmic bytes as bench.py's
    own count for that launch."""
    text = open(os.path.join(ROOT, "profiles", "gemv_nvfp4_31b_token_traffic.md")).read()
    m = re.search(r"= `([0-9a-f]{16})` \(bench.py reports", text)
    assert m, "source hash line missing from the traffic summary"
    assert m.group(1) == bench.GATE_UP_TRAFFIC["sources_sha256_16"]
    row = next(line for line in text.splitlines() if line.startswith("| fused gate\\|up 43008x5376 |"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    scaled, algorithmic = (int(c.replace(",", "")) for c in cells[-3:-1])
    assert scaled == bench.GATE_UP_TRAFFIC["bytes"]
    N, K, n_seg = _shapes()["gate_up"]
    assert algorithmic == bench.nvfp4_bytes(N, K, n_seg)
    assert abs(scaled / algorithmic - 1.0) < 0.01


@pytest.mark.parametrize("name", ["gemv_nvfp4_31b_token_kernel_stats.md", "gemv_nvfp4_31b_token_traffic.md",
                                  "gemv_nvfp4_31b_token_sq_counters.md", "gemm_small_m_31b_layer_sq_counters.md",
                                  "quantize_rank16_load_path.md"])
def test_profile_summaries_name_their_commands(name):
    text = open(os.path.join(ROOT, "profiles", name)).read()
    assert "rocprofv3" in text and "bench.py" in text
    assert "_work" not in text
