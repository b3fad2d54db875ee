"""bench.py's host-side pieces, no GPU: the multi-GPU refusal, the algorithmic
work it prices each kernel at (against closed forms of the layer's shapes),
and that the committed FETCH/WRITE summaries still describe the current
kernel sources (the bench reports roofline.traffic from them only then)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_prefill_kernel_work_closed_forms():
    cfg = workloads.config("qwen3_30b_a3b_prefill")
    T, H, E, k, I = 8192, 2048, 128, 8, 768
    P = T * k
    fl, by = bench.kernel_work("ffn_gate_up_bf16", cfg, touched=E)
    # gate and up: two [P, H] x [H, I] products; bytes: every expert's w13,
    # each token row once, h written once (bf16)
    assert fl == 2 * (2 * P * H * I) == 412316860416
    assert by == E * (2 * I) * H * 2 + T * H * 2 + P * I * 2 == 939524096
    fl, by = bench.kernel_work("ffn_down_bf16", cfg, touched=E)
    assert fl == 2 * P * I * H
    # y as the forward stores it at this shape: fp16 plus an int32 exponent per 64 columns
    assert bench.y_bytes_per_value(cfg) == 2 + 4 / 64
    assert by == E * H * I * 2 + P * I * 2 + P * H * (2 + 4 / 64)
    fl, by = bench.kernel_work("combine", cfg, touched=E)
    assert fl == 0 and by == P * H * (2 + 4 / 64) + P * 8 + T * H * 4


def test_decode_and_small_shapes_keep_fp32_y():
    assert bench.y_bytes_per_value(workloads.config("qwen15_moe_decode")) == 4.0
    assert bench.y_bytes_per_value(workloads.config("tiny_fp32")) == 4.0


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_traffic_summaries_match_current_sources(kernel):
    """A kernel source changed without regenerating its counter summary would
    make the bench report traffic null; this names the stale summary."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_qwen3_30b_a3b_prefill_traffic.txt")
    assert os.path.exists(path), path
    assert bench.measured_traffic(kernel, "qwen3_30b_a3b_prefill") is not None, f"{path} is stale"
