"""The bytes-per-token definition used by bench.py reproduces the roofline percentages the
roadmap page prints for its own decode measurements (golden file with citation)."""

import json
import os

from tile_scheduled_persistent_amd.configs import LLAMA_1B, QWEN3_06B, QWEN3_4B, WORKLOADS

HERE = os.path.dirname(os.path.abspath(__file__))


def test_pages_roofline_percentages_reproduced():
    g = json.load(open(os.path.join(HERE, "golden", "roadmap_decode_roofline.json")))
    models = {"qwen3-0.6b-shaped": QWEN3_06B, "qwen3-4b-shaped": QWEN3_4B}
    for case in g["cases"]:
        m = models[case["model"]]
        bytes_per_token = m.weight_bytes_per_token() - 2 * m.hidden + m.kv_bytes_per_position() * g["attended_positions"]
        roof = g["bandwidth_gb_s"] * 1e9 / bytes_per_token
        pct = 100.0 * case["tok_s"] / roof
        assert round(pct) == case["pct_of_roofline"], (case, pct)


def test_workload_bytes_per_token():
    # weights once (tied head once, one embedding row) + K/V of the attended positions (mean over
    # the 64 steps: 1023 + 32.5) + one K/V write
    wl = WORKLOADS["llama1b"]
    assert LLAMA_1B.weight_bytes_per_token() == 2_471_632_896
    assert LLAMA_1B.kv_bytes_per_position() == 32_768
    assert wl.bytes_per_token() == 2_471_632_896 + 32_768 * 1055.5 + 32_768
    assert WORKLOADS["qwen4b_32k"].bytes_per_token() == QWEN3_4B.weight_bytes_per_token() + 147_456 * (32767 + 16.5) + 147_456
